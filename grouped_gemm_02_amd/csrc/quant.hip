// FP8 (OCP E4M3) quantization with power-of-two block scales.
//
// The pages name blockwise FP8 and MXFP8 as the layer's low-precision modes
// (ic.work analysis, section on hardware constraints; MarkTechPost article,
// "How do developers use it?"). Here every block has one scale 2^e, stored
// as the E8M0 byte e + 127, so that the gfx950 scaled MFMA applies it:
//   * blockwise rule: e = smallest integer with 448 * 2^e >= amax (1x128
//     activation blocks along the reduction axis, 128x128 weight blocks);
//   * MX rule: e = floor(log2 amax) - 8 (1x32 blocks along the reduction
//     axis for every operand);
//   * an all-zero block gets e = 0.
// A value v becomes the E4M3 code nearest to v / 2^e (ties to the even code,
// saturating at +-448; a result of zero is stored as +0).
//
// Scales are always stored per (row, 32-wide block along the reduction
// axis); a 128-wide or 128x128 block writes its byte into every 32-block it
// covers, so the GEMMs read one layout for both modes.
//
// The blockwise rule with fp32 scales (kRuleF32: the EP=8-share workload's
// "fp32 scales") keeps the same blocks with s = amax / 448 in fp32: a value
// becomes the code of fl32(v * inv), inv = fl32(448 / amax), so the block
// maximum lands on +-448; an all-zero block, or one whose 448 / amax
// overflows fp32, gets s = 1 and zero codes. Its float takes the four bytes
// that the E8M0 layout gives the 128 values' four 32-blocks, so the arrays
// keep their size and every loader its offsets.
#include "device_common.h"
#include "kernels.h"

namespace moe {

// floor(log2 a) for a > 0 (exact, subnormals included)
__device__ __forceinline__ int floor_log2(float a) {
  uint32_t u = __float_as_uint(a);
  int bias = 127;
  if (((u >> 23) & 0xFFu) == 0u) {  // subnormal: scale up by 2^64 first
    u = __float_as_uint(a * 18446744073709551616.f);
    bias += 64;
  }
  return int((u >> 23) & 0xFFu) - bias;
}

// block exponent e (scale 2^e) for block maximum amax >= 0
__device__ __forceinline__ int block_exponent(float amax, int rule) {
  if (!(amax > 0.f)) return 0;
  const int q = floor_log2(amax);
  if (rule == kRuleMx) return q - 8;
  // 448 = 1.75 * 2^8: 448 * 2^(q-8) >= amax  <=>  mantissa(amax) <= 1.75
  uint32_t u = __float_as_uint(amax);
  if (((u >> 23) & 0xFFu) == 0u) u = __float_as_uint(amax * 18446744073709551616.f);
  const uint32_t mant = u & 0x7FFFFFu;
  return q - 8 + (mant > 0x600000u ? 1 : 0);
}

__device__ __forceinline__ int clamp_exp(int e) { return e < -127 ? -127 : (e > 127 ? 127 : e); }

// v * 2^-e, exact for the exponents that occur (two steps keep every factor
// a normal float)
__device__ __forceinline__ float scale_down(float v, int e) {
  const int h = -e / 2;
  return v * __builtin_ldexpf(1.f, h) * __builtin_ldexpf(1.f, -e - h);
}

// The E4M3 codes of v[0..3] / 2^e, one byte each in order. The conversion
// is the gfx950 instruction v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest
// even); magnitudes are clamped to 448 first, which is the saturation (a
// NaN becomes 448 with its sign bit), and a negative zero code (0x80)
// becomes +0.
__device__ __forceinline__ uint32_t pack4_codes(const float* v, int e) {
  float x[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float y = scale_down(v[q], e);
    x[q] = __builtin_copysignf(__builtin_fminf(__builtin_fabsf(y), 448.f), y);
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
  const uint32_t u = uint32_t(w);
  const uint32_t t = u ^ 0x80808080u;  // a 0x80 byte becomes 0x00
  const uint32_t z = ~(((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t | 0x7F7F7F7Fu);  // 0x80 where t's byte is 0
  return u & ~z;
}

// fp32-scale rule: inv = 448 / amax and s = amax / 448 (correctly rounded
// divisions); inv = 0, s = 1 for a zero block or where 448 / amax overflows
__device__ __forceinline__ void f32_block_rule(float amax, float& inv, float& s) {
  inv = 448.f / amax;
  s = amax / 448.f;
  if (!(amax > 0.f) || !(inv <= 3.40282347e38f)) {
    inv = 0.f;
    s = 1.f;
  }
}

// The E4M3 codes of fl32(v[0..3] * inv), saturating, +0 for zero results
__device__ __forceinline__ uint32_t pack4_codes_inv(const float* v, float inv) {
  float x[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float y = v[q] * inv;
    x[q] = __builtin_copysignf(__builtin_fminf(__builtin_fabsf(y), 448.f), y);
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
  const uint32_t u = uint32_t(w);
  const uint32_t t = u ^ 0x80808080u;
  const uint32_t z = ~(((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t | 0x7F7F7F7Fu);
  return u & ~z;
}

// ---------------------------------------------------------------- rows
// in: bf16 [rows, K]; out codes uint8 [rows, K], scales uint8 [rows, K/32].
// A work item is 8 consecutive values; the items of one block (4 for 32,
// 16 for 128) sit in aligned consecutive lanes and share its maximum through
// lane shuffles. Each thread takes kQItems items spaced one grid apart and
// issues all their loads before encoding, so enough bytes are in flight.
constexpr int kQItems = 4;

__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ in, int64_t rows, int K,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, int block, int rule) {
  const int per_row = K / 8;
  const int64_t total = rows * per_row;
  const int group = block / 8;  // 4 or 16 lanes, aligned within the wave
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t g0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; g0 - threadIdx.x < total;
       g0 += kQItems * stride) {
    u32x4 raw[kQItems];
#pragma unroll
    for (int u = 0; u < kQItems; ++u) {
      const int64_t g = g0 + u * stride;
      raw[u] = g < total ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in + g * 8)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kQItems; ++u) {
      const int64_t g = g0 + u * stride;
      float v[8];
      float amax = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        v[2 * d] = bf16_lo(raw[u][d]);
        v[2 * d + 1] = bf16_hi(raw[u][d]);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
      for (int off = 1; off < group; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      if (g < total) {
        if (rule == kRuleF32) {  // 128-blocks: one float per 16 items
          float inv, sc;
          f32_block_rule(amax, inv, sc);
          *reinterpret_cast<u32x2*>(codes + g * 8) = u32x2{pack4_codes_inv(v, inv), pack4_codes_inv(v + 4, inv)};
          if ((g & 15) == 0) reinterpret_cast<float*>(scales)[g / 16] = sc;
        } else {
          const int e = clamp_exp(block_exponent(amax, rule));
          const uint32_t lo = pack4_codes(v, e), hi = pack4_codes(v + 4, e);
          *reinterpret_cast<u32x2*>(codes + g * 8) = u32x2{lo, hi};
          if ((g & 3) == 0) scales[g / 4] = uint8_t(e + 127);
        }
      }
    }
  }
}

hipError_t launch_quant_rows(const uint16_t* in, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                             int block, int rule, hipStream_t st, KernelTimer* timer, const char* name) {
  if (rows <= 0) return hipSuccess;
  const int64_t items = rows * (K / 8);
  int64_t grid = (items + 256 * kQItems - 1) / (256 * kQItems);
  if (grid > 16384) grid = 16384;
  TimedLaunch tl(timer, name, st);
  hipLaunchKernelGGL(quant_rows_kernel, dim3(unsigned(grid)), dim3(256), 0, st, in, rows, K, codes, scales,
                     block, rule);
  return hipGetLastError();
}

// ---------------------------------------------------------------- weights
// One workgroup (256 threads) per 128 x 128 tile (e, rb, cb) of a stack of
// matrices W [E, R, C] (bf16); it reads the tile once and writes either or
// both of
//   plain:      codes [E, R, C] with scales [E, R, C/32]
//   transposed: codes [E, C, R] with scales [E, C, R/32]
// Blockwise rule: one exponent for the whole tile. MX rule: one exponent per
// 32 consecutive values of an output row.
//
// Thread t loads 16-byte pieces (8 values) of rows t/16 + 16*i, column
// chunk t % 16; the plain output is encoded from those registers (a 32-block
// is the 4 pieces of lanes 4j .. 4j+3). The transposed output is read back
// from a bf16 LDS copy: thread t takes source columns 2p, 2p+1 (p = t / 4)
// and rows 32q .. 32q+31 (q = t % 4), one 32-bit LDS word (two columns) per
// row, and writes 32 codes to each of its two output rows; lanes 4p .. 4p+3
// thus fill 128 contiguous bytes of an output row.
constexpr int kQLds = 128 + 2;  // bf16 per LDS row: an odd number of words keeps column reads 2-way at most


__global__ __launch_bounds__(256) void quant_weight_tiles_kernel(const uint16_t* __restrict__ W, int R, int C,
                                                                 uint8_t* __restrict__ pcodes,
                                                                 uint8_t* __restrict__ pscales,
                                                                 uint8_t* __restrict__ tcodes,
                                                                 uint8_t* __restrict__ tscales, int rule) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * kQLds];
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int cbn = C / 128, rbn = R / 128;
  const int cb = blockIdx.x % cbn;
  const int rb = (blockIdx.x / cbn) % rbn;
  const int64_t e = blockIdx.x / (int64_t(cbn) * rbn);
  const uint16_t* src = W + (e * R + int64_t(rb) * 128) * C + int64_t(cb) * 128;
  const int c8 = (t & 15) * 8;
  u32x4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) raw[i] = *reinterpret_cast<const u32x4*>(src + int64_t((t >> 4) + 16 * i) * C + c8);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (t >> 4) + 16 * i;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(raw[i][d])), fabsf(bf16_hi(raw[i][d]))));
      *reinterpret_cast<uint32_t*>(tile + r * kQLds + c8 + 2 * d) = raw[i][d];
    }
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  const float tile_amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int tile_e = rule == kRuleF32 ? 0 : clamp_exp(block_exponent(tile_amax, rule));
  float tile_inv = 0.f, tile_s = 1.f;
  if (rule == kRuleF32) f32_block_rule(tile_amax, tile_inv, tile_s);

  if (pcodes) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        v[2 * d] = bf16_lo(raw[i][d]);
        v[2 * d + 1] = bf16_hi(raw[i][d]);
      }
      int ex = tile_e;
      if (rule == kRuleMx) {
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        ex = clamp_exp(block_exponent(m, rule));
      }
      const int64_t orow = e * R + int64_t(rb) * 128 + (t >> 4) + 16 * i;
      if (rule == kRuleF32) {
        *reinterpret_cast<u32x2*>(pcodes + orow * C + int64_t(cb) * 128 + c8) =
            u32x2{pack4_codes_inv(v, tile_inv), pack4_codes_inv(v + 4, tile_inv)};
        if ((t & 15) == 0) reinterpret_cast<float*>(pscales)[orow * (C / 128) + cb] = tile_s;
        continue;
      }
      *reinterpret_cast<u32x2*>(pcodes + orow * C + int64_t(cb) * 128 + c8) = u32x2{pack4_codes(v, ex), pack4_codes(v + 4, ex)};
      if ((t & 3) == 0) pscales[orow * (C / 32) + cb * 4 + ((t & 15) >> 2)] = uint8_t(ex + 127);
    }
  }
  if (tcodes) {
    const int pc = (t >> 2) * 2;  // source columns pc, pc + 1
    const int q = t & 3;          // source rows 32q .. 32q + 31
    float v0[32], v1[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const uint32_t w2 = *reinterpret_cast<const uint32_t*>(tile + (32 * q + r) * kQLds + pc);
      v0[r] = bf16_lo(w2);
      v1[r] = bf16_hi(w2);
    }
    int e0 = tile_e, e1 = tile_e;
    if (rule == kRuleMx) {
      float m0 = 0.f, m1 = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        m0 = fmaxf(m0, fabsf(v0[r]));
        m1 = fmaxf(m1, fabsf(v1[r]));
      }
      e0 = clamp_exp(block_exponent(m0, rule));
      e1 = clamp_exp(block_exponent(m1, rule));
    }
    const int64_t orow = e * C + int64_t(cb) * 128 + pc;  // output rows are source columns
    const int64_t ocol = int64_t(rb) * 128 + 32 * q;
    uint8_t* d0 = tcodes + orow * R + ocol;
    uint8_t* d1 = d0 + R;
    if (rule == kRuleF32) {
      const float iv = tile_inv;
      *reinterpret_cast<u32x4*>(d0) = u32x4{pack4_codes_inv(v0, iv), pack4_codes_inv(v0 + 4, iv),
                                            pack4_codes_inv(v0 + 8, iv), pack4_codes_inv(v0 + 12, iv)};
      *reinterpret_cast<u32x4*>(d0 + 16) = u32x4{pack4_codes_inv(v0 + 16, iv), pack4_codes_inv(v0 + 20, iv),
                                                 pack4_codes_inv(v0 + 24, iv), pack4_codes_inv(v0 + 28, iv)};
      *reinterpret_cast<u32x4*>(d1) = u32x4{pack4_codes_inv(v1, iv), pack4_codes_inv(v1 + 4, iv),
                                            pack4_codes_inv(v1 + 8, iv), pack4_codes_inv(v1 + 12, iv)};
      *reinterpret_cast<u32x4*>(d1 + 16) = u32x4{pack4_codes_inv(v1 + 16, iv), pack4_codes_inv(v1 + 20, iv),
                                                 pack4_codes_inv(v1 + 24, iv), pack4_codes_inv(v1 + 28, iv)};
      if (q == 0) {
        reinterpret_cast<float*>(tscales)[orow * (R / 128) + rb] = tile_s;
        reinterpret_cast<float*>(tscales)[(orow + 1) * (R / 128) + rb] = tile_s;
      }
      return;
    }
    *reinterpret_cast<u32x4*>(d0) = u32x4{pack4_codes(v0, e0), pack4_codes(v0 + 4, e0), pack4_codes(v0 + 8, e0),
                                          pack4_codes(v0 + 12, e0)};
    *reinterpret_cast<u32x4*>(d0 + 16) = u32x4{pack4_codes(v0 + 16, e0), pack4_codes(v0 + 20, e0),
                                               pack4_codes(v0 + 24, e0), pack4_codes(v0 + 28, e0)};
    *reinterpret_cast<u32x4*>(d1) = u32x4{pack4_codes(v1, e1), pack4_codes(v1 + 4, e1), pack4_codes(v1 + 8, e1),
                                          pack4_codes(v1 + 12, e1)};
    *reinterpret_cast<u32x4*>(d1 + 16) = u32x4{pack4_codes(v1 + 16, e1), pack4_codes(v1 + 20, e1),
                                               pack4_codes(v1 + 24, e1), pack4_codes(v1 + 28, e1)};
    tscales[orow * (R / 32) + rb * 4 + q] = uint8_t(e0 + 127);
    tscales[(orow + 1) * (R / 32) + rb * 4 + q] = uint8_t(e1 + 127);
  }
}

// ---------------------------------------------------------------- along tokens
// Operands of the FP8 weight-gradient GEMMs, quantized along each expert's
// rows (the reduction axis of those GEMMs). Expert e owns permuted rows
// [offsets[e], offsets[e] + counts[e]); its r-th row is row offsets[e] + r of
// `in` (src_of == nullptr) or the token row src_of[offsets[e] + r] / kk.
// With Kp_e = counts[e] rounded up to 128 and poff_e = sum of Kp over the
// experts before e, the codes of column c are the Kp_e bytes at
//   codes + C * poff_e + c * Kp_e      (zero codes past counts[e])
// and its scale bytes the Kp_e / 32 bytes at
//   scales + C * poff_e / 32 + c * Kp_e / 32.
// Blockwise rule: one exponent per column per 128-row block (its byte
// repeated in the four 32-blocks); MX rule: one per column per 32 rows.
// One workgroup per (128-row block of an expert, kTokCols column tiles of
// 128): for each tile it loads the 128 x 128 bf16 values into LDS (rows past
// the expert's end as zeros) and writes them transposed like the weight
// quantizer: thread t takes columns 2p, 2p+1 (p = t / 4) and rows
// 32q .. 32q+31 (q = t % 4). The block lookup and the row indices are shared
// by the workgroup's tiles.
// With rcodes != nullptr the kernel also writes the rows' quantization along
// the columns (the moe_quantize_rows layout: codes [*, C] and scales
// [*, C/32] at the source row; 128-column or 32-column blocks by the rule),
// bit-identical to launch_quant_rows, from the same loads. Every source row
// must then occur once (a direct operand, or token rows with kk == 1).
constexpr int kTokCols = 4;
__global__ __launch_bounds__(256) void quant_tokens_kernel(const uint16_t* __restrict__ in, int64_t ld, int C,
                                                           const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ offsets, int E,
                                                           const int32_t* __restrict__ src_of, int kk,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales, int rule,
                                                           uint8_t* __restrict__ rcodes,
                                                           uint8_t* __restrict__ rscales) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * kQLds];
  __shared__ int32_t s_pref[1025];  // s_pref[e] = sum over e' < e of ceil(counts[e'] / 128)
  __shared__ int32_t s_part[256];
  const int t = threadIdx.x;
  // prefix of 128-row block counts (E <= 1024: 4 experts per thread)
  int32_t loc[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    loc[q] = e < E ? (counts[e] + 127) / 128 : 0;
    sum += loc[q];
  }
  s_part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int32_t add = t >= off ? s_part[t - off] : 0;
    __syncthreads();
    s_part[t] += add;
    __syncthreads();
  }
  int32_t run = s_part[t] - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    if (e < E) s_pref[e] = run;
    run += loc[q];
  }
  if (t == 255) s_pref[E] = s_part[255];
  __syncthreads();
  const int cgn = (C / 128 + kTokCols - 1) / kTokCols;  // column groups
  const int cg = int(blockIdx.x % unsigned(cgn));
  const int gb = int(blockIdx.x / unsigned(cgn));
  if (gb >= s_pref[E]) return;  // past the last block: the whole workgroup leaves
  int lo = 0, hi = E;           // expert with s_pref[e] <= gb < s_pref[e + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= gb) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int b = gb - s_pref[e];
  const int rows = counts[e];
  const int64_t off = offsets[e];
  const int64_t kp = int64_t(s_pref[e + 1] - s_pref[e]) * 128;  // Kp_e
  const int64_t poff = int64_t(s_pref[e]) * 128;                // poff_e
  const int c8 = (t & 15) * 8;
  int64_t srow[8];  // source row of tile rows (t >> 4) + 16 i, or -1
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = b * 128 + (t >> 4) + 16 * i;
    srow[i] = r < rows ? (src_of ? int64_t(src_of[off + r] / kk) : off + r) : -1;
  }
  const int pc = (t >> 2) * 2;  // columns pc, pc + 1 of a tile
  const int q = t & 3;          // rows 32q .. 32q + 31 of a tile
  const int cb_end = min(C / 128, (cg + 1) * kTokCols);
  for (int cb = cg * kTokCols; cb < cb_end; ++cb) {
    u32x4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      raw[i] = srow[i] >= 0 ? *reinterpret_cast<const u32x4*>(in + srow[i] * ld + int64_t(cb) * 128 + c8)
                            : u32x4{0u, 0u, 0u, 0u};
    if (rcodes) {  // along the columns: a row's 128 values sit in 16 aligned lanes
      const int group = rule == kRuleMx ? 4 : 16;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v[8];
        float m = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          v[2 * d] = bf16_lo(raw[i][d]);
          v[2 * d + 1] = bf16_hi(raw[i][d]);
        }
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) m = fmaxf(m, fabsf(v[q8]));
        for (int o = 1; o < group; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        if (srow[i] >= 0) {
          const int ex = clamp_exp(block_exponent(m, rule));
          *reinterpret_cast<u32x2*>(rcodes + srow[i] * C + int64_t(cb) * 128 + c8) =
              u32x2{pack4_codes(v, ex), pack4_codes(v + 4, ex)};
          if ((t & 3) == 0) rscales[srow[i] * (C / 32) + cb * 4 + ((t & 15) >> 2)] = uint8_t(ex + 127);
        }
      }
    }
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        *reinterpret_cast<uint32_t*>(tile + ((t >> 4) + 16 * i) * kQLds + c8 + 2 * d) = raw[i][d];
    __syncthreads();
    float v0[32], v1[32];
    float m0 = 0.f, m1 = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const uint32_t w2 = *reinterpret_cast<const uint32_t*>(tile + (32 * q + r) * kQLds + pc);
      v0[r] = bf16_lo(w2);
      v1[r] = bf16_hi(w2);
      m0 = fmaxf(m0, fabsf(v0[r]));
      m1 = fmaxf(m1, fabsf(v1[r]));
    }
    if (rule != kRuleMx) {  // 128-row blocks: the four threads of these columns share their maxima
      m0 = fmaxf(m0, __shfl_xor(m0, 1));
      m0 = fmaxf(m0, __shfl_xor(m0, 2));
      m1 = fmaxf(m1, __shfl_xor(m1, 1));
      m1 = fmaxf(m1, __shfl_xor(m1, 2));
    }
    const int e0 = clamp_exp(block_exponent(m0, rule));
    const int e1 = clamp_exp(block_exponent(m1, rule));
    const int64_t col = int64_t(cb) * 128 + pc;
    uint8_t* d0 = codes + int64_t(C) * poff + col * kp + int64_t(b) * 128 + 32 * q;
    uint8_t* d1 = d0 + kp;
    *reinterpret_cast<u32x4*>(d0) = u32x4{pack4_codes(v0, e0), pack4_codes(v0 + 4, e0), pack4_codes(v0 + 8, e0),
                                          pack4_codes(v0 + 12, e0)};
    *reinterpret_cast<u32x4*>(d0 + 16) = u32x4{pack4_codes(v0 + 16, e0), pack4_codes(v0 + 20, e0),
                                               pack4_codes(v0 + 24, e0), pack4_codes(v0 + 28, e0)};
    *reinterpret_cast<u32x4*>(d1) = u32x4{pack4_codes(v1, e1), pack4_codes(v1 + 4, e1), pack4_codes(v1 + 8, e1),
                                          pack4_codes(v1 + 12, e1)};
    *reinterpret_cast<u32x4*>(d1 + 16) = u32x4{pack4_codes(v1 + 16, e1), pack4_codes(v1 + 20, e1),
                                               pack4_codes(v1 + 24, e1), pack4_codes(v1 + 28, e1)};
    uint8_t* s0 = scales + int64_t(C) * poff / 32 + col * (kp / 32) + b * 4 + q;
    s0[0] = uint8_t(e0 + 127);
    s0[kp / 32] = uint8_t(e1 + 127);
  }
}

hipError_t launch_quant_tokens(const uint16_t* in, int64_t ld, int C, const int32_t* counts, const int32_t* offsets,
                               int E, int64_t M, const int32_t* src_of, int kk, uint8_t* codes, uint8_t* scales,
                               int rule, hipStream_t st, KernelTimer* timer, const char* name, uint8_t* rcodes,
                               uint8_t* rscales) {
  // an upper bound of the number of 128-row blocks: M / 128 + E
  const int64_t blocks = (M / 128 + E) * ((C / 128 + kTokCols - 1) / kTokCols);
  if (M <= 0 || blocks <= 0) return hipSuccess;
  TimedLaunch tl(timer, name, st);
  hipLaunchKernelGGL(quant_tokens_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, in, ld, C, counts, offsets, E,
                     src_of, kk, codes, scales, rule, rcodes, rscales);
  return hipGetLastError();
}

// ---------------------------------------------------------------- FP4 weights
// E2M1 (OCP MX FP4: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) weights for the
// FP8 x FP4 forward, in blocks of 32 consecutive values along each row of
// W [rows, C] (the GEMM's reduction axis), with the MX rule for E2M1:
// e = floor(log2 amax) - 2 (0 for a zero block), so a block's values reach
// just under 8 * 2^e and those above 6 * 2^e saturate. codes [rows, C/2]:
// value 2j of a row in the low nibble of byte j, 2j+1 in the high nibble
// (the order the scaled MFMA reads an FP4 operand in); scales [rows, C/32].
// Thread = one block: 64 bytes in, 16 bytes of codes and one scale byte out.

// E2M1 code of a = |v| / 2^e >= 0 (ties to the even code, saturating at 6):
// the number of rounding boundaries a lies above, with a boundary that a
// meets exactly counted when the code above it is even.
__device__ __forceinline__ uint32_t e2m1_code(float v, int e) {
  const float a = fabsf(scale_down(v, e));
  const uint32_t c = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                     uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.f);
  return c | ((v < 0.f && c != 0u) ? 8u : 0u);
}

__global__ __launch_bounds__(256) void quant_fp4_rows_kernel(const uint16_t* __restrict__ in, int64_t blocks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  for (int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; b < blocks;
       b += int64_t(gridDim.x) * blockDim.x) {
    u32x4 raw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) raw[q] = *reinterpret_cast<const u32x4*>(in + b * 32 + 8 * q);
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        v[8 * q + 2 * d] = bf16_lo(raw[q][d]);
        v[8 * q + 2 * d + 1] = bf16_hi(raw[q][d]);
      }
#pragma unroll
    for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
    const int e = amax > 0.f ? clamp_exp(floor_log2(amax) - 2) : 0;
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) word |= e2m1_code(v[8 * w + n], e) << (4 * n);
      out[w] = word;
    }
    *reinterpret_cast<u32x4*>(codes + b * 16) = out;
    scales[b] = uint8_t(e + 127);
  }
}

hipError_t launch_quant_fp4_rows(const uint16_t* in, int64_t rows, int C, uint8_t* codes, uint8_t* scales,
                                 hipStream_t st, KernelTimer* timer) {
  const int64_t blocks = rows * (C / 32);
  if (blocks <= 0) return hipSuccess;
  int64_t grid = (blocks + 255) / 256;
  if (grid > 16384) grid = 16384;
  TimedLaunch tl(timer, "quant_weights_fp4", st);
  hipLaunchKernelGGL(quant_fp4_rows_kernel, dim3(unsigned(grid)), dim3(256), 0, st, in, blocks, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_weights(const uint16_t* W, int64_t E, int R, int C, uint8_t* pcodes, uint8_t* pscales,
                                uint8_t* tcodes, uint8_t* tscales, int rule, hipStream_t st, KernelTimer* timer) {
  const int64_t tiles = E * (R / 128) * (C / 128);
  if (tiles <= 0 || (!pcodes && !tcodes)) return hipSuccess;
  TimedLaunch tl(timer, "quant_weights", st);
  hipLaunchKernelGGL(quant_weight_tiles_kernel, dim3(unsigned(tiles)), dim3(256), 0, st, W, R, C, pcodes, pscales,
                     tcodes, tscales, rule);
  return hipGetLastError();
}

}  // namespace moe
