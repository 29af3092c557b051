// Grouped GEMMs of the MoE layer on gfx950 bf16 MFMA.
//
// One grouped GEMM call runs many differently-sized per-expert matrix
// products, each indexed by the expert's group offset into the permuted rows
// (kongchang.com explainer, grouped-GEMM note). Six products make up the
// layer: the gate/up GEMM with SwiGLU in its epilogue and the down GEMM with
// the routing-weight scale in its epilogue (MarkTechPost article, "How does
// the fused kernel work?"), and in the backward the dH GEMM with the SwiGLU
// derivative and routing-weight-gradient partials in its epilogue, the dX
// GEMM, and the two weight-gradient GEMMs whose reduction dimension is each
// expert's row count.
//
// Structure shared by all six:
//   * Output tile C[m][n] of BM x BN, m on the "P" operand, n on the "Q"
//     operand, C = sum_k P[m][k] Q[n][k], fp32 accumulation in MFMA
//     registers. Workgroup of 256 threads = 4 waves in a 2 x 2 grid, each wave
//     a (BM/2) x (BN/2) block of 32x32 MFMA sub-tiles
//     (v_mfma_f32_32x32x16_bf16). The MFMA's A operand is the Q fragment and
//     its B operand the P fragment, so each lane ends up holding one row m and
//     16 columns n of a sub-tile (4 runs of 4 consecutive n): per-row
//     epilogue scalars (routing weight, row sums) live in one lane.
//   * Both operands are staged through LDS as rows of BK = 64 k-values with
//     a 16-byte pad per row (conflict-free 16-byte fragment reads), double
//     buffered: the global loads of k-tile kt+1 are in flight while tile kt
//     is multiplied. Operands whose k runs along rows in global memory are
//     copied as 16-byte chunks; operands whose k runs across rows (weights
//     read transposed, and both operands of the weight gradients) are loaded
//     as 8 k-rows x V entities per thread and transposed in registers.
//   * Persistent grid: each workgroup walks tiles blockIdx, +grid, ...; tile
//     ids are remapped so that the eight XCDs each take a contiguous range
//     (tiles of one expert share its weight panel in that XCD's L2).
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int BK = 64;
constexpr int LDS_LD = BK + 8;  // bf16 elements per LDS row: 128 B of data + 16 B pad
constexpr int kThreads = 256;

// ------------------------------------------------------------------ loaders

// A tile of ROWS entities whose k-values are contiguous in global memory.
// Thread t copies the 16-byte chunk (t % 8) of rows t/8 + 32*i.
template <int ROWS>
struct KMajorLoader {
  static constexpr int kPer = ROWS / 32;
  const uint16_t* ptr[kPer];  // row start (k = 0), nullptr = zero row
  u32x4 reg[kPer];

  __device__ __forceinline__ void set_row(int i, const uint16_t* row) {
    ptr[i] = row ? row + (threadIdx.x & 7) * 8 : nullptr;
  }
  __device__ __forceinline__ static int row_of_thread(int i) { return (threadIdx.x >> 3) + 32 * i; }

  __device__ __forceinline__ void fetch(int kt) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (ptr[i]) {
        reg[i] = *reinterpret_cast<const u32x4*>(ptr[i] + kt * BK);
      } else {
        reg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
    const int r0 = threadIdx.x >> 3, c = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      *reinterpret_cast<u32x4*>(lds + (r0 + 32 * i) * LDS_LD + c * 8) = reg[i];
  }
};

// A tile of MN entities x BK k-values where each k is one row in global
// memory holding the MN entities contiguously. Thread t loads k-rows
// kb*8 .. kb*8+7 (kb = t / 32) at entities mb*V .. mb*V+V-1 (mb = t % 32) and
// writes them transposed: LDS row (entity) gets 8 consecutive k-values.
// RowFn gives, for an absolute k, the global address of entity 0 of that
// k-row (nullptr = zeros) and a scale (applied in fp32 when SCALED).
template <int MN, bool SCALED, class RowFn>
struct MNMajorLoader {
  static constexpr int V = MN / 32;  // 4 or 8 entities per thread
  static_assert(V == 4 || V == 8, "MN must be 128 or 256");
  RowFn fn;
  uint32_t reg[8][V / 2];
  float scl[8];

  __device__ __forceinline__ void fetch(int kt) {
    const int kb = threadIdx.x >> 5, mb = threadIdx.x & 31;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = kt * BK + kb * 8 + i;
      float s = 1.f;
      const uint16_t* p = fn.row(k, s);
      if (SCALED) scl[i] = s;
      if (p) {
        if constexpr (V == 8) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(p + mb * V);
          reg[i][0] = v[0]; reg[i][1] = v[1]; reg[i][2] = v[2]; reg[i][3] = v[3];
        } else {
          const u32x2 v = *reinterpret_cast<const u32x2*>(p + mb * V);
          reg[i][0] = v[0]; reg[i][1] = v[1];
        }
      } else {
#pragma unroll
        for (int d = 0; d < V / 2; ++d) reg[i][d] = 0u;
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds) const {
    const int kb = threadIdx.x >> 5, mb = threadIdx.x & 31;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      u32x4 out;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = reg[2 * p][v >> 1];
        const uint32_t b = reg[2 * p + 1][v >> 1];
        if (SCALED) {
          const float fa = (v & 1) ? bf16_hi(a) : bf16_lo(a);
          const float fb = (v & 1) ? bf16_hi(b) : bf16_lo(b);
          out[p] = pack_bf16x2(fa * scl[2 * p], fb * scl[2 * p + 1]);
        } else {
          out[p] = (v & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
      }
      *reinterpret_cast<u32x4*>(lds + (mb * V + v) * LDS_LD + kb * 8) = out;
    }
  }
};

// ------------------------------------------------------------------ MFMA core

template <int BM, int BN>
struct Acc {
  static constexpr int TM = BM / 64;
  static constexpr int TN = BN / 64;
  f32x16 c[TM][TN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[i][j][r] = 0.f;
  }
};

__device__ __forceinline__ int wave_m() { return (threadIdx.x >> 6) & 1; }
__device__ __forceinline__ int wave_n() { return threadIdx.x >> 7; }

// row (within the tile) held by this lane for sub-tile tm
template <int BM>
__device__ __forceinline__ int lane_row(int tm) {
  return wave_m() * (BM / 2) + tm * 32 + (lane_id() & 31);
}
// first of 4 consecutive columns (within the tile) held in registers 4*g..4*g+3
template <int BN>
__device__ __forceinline__ int lane_col(int tn, int g) {
  return wave_n() * (BN / 2) + tn * 32 + 8 * g + 4 * (lane_id() >> 5);
}

template <int BM, int BN>
__device__ __forceinline__ void mma_ktile(const uint16_t* ldsP, const uint16_t* ldsQ,
                                          Acc<BM, BN>& acc) {
  constexpr int TM = BM / 64, TN = BN / 64;
  const int lane = lane_id();
  const uint16_t* pb = ldsP + (wave_m() * (BM / 2) + (lane & 31)) * LDS_LD + (lane >> 5) * 8;
  const uint16_t* qb = ldsQ + (wave_n() * (BN / 2) + (lane & 31)) * LDS_LD + (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8 pf[TM], qf[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) pf[i] = *reinterpret_cast<const bf16x8*>(pb + i * 32 * LDS_LD + kk * 16);
#pragma unroll
    for (int j = 0; j < TN; ++j) qf[j] = *reinterpret_cast<const bf16x8*>(qb + j * 32 * LDS_LD + kk * 16);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc.c[i][j] = mfma_32x32x16(qf[j], pf[i], acc.c[i][j]);
  }
}

template <int BM, int BN, class LP, class LQ>
__device__ __forceinline__ void mainloop(LP& lp, LQ& lq, int nk, uint16_t* lds, Acc<BM, BN>& acc) {
  constexpr int kStage = (BM + BN) * LDS_LD;
  if (nk <= 0) return;
  lp.fetch(0);
  lq.fetch(0);
  lp.store(lds);
  lq.store(lds + BM * LDS_LD);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint16_t* cur = lds + (kt & 1) * kStage;
    uint16_t* nxt = lds + ((kt + 1) & 1) * kStage;
    const bool more = kt + 1 < nk;
    if (more) {
      lp.fetch(kt + 1);
      lq.fetch(kt + 1);
    }
    mma_ktile<BM, BN>(cur, cur + BM * LDS_LD, acc);
    if (more) {
      lp.store(nxt);
      lq.store(nxt + BM * LDS_LD);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ scheduling

// Tile t of a persistent walk, remapped so that XCD x (= blockIdx % 8 under
// round-robin dispatch) owns a contiguous block of tile ids in every round.
__device__ __forceinline__ int64_t first_tile() {
  const int G = gridDim.x, b = blockIdx.x;
  if ((G & 7) == 0) return int64_t(b & 7) * (G >> 3) + (b >> 3);
  return b;
}

// s_pref[e] = sum_{e' < e} ceil(counts[e'] / BM), e = 0..E (E <= 1024).
__device__ void tile_prefix(const int32_t* counts, int E, int BM, int32_t* s_pref,
                            int32_t* s_tmp) {
  const int tid = threadIdx.x;
  int32_t loc[4];
  int32_t sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    loc[q] = e < E ? (counts[e] + BM - 1) / BM : 0;
    sum += loc[q];
  }
  s_tmp[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int32_t add = tid >= off ? s_tmp[tid - off] : 0;
    __syncthreads();
    s_tmp[tid] += add;
    __syncthreads();
  }
  int32_t run = s_tmp[tid] - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < E) s_pref[e] = run;
    run += loc[q];
  }
  if (tid == kThreads - 1) s_pref[E] = s_tmp[tid];
  __syncthreads();
}

// expert e with s_pref[e] <= gm < s_pref[e+1]
__device__ __forceinline__ int find_expert(const int32_t* s_pref, int E, int32_t gm) {
  int lo = 0, hi = E;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= gm) lo = mid; else hi = mid;
  }
  return lo;
}

struct RowTile {
  int e;
  int64_t row0;  // first permuted row of the tile
  int rows;      // valid rows in the tile (<= BM)
  int nt;        // n-tile index
};

template <int BM>
__device__ __forceinline__ RowTile decode_row_tile(int64_t t, int NT, const int32_t* s_pref, int E,
                                                   const int32_t* counts, const int32_t* offsets) {
  RowTile r;
  r.nt = int(t % NT);
  const int32_t gm = int32_t(t / NT);
  r.e = find_expert(s_pref, E, gm);
  const int mt = gm - s_pref[r.e];
  r.row0 = int64_t(offsets[r.e]) + int64_t(mt) * BM;
  r.rows = min(BM, counts[r.e] - mt * BM);
  return r;
}

// ------------------------------------------------------------------ epilogue helpers

__device__ __forceinline__ void store4_bf16(uint16_t* p, float a, float b, float c, float d) {
  u32x2 v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<u32x2*>(p) = v;
}

__device__ __forceinline__ void load4_bf16(const uint16_t* p, float* o) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  o[0] = bf16_lo(v[0]); o[1] = bf16_hi(v[0]); o[2] = bf16_lo(v[1]); o[3] = bf16_hi(v[1]);
}

// ================================================================== forward GEMM1
// C[r][q] = x[tok(r)] . W13[e][wrow(q)],  K = H. Q rows are arranged so that
// every wave holds gate and up columns of the same intermediate index in
// paired sub-tiles; the epilogue forms a = silu(g) * u and stores g, u (for
// the backward) and a, all as bf16.
namespace g1 {
constexpr int BM = 256, BN = 128;
constexpr int TN = BN / 64;                 // sub-tiles per wave along n (pairs of g/u)
constexpr int IPT = BN / 2;                 // intermediate indices per tile
__device__ __forceinline__ int q_to_w13_row(int q, int nt, int I) {
  const int wn = q / (BN / 2);
  const int s = (q % (BN / 2)) / 32;        // sub-tile within the wave
  const int i = nt * IPT + wn * (BN / 4) + (s >> 1) * 32 + (q & 31);
  return (s & 1) * I + i;
}
}  // namespace g1

__global__ __launch_bounds__(kThreads) void gemm1_swiglu_kernel(GemmProblem p, const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ W13,
                                                                uint16_t* __restrict__ h13,
                                                                uint16_t* __restrict__ act) {
  using namespace g1;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (BM + BN) * LDS_LD];
  __shared__ int32_t s_pref[1025];
  __shared__ int32_t s_tmp[kThreads];
  const int E = int(p.E), H = int(p.H), I = int(p.I), k = int(p.k);
  const int NT = (2 * I) / BN;
  tile_prefix(p.counts, E, BM, s_pref, s_tmp);
  const int64_t total = int64_t(s_pref[E]) * NT;
  const int nk = H / BK;
  for (int64_t t = first_tile(); t < total; t += gridDim.x) {
    const RowTile rt = decode_row_tile<BM>(t, NT, s_pref, E, p.counts, p.offsets);
    KMajorLoader<BM> lp;
#pragma unroll
    for (int i = 0; i < lp.kPer; ++i) {
      const int m = lp.row_of_thread(i);
      const uint16_t* row = nullptr;
      if (m < rt.rows) row = x + int64_t(p.src_of[rt.row0 + m] / k) * H;
      lp.set_row(i, row);
    }
    KMajorLoader<BN> lq;
#pragma unroll
    for (int i = 0; i < lq.kPer; ++i) {
      const int q = lq.row_of_thread(i);
      lq.set_row(i, W13 + (int64_t(rt.e) * 2 * I + q_to_w13_row(q, rt.nt, I)) * H);
    }
    Acc<BM, BN> acc;
    acc.zero();
    mainloop<BM, BN>(lp, lq, nk, lds, acc);
    // epilogue: pairs (2p, 2p+1) of sub-tiles are (gate, up)
#pragma unroll
    for (int tm = 0; tm < acc.TM; ++tm) {
      const int m = lane_row<BM>(tm);
      if (m >= rt.rows) continue;
      const int64_t r = rt.row0 + m;
#pragma unroll
      for (int pr = 0; pr < TN / 2; ++pr) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // column of the gate sub-tile 2*pr -> intermediate index
          const int i = rt.nt * IPT + wave_n() * (BN / 4) + pr * 32 + 8 * g + 4 * (lane_id() >> 5);
          float gv[4], uv[4], av[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gv[q] = acc.c[tm][2 * pr][4 * g + q];
            uv[q] = acc.c[tm][2 * pr + 1][4 * g + q];
            av[q] = gv[q] * sigmoidf_fast(gv[q]) * uv[q];
          }
          if (h13) {
            store4_bf16(h13 + r * 2 * I + i, gv[0], gv[1], gv[2], gv[3]);
            store4_bf16(h13 + r * 2 * I + I + i, uv[0], uv[1], uv[2], uv[3]);
          }
          store4_bf16(act + r * I + i, av[0], av[1], av[2], av[3]);
        }
      }
    }
  }
}

// ================================================================== forward GEMM2
// O[r][h] = topk_w[src_of[r]] * (a[r] . W2[e][h]),  K = I.
namespace g2 {
constexpr int BM = 256, BN = 128;
}

__global__ __launch_bounds__(kThreads) void gemm2_scale_kernel(GemmProblem p, const uint16_t* __restrict__ act,
                                                               const uint16_t* __restrict__ W2,
                                                               uint16_t* __restrict__ out) {
  using namespace g2;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (BM + BN) * LDS_LD];
  __shared__ int32_t s_pref[1025];
  __shared__ int32_t s_tmp[kThreads];
  const int E = int(p.E), H = int(p.H), I = int(p.I);
  const int NT = H / BN;
  tile_prefix(p.counts, E, BM, s_pref, s_tmp);
  const int64_t total = int64_t(s_pref[E]) * NT;
  const int nk = I / BK;
  for (int64_t t = first_tile(); t < total; t += gridDim.x) {
    const RowTile rt = decode_row_tile<BM>(t, NT, s_pref, E, p.counts, p.offsets);
    KMajorLoader<BM> lp;
#pragma unroll
    for (int i = 0; i < lp.kPer; ++i) {
      const int m = lp.row_of_thread(i);
      lp.set_row(i, m < rt.rows ? act + (rt.row0 + m) * I : nullptr);
    }
    KMajorLoader<BN> lq;
#pragma unroll
    for (int i = 0; i < lq.kPer; ++i) {
      const int q = lq.row_of_thread(i);
      lq.set_row(i, W2 + (int64_t(rt.e) * H + int64_t(rt.nt) * BN + q) * I);
    }
    Acc<BM, BN> acc;
    acc.zero();
    mainloop<BM, BN>(lp, lq, nk, lds, acc);
#pragma unroll
    for (int tm = 0; tm < acc.TM; ++tm) {
      const int m = lane_row<BM>(tm);
      if (m >= rt.rows) continue;
      const int64_t r = rt.row0 + m;
      const float w = p.topk_w[p.src_of[r]];
#pragma unroll
      for (int tn = 0; tn < acc.TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = rt.nt * BN + lane_col<BN>(tn, g);
          const f32x16& c = acc.c[tm][tn];
          store4_bf16(out + r * H + n, w * c[4 * g], w * c[4 * g + 1], w * c[4 * g + 2], w * c[4 * g + 3]);
        }
    }
  }
}

// ================================================================== backward dH
// dA_u[r][i] = dY[tok(r)] . W2[e][:, i]  (K = H; W2 read transposed), then per
// element, with g, u from the saved [g | u]:
//   a = silu(g) u,  dw partial += dA_u a,  dA = w dA_u,
//   dg = dA u sig(g) (1 + g (1 - sig(g))),  du = dA silu(g).
// dwpart[r][2*nt + wave_n] holds this wave's partial sum of dA_u * a.
namespace gdh {
constexpr int BM = 256, BN = 128;
struct W2Rows {  // k = h: row h of W2[e], entities i from n0
  const uint16_t* base;
  int64_t ld;
  __device__ __forceinline__ const uint16_t* row(int k, float&) const { return base + int64_t(k) * ld; }
};
}  // namespace gdh

int dh_num_parts(int64_t I) { return int(I / gdh::BN) * 2; }

__global__ __launch_bounds__(kThreads) void gemm_dh_kernel(GemmProblem p, const uint16_t* __restrict__ dy,
                                                           const uint16_t* __restrict__ W2,
                                                           const uint16_t* __restrict__ h13,
                                                           uint16_t* __restrict__ dh13,
                                                           float* __restrict__ dwpart) {
  using namespace gdh;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (BM + BN) * LDS_LD];
  __shared__ int32_t s_pref[1025];
  __shared__ int32_t s_tmp[kThreads];
  const int E = int(p.E), H = int(p.H), I = int(p.I), k = int(p.k);
  const int NT = I / BN;
  const int nparts = 2 * NT;
  tile_prefix(p.counts, E, BM, s_pref, s_tmp);
  const int64_t total = int64_t(s_pref[E]) * NT;
  const int nk = H / BK;
  for (int64_t t = first_tile(); t < total; t += gridDim.x) {
    const RowTile rt = decode_row_tile<BM>(t, NT, s_pref, E, p.counts, p.offsets);
    KMajorLoader<BM> lp;
#pragma unroll
    for (int i = 0; i < lp.kPer; ++i) {
      const int m = lp.row_of_thread(i);
      const uint16_t* row = nullptr;
      if (m < rt.rows) row = dy + int64_t(p.src_of[rt.row0 + m] / k) * H;
      lp.set_row(i, row);
    }
    MNMajorLoader<BN, false, W2Rows> lq;
    lq.fn.base = W2 + int64_t(rt.e) * H * I + int64_t(rt.nt) * BN;
    lq.fn.ld = I;
    Acc<BM, BN> acc;
    acc.zero();
    mainloop<BM, BN>(lp, lq, nk, lds, acc);
#pragma unroll
    for (int tm = 0; tm < acc.TM; ++tm) {
      const int m = lane_row<BM>(tm);
      const bool valid = m < rt.rows;
      const int64_t r = rt.row0 + (valid ? m : 0);
      const float w = valid ? p.topk_w[p.src_of[r]] : 0.f;
      float dws = 0.f;
      if (valid) {
#pragma unroll
        for (int tn = 0; tn < acc.TN; ++tn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int i = rt.nt * BN + lane_col<BN>(tn, g);
            float gv[4], uv[4], dg[4], du[4];
            load4_bf16(h13 + r * 2 * I + i, gv);
            load4_bf16(h13 + r * 2 * I + I + i, uv);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float dau = acc.c[tm][tn][4 * g + q];
              const float s = sigmoidf_fast(gv[q]);
              const float sg = gv[q] * s;  // silu(g)
              dws += dau * sg * uv[q];
              const float da = w * dau;
              dg[q] = da * uv[q] * s * (1.f + gv[q] * (1.f - s));
              du[q] = da * sg;
            }
            store4_bf16(dh13 + r * 2 * I + i, dg[0], dg[1], dg[2], dg[3]);
            store4_bf16(dh13 + r * 2 * I + I + i, du[0], du[1], du[2], du[3]);
          }
      }
      dws += __shfl_xor(dws, 32);
      if (valid && lane_id() < 32) dwpart[r * nparts + 2 * rt.nt + wave_n()] = dws;
    }
  }
}

// ================================================================== backward dX
// dXr[r][h] = [dg | du][r] . W13[e][:, h]  (K = 2I; W13 read transposed).
namespace gdx {
constexpr int BM = 256, BN = 128;
struct W13Rows {  // k = c: row c of W13[e], entities h from n0
  const uint16_t* base;
  int64_t ld;
  __device__ __forceinline__ const uint16_t* row(int k, float&) const { return base + int64_t(k) * ld; }
};
}  // namespace gdx

__global__ __launch_bounds__(kThreads) void gemm_dx_kernel(GemmProblem p, const uint16_t* __restrict__ dh13,
                                                           const uint16_t* __restrict__ W13,
                                                           uint16_t* __restrict__ out) {
  using namespace gdx;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (BM + BN) * LDS_LD];
  __shared__ int32_t s_pref[1025];
  __shared__ int32_t s_tmp[kThreads];
  const int E = int(p.E), H = int(p.H), I = int(p.I);
  const int NT = H / BN;
  tile_prefix(p.counts, E, BM, s_pref, s_tmp);
  const int64_t total = int64_t(s_pref[E]) * NT;
  const int nk = (2 * I) / BK;
  for (int64_t t = first_tile(); t < total; t += gridDim.x) {
    const RowTile rt = decode_row_tile<BM>(t, NT, s_pref, E, p.counts, p.offsets);
    KMajorLoader<BM> lp;
#pragma unroll
    for (int i = 0; i < lp.kPer; ++i) {
      const int m = lp.row_of_thread(i);
      lp.set_row(i, m < rt.rows ? dh13 + (rt.row0 + m) * 2 * I : nullptr);
    }
    MNMajorLoader<BN, false, W13Rows> lq;
    lq.fn.base = W13 + int64_t(rt.e) * 2 * I * H + int64_t(rt.nt) * BN;
    lq.fn.ld = H;
    Acc<BM, BN> acc;
    acc.zero();
    mainloop<BM, BN>(lp, lq, nk, lds, acc);
#pragma unroll
    for (int tm = 0; tm < acc.TM; ++tm) {
      const int m = lane_row<BM>(tm);
      if (m >= rt.rows) continue;
      const int64_t r = rt.row0 + m;
#pragma unroll
      for (int tn = 0; tn < acc.TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = rt.nt * BN + lane_col<BN>(tn, g);
          const f32x16& c = acc.c[tm][tn];
          store4_bf16(out + r * H + n, c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]);
        }
    }
  }
}

// ================================================================== weight gradients
// dW13[e][c][h] = sum_{r in seg e} dH13[r][c] x[tok(r)][h]
// dW2[e][h][i]  = sum_{r in seg e} (w_r dY[tok(r)][h]) a[r][i]
// The reduction runs over the expert's rows (K = rows_e, ragged tail
// zero-filled); an expert without rows produces an exact-zero tile.
namespace gw {
constexpr int BM = 256, BN = 128;
struct SegRows {  // k = r within the segment: direct rows
  const uint16_t* base;  // row 0 of the segment, column offset applied
  int64_t ld;
  int rows;
  __device__ __forceinline__ const uint16_t* row(int k, float&) const {
    return k < rows ? base + int64_t(k) * ld : nullptr;
  }
};
struct GatherRows {  // k = r within the segment: token row tok(r) of a [T, ld] tensor
  const uint16_t* base;  // column offset applied
  int64_t ld;
  const int32_t* src;    // src_of + segment start
  int rows;
  int kk;
  __device__ __forceinline__ const uint16_t* row(int k, float&) const {
    return k < rows ? base + int64_t(src[k] / kk) * ld : nullptr;
  }
};
struct GatherRowsScaled {  // as GatherRows, scaled by topk_w of the pair
  const uint16_t* base;
  int64_t ld;
  const int32_t* src;
  const float* w;
  int rows;
  int kk;
  __device__ __forceinline__ const uint16_t* row(int k, float& s) const {
    if (k >= rows) return nullptr;
    const int32_t f = src[k];
    s = w[f];
    return base + int64_t(f / kk) * ld;
  }
};
}  // namespace gw

__global__ __launch_bounds__(kThreads) void gemm_dw13_kernel(GemmProblem p, const uint16_t* __restrict__ dh13,
                                                             const uint16_t* __restrict__ x,
                                                             uint16_t* __restrict__ dW13) {
  using namespace gw;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (BM + BN) * LDS_LD];
  const int H = int(p.H), I = int(p.I);
  const int MT = (2 * I) / BM, NT = H / BN;
  const int64_t total = p.E * MT * NT;
  for (int64_t t = first_tile(); t < total; t += gridDim.x) {
    const int nt = int(t % NT);
    const int mt = int((t / NT) % MT);
    const int e = int(t / (int64_t(NT) * MT));
    const int rows = p.counts[e];
    const int64_t off = p.offsets[e];
    MNMajorLoader<BM, false, SegRows> lp;
    lp.fn.base = dh13 + off * 2 * I + int64_t(mt) * BM;
    lp.fn.ld = 2 * I;
    lp.fn.rows = rows;
    MNMajorLoader<BN, false, GatherRows> lq;
    lq.fn.base = x + int64_t(nt) * BN;
    lq.fn.ld = H;
    lq.fn.src = p.src_of + off;
    lq.fn.rows = rows;
    lq.fn.kk = int(p.k);
    Acc<BM, BN> acc;
    acc.zero();
    mainloop<BM, BN>(lp, lq, (rows + BK - 1) / BK, lds, acc);
    uint16_t* o = dW13 + int64_t(e) * 2 * I * H;
#pragma unroll
    for (int tm = 0; tm < acc.TM; ++tm) {
      const int64_t c = int64_t(mt) * BM + lane_row<BM>(tm);
#pragma unroll
      for (int tn = 0; tn < acc.TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int h = nt * BN + lane_col<BN>(tn, g);
          const f32x16& a = acc.c[tm][tn];
          store4_bf16(o + c * H + h, a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
    }
  }
}

__global__ __launch_bounds__(kThreads) void gemm_dw2_kernel(GemmProblem p, const uint16_t* __restrict__ dy,
                                                            const uint16_t* __restrict__ act,
                                                            uint16_t* __restrict__ dW2) {
  using namespace gw;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (BM + BN) * LDS_LD];
  const int H = int(p.H), I = int(p.I);
  const int MT = H / BM, NT = I / BN;
  const int64_t total = p.E * MT * NT;
  for (int64_t t = first_tile(); t < total; t += gridDim.x) {
    const int nt = int(t % NT);
    const int mt = int((t / NT) % MT);
    const int e = int(t / (int64_t(NT) * MT));
    const int rows = p.counts[e];
    const int64_t off = p.offsets[e];
    MNMajorLoader<BM, true, GatherRowsScaled> lp;
    lp.fn.base = dy + int64_t(mt) * BM;
    lp.fn.ld = H;
    lp.fn.src = p.src_of + off;
    lp.fn.w = p.topk_w;
    lp.fn.rows = rows;
    lp.fn.kk = int(p.k);
    MNMajorLoader<BN, false, SegRows> lq;
    lq.fn.base = act + off * I + int64_t(nt) * BN;
    lq.fn.ld = I;
    lq.fn.rows = rows;
    Acc<BM, BN> acc;
    acc.zero();
    mainloop<BM, BN>(lp, lq, (rows + BK - 1) / BK, lds, acc);
    uint16_t* o = dW2 + int64_t(e) * H * I;
#pragma unroll
    for (int tm = 0; tm < acc.TM; ++tm) {
      const int64_t h = int64_t(mt) * BM + lane_row<BM>(tm);
#pragma unroll
      for (int tn = 0; tn < acc.TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int i = nt * BN + lane_col<BN>(tn, g);
          const f32x16& a = acc.c[tm][tn];
          store4_bf16(o + h * I + i, a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
    }
  }
}

// ================================================================== launchers

static int grid_for(int64_t tiles, int num_cus) {
  int64_t g = int64_t(num_cus);  // one 256-thread workgroup per CU (LDS-bound)
  if (tiles < g) g = tiles;
  if (g < 1) g = 1;
  return int(g);
}

static int64_t row_tiles_upper(const GemmProblem& p, int BM) {
  return (p.T * p.k + BM - 1) / BM + p.E;
}

hipError_t launch_gemm1_swiglu(const GemmProblem& p, const uint16_t* x, const uint16_t* W13,
                               uint16_t* h13, uint16_t* act, hipStream_t st, KernelTimer* timer) {
  const int NT = int(2 * p.I / g1::BN);
  const int grid = grid_for(row_tiles_upper(p, g1::BM) * NT, p.num_cus);
  TimedLaunch tl(timer, "gemm1_swiglu", st);
  hipLaunchKernelGGL(gemm1_swiglu_kernel, dim3(grid), dim3(kThreads), 0, st, p, x, W13, h13, act);
  return hipGetLastError();
}

hipError_t launch_gemm2_scale(const GemmProblem& p, const uint16_t* act, const uint16_t* W2,
                              uint16_t* out_rows, hipStream_t st, KernelTimer* timer) {
  const int NT = int(p.H / g2::BN);
  const int grid = grid_for(row_tiles_upper(p, g2::BM) * NT, p.num_cus);
  TimedLaunch tl(timer, "gemm2_scale", st);
  hipLaunchKernelGGL(gemm2_scale_kernel, dim3(grid), dim3(kThreads), 0, st, p, act, W2, out_rows);
  return hipGetLastError();
}

hipError_t launch_gemm_dh(const GemmProblem& p, const uint16_t* dy, const uint16_t* W2,
                          const uint16_t* h13, uint16_t* dh13, float* dwpart, hipStream_t st,
                          KernelTimer* timer) {
  const int NT = int(p.I / gdh::BN);
  const int grid = grid_for(row_tiles_upper(p, gdh::BM) * NT, p.num_cus);
  TimedLaunch tl(timer, "gemm_dh_dswiglu", st);
  hipLaunchKernelGGL(gemm_dh_kernel, dim3(grid), dim3(kThreads), 0, st, p, dy, W2, h13, dh13, dwpart);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const GemmProblem& p, const uint16_t* dh13, const uint16_t* W13,
                          uint16_t* dx_rows, hipStream_t st, KernelTimer* timer) {
  const int NT = int(p.H / gdx::BN);
  const int grid = grid_for(row_tiles_upper(p, gdx::BM) * NT, p.num_cus);
  TimedLaunch tl(timer, "gemm_dx", st);
  hipLaunchKernelGGL(gemm_dx_kernel, dim3(grid), dim3(kThreads), 0, st, p, dh13, W13, dx_rows);
  return hipGetLastError();
}

hipError_t launch_gemm_dw13(const GemmProblem& p, const uint16_t* dh13, const uint16_t* x,
                            uint16_t* dW13, hipStream_t st, KernelTimer* timer) {
  const int64_t tiles = p.E * (2 * p.I / gw::BM) * (p.H / gw::BN);
  const int grid = grid_for(tiles, p.num_cus);
  TimedLaunch tl(timer, "gemm_dw13", st);
  hipLaunchKernelGGL(gemm_dw13_kernel, dim3(grid), dim3(kThreads), 0, st, p, dh13, x, dW13);
  return hipGetLastError();
}

hipError_t launch_gemm_dw2(const GemmProblem& p, const uint16_t* dy, const uint16_t* act,
                           uint16_t* dW2, hipStream_t st, KernelTimer* timer) {
  const int64_t tiles = p.E * (p.H / gw::BM) * (p.I / gw::BN);
  const int grid = grid_for(tiles, p.num_cus);
  TimedLaunch tl(timer, "gemm_dw2", st);
  hipLaunchKernelGGL(gemm_dw2_kernel, dim3(grid), dim3(kThreads), 0, st, p, dy, act, dW2);
  return hipGetLastError();
}

}  // namespace moe
