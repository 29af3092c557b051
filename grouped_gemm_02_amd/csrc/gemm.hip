// Grouped GEMMs of the MoE layer on gfx950 bf16 MFMA.
//
// One grouped GEMM call runs many differently-sized per-expert matrix
// products, each indexed by the expert's group offset into the permuted rows
// (kongchang.com explainer, grouped-GEMM note). Six products make up the
// layer: the gate/up GEMM with SwiGLU in its epilogue and the down GEMM
// (MarkTechPost article, "How does the fused kernel work?"), and in the
// backward the dH GEMM with the SwiGLU derivative and routing-weight-gradient
// partials in its epilogue, the dX GEMM, and the two weight-gradient GEMMs
// whose reduction dimension is each expert's row count.
//
// Structure shared by all six:
//   * Output tile C[m][n] of 256 x 256, C = sum_k P[m][k] Q[n][k], fp32
//     accumulation in MFMA registers. 512 threads = 8 waves in a 2 x 4 grid
//     (two waves per SIMD, so one wave's LDS and memory waits overlap the
//     other's MFMAs), each wave a 128 x 64 block of 4 x 2 sub-tiles of
//     v_mfma_f32_32x32x16_bf16 (128 accumulator registers per lane). The
//     MFMA's A operand is the Q fragment and its B operand the P fragment, so
//     each lane holds one row m and 16 columns n of a sub-tile (4 runs of 4
//     consecutive n): per-row scalars of the epilogue live in one lane.
//   * Both operands are staged through LDS in k-slabs of BK = 64, double
//     buffered: the global loads of slab kt+1 are in flight while slab kt is
//     multiplied. Every global load is a 16-byte chunk of a contiguous row:
//       - "k-major" operands (k contiguous in memory: activations as GEMM
//         rows, weights in the forward) sit in LDS as [entity][64 + 8 pad]
//         and are read with 16-byte ds_read_b128 fragments; where both
//         operands are k-major bf16 (the gate/up and down GEMMs) they use an
//         unpadded, XOR-swizzled [entity][64] layout instead, which loads
//         straight into LDS (buffer_load ... lds) can write, so those slabs
//         never pass through registers;
//       - "mn-major" operands (entities contiguous, one memory row per k:
//         weights in the backward data-gradient GEMMs and both operands of
//         the weight-gradient GEMMs, whose k is the token row) sit in LDS as
//         [k][entities + 32 pad] and are read with the gfx950 LDS transpose
//         read ds_read_b64_tr_b16, which hands every lane 4 consecutive k of
//         one entity. No register transposes.
//   * Epilogues go through LDS: the accumulators of one column half are
//     written there in fp32, then every thread handles 16-byte row pieces,
//     so global stores (and the loads some epilogues need) are coalesced.
//   * Persistent grid: each workgroup walks tiles blockIdx, +grid, ...; tile
//     ids are remapped so that the eight XCDs each take a contiguous range
//     (tiles of one expert share its weight panel in that XCD's L2).
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int BK = 64;
constexpr int BM = 256;   // tile rows (P entities)
constexpr int BN = 256;   // tile columns (Q entities)
constexpr int kThreads = 512;
constexpr int kWavesM = 2;
constexpr int kWavesN = 4;
constexpr int WTM = BM / kWavesM;  // 128 rows per wave
constexpr int WTN = BN / kWavesN;  // 64 columns per wave
constexpr int TM = WTM / 32;       // 4 sub-tiles
constexpr int TN = WTN / 32;       // 2 sub-tiles
constexpr int LDK = BK + 8;        // k-major LDS row: 64 k + 8 pad (bf16 elements)
constexpr int LDN = 256 + 32;      // mn-major LDS row: 256 entities + 32 pad
constexpr int kOperandLds = 256 * LDK;  // == 64 * LDN: both layouts take 36 KiB
static_assert(256 * LDK == 64 * LDN, "operand layouts must have the same LDS size");
constexpr int kStageLds = 2 * kOperandLds;  // P + Q
constexpr int kPer = 256 * 8 / kThreads;   // 16-byte chunks per thread per operand slab

// The two operand stages of the k loop are separate LDS objects, so that the
// compiler can tell reads of one stage from loads still in flight into the
// other (with one array it waits for every load into LDS before any LDS
// read). After the k loop they hold the epilogue's tile images: rows
// [0, 128) in stage 0, rows [128, 256) in stage 1.
__shared__ __attribute__((aligned(16))) uint16_t g_stage0[kStageLds];
__shared__ __attribute__((aligned(16))) uint16_t g_stage1[kStageLds];
__device__ __forceinline__ uint16_t* stage_buf(int s) { return s ? g_stage1 : g_stage0; }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ------------------------------------------------------------------ loaders

// Raw buffer resource over [base, base + bytes) (bytes < 2^32; dword 3 as
// gfx9 parts expect for untyped loads). Base and extent must be uniform and
// visibly so to the compiler (derived from scalar values), or every load
// through the resource becomes a loop over the distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(uint32_t(bytes)), 0x00020000);
}

// Register stage of one operand's k-slab plus a zero-fill mask (bit i set:
// chunk i is real data).
struct Stage {
  u32x4 r[kPer];
  uint32_t ok;
};

// k-major operand: 256 entity rows, each with its k-values contiguous.
// Loads go through a buffer resource (tile-uniform base and extent in scalar
// registers, a 32-bit byte offset per row in a vector register): an offset
// past the extent reads zero instead of faulting. Every offset addresses a
// real row: rows of the token side past the end of a ragged tile are pointed
// at a valid row and their results are never stored, so the loads need no
// predicate.
//
// Two LDS layouts of a bf16 k-major slab:
//   * padded (SWZ = false): row r at r * LDK elements (64 k + 8 pad), chunk c
//     at its own position; thread t moves chunk t % 8 of rows t/8 + 64*i
//     through registers (fetch, then store after the MFMAs).
//   * swizzled (SWZ = true): row r at r * BK elements (128 bytes, no pad),
//     its eight 16-byte k-chunks permuted: position p holds chunk p ^ swz(r),
//     swz(r) = (r / 2) % 8. Sixteen consecutive rows then put any one chunk
//     in sixteen different 16-byte bank groups, so fragment reads are free of
//     bank conflicts without padding. Thread t owns LDS slot t % 8 of rows
//     t/8 + 64*i, i.e. a wave's 64 lanes fill 1 KB of LDS contiguously, and
//     it loads the chunk that belongs in that slot. This is the layout a load
//     straight into LDS (buffer_load ... lds: no registers, no LDS store
//     instructions) can write, and slabs after a tile's first one are moved
//     that way (dma); slab 0 still goes through registers.
// The swizzled layout is used for the bf16 k-major operands that are loaded
// straight into LDS: both operands of the gate/up and down GEMMs and the
// k-major operand of the dX GEMM. The dH GEMM keeps the padded layout (there
// the XOR addressing costs registers and the straight loads did not pay).
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }

template <bool SWZ>
struct KMajorLoaderT {
  static constexpr bool kDirect = SWZ;
  __amdgpu_buffer_rsrc_t data;
  uint32_t off[kPer];  // byte offset of this thread's 16 bytes of row i in slab 0

  __device__ __forceinline__ static int row_of_thread(int i) { return (threadIdx.x >> 3) + 64 * i; }
  // base: element 0 of row 0; units: extent in 16-bit units
  __device__ __forceinline__ void set_base(const uint16_t* base, int64_t units) { data = make_rsrc(base, units * 2); }
  // row_off: offset of the row in 16-bit units. Swizzled, the chunk of slot
  // t % 8 of row t/8 + 64*i is (t % 8) ^ swz(row), the same for every i.
  __device__ __forceinline__ void set_row(int i, int64_t row_off) {
    const int c = SWZ ? int(threadIdx.x & 7) ^ kswz(int(threadIdx.x >> 3)) : int(threadIdx.x & 7);
    off[i] = uint32_t(row_off * 2) + c * 16;
  }
  __device__ __forceinline__ void fetch(int kt, Stage& st) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) st.r[i] = __builtin_amdgcn_raw_buffer_load_b128(data, off[i], kt * 2 * BK, 0);
    st.ok = ~0u;
  }
  __device__ __forceinline__ void store(uint16_t* lds, const Stage& st) const {
    const int r0 = threadIdx.x >> 3, c = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      uint16_t* dst = SWZ ? lds + (int(threadIdx.x) + 512 * i) * 8 : lds + (r0 + 64 * i) * LDK + c * 8;
      *reinterpret_cast<u32x4*>(dst) = st.r[i];
    }
  }
  // offsets of a k-major slab follow from kt alone (scalar offset)
  __device__ __forceinline__ void advance(int) {}
  // swizzled only: slab kt straight into LDS; wave w's load i fills rows
  // 8w + 64i .. +7, lane l's 16 bytes landing at byte 16 l of that 1 KB block
  __device__ __forceinline__ void dma(int kt, uint16_t* lds) const {
    static_assert(SWZ, "loads straight into LDS write the swizzled layout");
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          data, (__attribute__((address_space(3))) void*)(lds + (8 * w + 64 * i) * BK), 16, off[i], kt * 2 * BK, 0, 0);
  }
};
using KMajorLoader = KMajorLoaderT<false>;
using KMajorLoaderD = KMajorLoaderT<true>;

// mn-major operand in an unpadded, swizzled layout that loads straight into
// LDS can write: k-row k of the slab at k * 256 elements (512 bytes, the
// tile's 256 entities), its 16-byte chunk c (entities 8c .. 8c+7) at slot
// c ^ 4 (k % 4). The transpose read of a fragment has each 16-lane group
// read 4 consecutive k-rows at 4 chunks; with the XOR those 16 (row, chunk)
// pairs fall in 16 different slots of a 256-byte bank window, so the reads
// are free of bank conflicts without padding. Load i of wave w fills k-rows
// 2 (8 i + w) and 2 (8 i + w) + 1: lane l writes slot l % 32 of k-row
// 2 (8 i + w) + l / 32, loading the chunk that belongs there. k-rows past
// the end (RowFn::valid false) and chunks past the tile's columns get an
// offset beyond the buffer resource's extent, which the buffer unit reads
// as zero (into LDS too): the zero-fill costs no instruction.
//
// The rows may come from an index array (a gathered operand), and the
// vector-memory counter retires loads in order, so a wait for an index load
// issued after a slab's loads would also wait for that slab. Hence the
// offsets of a slab are built in two steps: dma(kt) issues slab kt and then
// the index loads of slab kt + 1 (request); advance(kt + 1), called after
// the slab barrier's vmcnt(0), turns them into offsets. prime(kt) does both
// at once (a tile's first slab). Slab 0 of a row tile may also go through
// registers (fetch, store) when the persistent walk prefetches it during the
// previous tile's epilogue.
constexpr uint32_t kPastExtent = 0x80000000u;  // beyond any operand's extent (< 2 GiB)

template <class RowFn>
struct MNMajorLoaderD {
  static constexpr bool kDirect = true;
  RowFn fn;
  __amdgpu_buffer_rsrc_t data;
  int nchunks = 32;           // 16-byte chunks of the tile that exist (partial last n-tile)
  uint32_t nxt[kPer];         // byte offsets of this lane's 16 bytes in the next slab
  typename RowFn::Raw raw[kPer];  // the next slab's row indices as loaded

  __device__ __forceinline__ void set_base(const uint16_t* base, int64_t units) {
    data = make_rsrc(base, units > 0 ? units * 2 : 0);
  }
  __device__ __forceinline__ static int krow(int i) { return 2 * (8 * i + int(threadIdx.x >> 6)) + (lane_id() >> 5); }
  __device__ __forceinline__ void request(int kt) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) raw[i] = fn.load(kt * BK + krow(i));
  }
  __device__ __forceinline__ void advance(int kt) {
    const int p = lane_id() & 31;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int kr = krow(i);
      const int c = p ^ (4 * (kr & 3));
      const int k = kt * BK + kr;
      // computed for every lane (row() of a clamped index is a real row, so the
      // offset is inside the extent, below 2^31) and pushed past the extent
      // where the k-row or the chunk does not exist: no branch, one select
      const uint32_t off = uint32_t(fn.row(raw[i])) * uint32_t(fn.ld) * 2u + uint32_t(c) * 16u;
      nxt[i] = off | ((fn.valid(k) && c < nchunks) ? 0u : kPastExtent);
    }
  }
  __device__ __forceinline__ void prime(int kt) {
    request(kt);
    advance(kt);
  }
  // slab kt (advanced) straight into LDS, then the index loads of slab kt + 1
  __device__ __forceinline__ void dma(int kt, uint16_t* lds) {
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          data, (__attribute__((address_space(3))) void*)(lds + (8 * i + w) * 512), 16, nxt[i], 0, 0, 0);
    request(kt + 1);
  }
  __device__ __forceinline__ void fetch(int kt, Stage& st) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) st.r[i] = __builtin_amdgcn_raw_buffer_load_b128(data, nxt[i], 0, 0);
    st.ok = ~0u;
    request(kt + 1);
  }
  __device__ __forceinline__ void store(uint16_t* lds, const Stage& st) const {
    const int w = int(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kPer; ++i) *reinterpret_cast<u32x4*>(lds + (8 * i + w) * 512 + lane_id() * 8) = st.r[i];
  }
};

// ------------------------------------------------------------------ fragments

// 32 entities x 16 k of a k-major tile: lane holds entity (lane % 32),
// k = kk*16 + 8*(lane/32) + 0..7, i.e. chunk 2 kk + lane/32 of its row.
template <bool SWZ>
__device__ __forceinline__ bf16x8 frag_k(const uint16_t* lds, int ent0, int kk) {
  const int lane = lane_id();
  const int e = ent0 + (lane & 31);
  const int c = 2 * kk + (lane >> 5);
  if constexpr (SWZ) return *reinterpret_cast<const bf16x8*>(lds + e * BK + ((c ^ kswz(e)) << 3));
  return *reinterpret_cast<const bf16x8*>(lds + e * LDK + c * 8);
}

// The same fragment from the swizzled unpadded mn-major layout of
// MNMajorLoaderD, with two transpose reads. In each 16-lane group,
// ds_read_b64_tr_b16 gives lane p element (p % 4) of the 8-byte chunk
// addressed by lane 4j + p/4, for j = 0..3. Lane p therefore addresses k-row
// k0 + p/4 at entities n0 + 4*(p % 4), and receives the 4 consecutive k of
// entity n0 + p. Rows k and k + 4, and k + 16 kk, have the same k % 4, so
// all of a sub-tile's reads share one lane offset and differ by constants.
// That offset is passed through an empty asm operand: otherwise the
// optimizer splits the address into a chain of pointer steps too long for
// the compiler to see which LDS variable the read touches, and it then
// waits for every load into LDS in flight (other stage included) first.
__device__ __forceinline__ bf16x8 frag_ms(const uint16_t* lds, int ent0, int kk) {
  const int lane = lane_id();
  const int g = lane >> 4, p = lane & 15;
  const int n = ent0 + 16 * (g & 1) + 4 * (p & 3);
  const int k0 = 8 * (g >> 1) + (p >> 2);
  int off = k0 * 256 + (((n >> 3) ^ (4 * (k0 & 3))) << 3) + (n & 7);
  asm("" : "+v"(off));
  const uint16_t* a = lds + off + kk * 16 * 256;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a + 4 * 256));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------------------ MFMA core

struct Acc {
  f32x16 c[TM][TN];
  // fp32 block scales only: the scale mantissas the accumulators are in
  // units of (see mma_slab_fp8_f32s)
  float mP[TM], mQ[TN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[i][j][r] = 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i) mP[i] = 1.f;
#pragma unroll
    for (int j = 0; j < TN; ++j) mQ[j] = 1.f;
  }
};

__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
// Waves w and w + 4 share a SIMD (w % 4) and own the two row halves of the
// same column block, so a tile whose rows end in the first half leaves each
// SIMD one wave with MFMA work instead of idling two SIMDs.
__device__ __forceinline__ int wave_m() { return wave_id() / kWavesN; }
__device__ __forceinline__ int wave_n() { return wave_id() % kWavesN; }

// tile row held by this lane in sub-tile tm
__device__ __forceinline__ int lane_row(int tm) { return wave_m() * WTM + tm * 32 + (lane_id() & 31); }
// first of 4 consecutive tile columns held in registers 4g .. 4g+3 of sub-tile tn
__device__ __forceinline__ int lane_col(int tn, int g) {
  return wave_n() * WTN + tn * 32 + 8 * g + 4 * (lane_id() >> 5);
}

// SWZ: both operands are in the layouts loads straight into LDS write (the
// swizzled k-major layout of KMajorLoaderT, the swizzled mn-major layout of
// MNMajorLoaderD); otherwise the padded layouts.
template <bool MN, bool SWZ>
__device__ __forceinline__ bf16x8 frag(const uint16_t* lds, int ent0, int kk) {
  static_assert(!MN || SWZ, "mn-major operands are staged only in the swizzled layout");
  if constexpr (MN) return frag_ms(lds, ent0, kk);
  return frag_k<SWZ>(lds, ent0, kk);
}

template <bool P_MN, bool Q_MN, bool SWZ = false>
__device__ __forceinline__ void load_frags(const uint16_t* ldsP, const uint16_t* ldsQ, int kk,
                                           bf16x8 (&pf)[TM], bf16x8 (&qf)[TN]) {
  const int pm0 = wave_m() * WTM, qn0 = wave_n() * WTN;
#pragma unroll
  for (int j = 0; j < TN; ++j) qf[j] = frag<Q_MN, SWZ>(ldsQ, qn0 + 32 * j, kk);
#pragma unroll
  for (int i = 0; i < TM; ++i) pf[i] = frag<P_MN, SWZ>(ldsP, pm0 + 32 * i, kk);
}

__device__ __forceinline__ void mma_step(const bf16x8 (&pf)[TM], const bf16x8 (&qf)[TN], Acc& acc) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc.c[i][j] = mfma_32x32x16(qf[j], pf[i], acc.c[i][j]);
}

// One k-slab (4 steps of 16) of MFMAs for this wave. With two waves per SIMD
// the other wave's MFMAs cover this wave's fragment reads, so fragments are
// single buffered (register budget: 128 accumulators share the 256 VGPRs).
template <bool P_MN, bool Q_MN, bool SWZ = false>
__device__ __forceinline__ void mma_slab(const uint16_t* ldsP, const uint16_t* ldsQ, Acc& acc) {
  // The compiler's own interleave of the fragment reads with the MFMAs
  // leaves LDS latency exposed; its built-in MFMA/DS interleave strategy 0
  // measured 2-5 % faster. (Strategy 1 was better for two k-major operands
  // while their slabs went through registers; with the slabs loaded straight
  // into LDS, strategy 0 is 1-2 % faster there too.)
  __builtin_amdgcn_iglp_opt(0);
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8 pf[TM], qf[TN];
    load_frags<P_MN, Q_MN, SWZ>(ldsP, ldsQ, kk, pf, qf);
    mma_step(pf, qf, acc);
  }
}

// Slab kt of both operands into stage buffer `buf`: when both loaders can,
// straight into LDS now; otherwise into registers (stored by store_next after
// the MFMAs). Both or neither: a slab mixing the two would need its own order
// of loads and fragment reads.
template <class LP, class LQ>
constexpr bool kBothDirect = LP::kDirect && LQ::kDirect;

template <class LP, class LQ, class SP, class SQ>
__device__ __forceinline__ void fetch_next(LP& lp, LQ& lq, int kt, uint16_t* buf, SP& sp, SQ& sq) {
  if constexpr (kBothDirect<LP, LQ>) {
    lp.dma(kt, buf);
    lq.dma(kt, buf + kOperandLds);
  } else {
    lp.fetch(kt, sp);
    lq.fetch(kt, sq);
  }
}
// Before the slab barrier: the straight-to-LDS loads of the wave have
// landed (vmcnt(0); expcnt and lgkmcnt left at their maxima).
template <class LP, class LQ>
__device__ __forceinline__ void wait_direct() {
  if constexpr (kBothDirect<LP, LQ>) __builtin_amdgcn_s_waitcnt(0x0F70);
}
template <class LP, class LQ, class SP, class SQ>
__device__ __forceinline__ void store_next(const LP& lp, const LQ& lq, uint16_t* buf, const SP& sp, const SQ& sq) {
  if constexpr (!kBothDirect<LP, LQ>) {
    lp.store(buf, sp);
    lq.store(buf + kOperandLds, sq);
  }
}

// One slab kt of the k loop out of stage `cur`; slab kt+1 (if any) goes to
// stage `nxt`. Both stages are named at compile time by the caller (the loop
// is unrolled by two), which is what lets the slab's fragment reads run while
// straight-to-LDS loads into the other stage are in flight.
template <bool P_MN, bool Q_MN, class LP, class LQ>
__device__ __forceinline__ void plain_slab(LP& lp, LQ& lq, int kt, int nk, uint16_t* cur, uint16_t* nxt, Acc& acc,
                                           bool active, Stage& sp, Stage& sq) {
  const bool more = kt + 1 < nk;
  if (more) fetch_next(lp, lq, kt + 1, nxt, sp, sq);
  if (active) mma_slab<P_MN, Q_MN, kBothDirect<LP, LQ>>(cur, cur + kOperandLds, acc);
  if (more) store_next(lp, lq, nxt, sp, sq);
  wait_direct<LP, LQ>();
  __syncthreads();
  if constexpr (kBothDirect<LP, LQ>) {
    // slab kt + 2's offsets from the indices requested with slab kt + 1's
    // loads, which the vmcnt(0) above has seen land
    if (kt + 2 < nk) {
      lp.advance(kt + 2);
      lq.advance(kt + 2);
    }
  }
}

// Straight-to-LDS slabs 0 .. nk-1, slab 0 already in stage 0: unrolled by
// two so that each slab's stages are known at compile time (the compiler
// can then tell a slab's fragment reads, transpose reads included, from the
// loads in flight into the other stage), in whole pairs and a last odd slab:
// a loop with an exit between the two halves made the compiler keep extra
// copies of values live across it (spills).
template <bool P_MN, bool Q_MN, class LP, class LQ>
__device__ __forceinline__ void direct_pairs(LP& lp, LQ& lq, int nk, Acc& acc, bool active, Stage& sp, Stage& sq) {
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    plain_slab<P_MN, Q_MN>(lp, lq, kt, nk, g_stage0, g_stage1, acc, active, sp, sq);
    plain_slab<P_MN, Q_MN>(lp, lq, kt + 1, nk, g_stage1, g_stage0, acc, active, sp, sq);
  }
  if (kt < nk) plain_slab<P_MN, Q_MN>(lp, lq, kt, nk, g_stage0, g_stage1, acc, active, sp, sq);
}

// Runs the k loop of one tile: the global loads of slab kt+1 are in flight
// while slab kt is multiplied out of one LDS stage, either straight into the
// other stage or into registers that are written there after the MFMAs.
// `active` (uniform per wave) is false for a wave whose tile rows are all
// past the end of a ragged tile: it still moves data, but skips the MFMAs.
// mainloop_staged runs the k loop with slab 0 already fetched into sp, sq
// (the persistent row-tile kernels fetch a tile's first slab during the
// previous tile's epilogue); mainloop fetches it itself.
template <bool P_MN, bool Q_MN, class LP, class LQ>
__device__ __forceinline__ void mainloop_staged(LP& lp, LQ& lq, int nk, Acc& acc, bool active, Stage& sp,
                                                Stage& sq) {
  if (nk <= 0) return;
  lp.store(g_stage0, sp);
  lq.store(g_stage0 + kOperandLds, sq);
  __syncthreads();
  if constexpr (kBothDirect<LP, LQ>) {
    if (nk > 1) {
      lp.advance(1);
      lq.advance(1);
    }
  }
  static_assert(LP::kDirect == LQ::kDirect, "both operands or neither load straight into LDS");
  if constexpr (!kBothDirect<LP, LQ>) {
    // slabs through registers: one loop body (unrolled by two it would not
    // fit the registers of the weight-gradient GEMMs)
    for (int kt = 0; kt < nk; ++kt)
      plain_slab<P_MN, Q_MN>(lp, lq, kt, nk, stage_buf(kt & 1), stage_buf((kt + 1) & 1), acc, active, sp, sq);
  } else {
    direct_pairs<P_MN, Q_MN>(lp, lq, nk, acc, active, sp, sq);
  }
}

template <bool P_MN, bool Q_MN, class LP, class LQ>
__device__ __forceinline__ void mainloop(LP& lp, LQ& lq, int nk, Acc& acc, bool active = true) {
  if (nk <= 0) return;
  Stage sp, sq;
  lp.fetch(0, sp);
  lq.fetch(0, sq);
  mainloop_staged<P_MN, Q_MN>(lp, lq, nk, acc, active, sp, sq);
}

// The k loop of a tile whose operands both load straight into LDS, with
// slab 0 loaded the same way (no register stage): the weight-gradient
// GEMMs, which do not prefetch across tiles.
template <bool P_MN, bool Q_MN, class LP, class LQ>
__device__ __forceinline__ void mainloop_direct(LP& lp, LQ& lq, int nk, Acc& acc, bool active = true) {
  static_assert(kBothDirect<LP, LQ>, "both operands load straight into LDS");
  if (nk <= 0) return;
  lp.dma(0, g_stage0);
  lq.dma(0, g_stage0 + kOperandLds);
  wait_direct<LP, LQ>();
  __syncthreads();
  if (nk > 1) {
    lp.advance(1);
    lq.advance(1);
  }
  Stage sp, sq;  // unused: straight-to-LDS slabs pass no registers
  direct_pairs<P_MN, Q_MN>(lp, lq, nk, acc, active, sp, sq);
}

// ------------------------------------------------------------------ FP8 core
// FP8 (E4M3) operands use the k-major LDS layout with bytes in place of bf16
// elements: a k-slab is 128 codes = 128 bytes per row, the bytes of a bf16
// slab, so the same 16-byte loads move it. The row's 4 scale bytes of the
// slab (one per 32 codes) go into the row's LDS padding, at byte 128.
//
// Each 64-deep step is one v_mfma_scale_f32_32x32x64_f8f6f4 per sub-tile
// pair. Operand layout (measured on gfx950): a lane of half h = lane / 32
// holds row lane % 32 with k = 16h .. 16h+15 in its registers 0-3 and
// k = 32+16h .. 32+16h+15 in registers 4-7, while its scale operand is the
// scale of k-block h (k = 32h .. 32h+31) of that row. The registers are
// filled so that register order is memory order; the lane then passes the
// scale byte of memory block h of the step.
typedef int i32x8 __attribute__((ext_vector_type(8)));

struct Stage8 {
  u32x4 r[kPer];
  uint32_t s;  // the slab's 4 scale bytes of row t/8 + 64 * (t % 4)
};

// k-major E4M3 operand with scales [rows, K/32]. Loads go through buffer
// resources (base and extent in scalar registers, a 32-bit byte offset per
// row in a vector register): an address past the extent reads zero instead
// of faulting, and no 64-bit per-row pointers occupy vector registers.
// Offsets are set in 16-bit units like KMajorLoader's (K/2 units per row);
// the scale row of a code row at byte offset o is at byte o/32 of the scales.
// Of the 8 threads that share 4 rows, thread t also moves the scales of row
// t/8 + 64 * (t % 4) (threads t and t+4 duplicate each other, which keeps
// every load and LDS write unconditional).
struct KMajorLoader8 : KMajorLoader {
  static constexpr bool kDirect = false;
  __amdgpu_buffer_rsrc_t scale;
  uint32_t soff;  // byte offset of the scale row this thread moves

  // base: codes of row 0 (as 16-bit units), units: extent in 16-bit units;
  // sbase / sbytes: the matching scale bytes
  __device__ __forceinline__ void set_base(const uint16_t* base, int64_t units, const uint8_t* sbase,
                                           int64_t sbytes) {
    KMajorLoader::set_base(base, units);
    scale = make_rsrc(sbase, sbytes);
  }
  // (the FP8 layout keeps chunk t % 8 in slot t % 8, rows padded to LDK)
  __device__ __forceinline__ void set_row(int i, int64_t row_off) {
    off[i] = uint32_t(row_off * 2) + (threadIdx.x & 7) * 16;
    if (int(threadIdx.x & 3) == i) soff = uint32_t(row_off * 2) >> 5;
  }
  __device__ __forceinline__ void fetch(int kt, Stage8& st) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) st.r[i] = __builtin_amdgcn_raw_buffer_load_b128(data, off[i], kt * 2 * BK, 0);
    st.s = __builtin_amdgcn_raw_buffer_load_b32(scale, soff, kt * 4, 0);
  }
  __device__ __forceinline__ void store(uint16_t* lds, const Stage8& st) const {
    const int r0 = threadIdx.x >> 3, c = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < kPer; ++i) *reinterpret_cast<u32x4*>(lds + (r0 + 64 * i) * LDK + c * 8) = st.r[i];
    *reinterpret_cast<uint32_t*>(lds + (r0 + 64 * (c & 3)) * LDK + BK) = st.s;
  }
};

// An E4M3 operand loaded straight into LDS: the codes in the swizzled
// k-major layout of KMajorLoaderD (a row's slab is 128 codes, the 128 bytes
// of a bf16 slab), the slab's scale words (4 bytes per row: four E8M0 bytes,
// or one fp32 block scale) after them, at kScaleWords8, in thread order:
// thread t moves the word of row (t / 8) + 64 (t % 4), whose code offsets it
// already holds, to word t (each row twice), so row e's word is word
// 8 (e % 64) + e / 64. Slab 0 of a row tile may go through registers
// (fetch, store) when the persistent walk prefetches it.
constexpr int kScaleWords8 = 16384;  // 16-bit units: byte 32768 of an operand region
static_assert(2 * kScaleWords8 + 4 * kThreads <= 2 * kOperandLds, "codes and scale words fit an operand region");

struct KMajorLoader8D : KMajorLoaderD {
  __amdgpu_buffer_rsrc_t scale;
  uint32_t soff;  // byte offset of the scale word this thread moves (slab 0)

  __device__ __forceinline__ void set_base(const uint16_t* base, int64_t units, const uint8_t* sbase,
                                           int64_t sbytes) {
    KMajorLoaderD::set_base(base, units);
    scale = make_rsrc(sbase, sbytes);
  }
  __device__ __forceinline__ void set_row(int i, int64_t row_off) {
    KMajorLoaderD::set_row(i, row_off);
    if (int(threadIdx.x & 3) == i) soff = uint32_t(row_off * 2) >> 5;
  }
  __device__ __forceinline__ void fetch(int kt, Stage8& st) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) st.r[i] = __builtin_amdgcn_raw_buffer_load_b128(data, off[i], kt * 2 * BK, 0);
    st.s = __builtin_amdgcn_raw_buffer_load_b32(scale, soff, kt * 4, 0);
  }
  __device__ __forceinline__ void store(uint16_t* lds, const Stage8& st) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) *reinterpret_cast<u32x4*>(lds + (int(threadIdx.x) + 512 * i) * 8) = st.r[i];
    *reinterpret_cast<uint32_t*>(lds + kScaleWords8 + 2 * int(threadIdx.x)) = st.s;
  }
  __device__ __forceinline__ void dma(int kt, uint16_t* lds) const {
    KMajorLoaderD::dma(kt, lds);
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        scale, (__attribute__((address_space(3))) void*)(lds + kScaleWords8 + w * 128), 4, soff, kt * 4, 0, 0);
  }
};

template <bool FP8>
using KLoader = typename std::conditional<FP8, KMajorLoader8, KMajorLoader>::type;
// the bf16 operand moved straight into LDS (swizzled layout); E4M3 operands
// of the row-tile walks stay on the register path (straight into LDS, their
// kernels spill 6-14 registers and measured 1.4-7 % slower)
template <bool FP8>
using KLoaderD = typename std::conditional<FP8, KMajorLoader8, KMajorLoaderD>::type;

// k-major E2M1 operand (FP4 weights: two codes per byte, the even k in the
// low nibble) with scales [rows, K/32]. A k-slab is 128 codes = 64 bytes per
// row, kept in the first 64 bytes of the FP8 LDS row, its 4 scale bytes at
// byte 128 as for FP8. Thread t moves chunk t % 4 of rows t/4 and t/4 + 128,
// and the scale bytes of row t/4 + 128 * (t % 2) (threads t and t+2
// duplicate each other, which keeps every load and LDS write unconditional).
// Offsets are set in 16-bit units (K/4 units per row); the scale row of a
// code row at byte offset o is at byte o/16 of the scales.
struct Stage4 {
  u32x4 r[2];
  uint32_t s;
};

struct KMajorLoader4 {
  static constexpr bool kDirect = false;
  __amdgpu_buffer_rsrc_t data, scale;
  uint32_t off[2];
  uint32_t soff;
  static constexpr int kRows = 2;

  __device__ __forceinline__ static int row_of_thread(int i) { return (threadIdx.x >> 2) + 128 * i; }
  __device__ __forceinline__ void set_base(const uint16_t* base, int64_t units, const uint8_t* sbase,
                                           int64_t sbytes) {
    data = make_rsrc(base, units * 2);
    scale = make_rsrc(sbase, sbytes);
  }
  __device__ __forceinline__ void set_row(int i, int64_t row_off) {
    off[i] = uint32_t(row_off * 2) + (threadIdx.x & 3) * 16;
    if (int(threadIdx.x & 1) == i) soff = uint32_t(row_off * 2) >> 4;
  }
  __device__ __forceinline__ void fetch(int kt, Stage4& st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) st.r[i] = __builtin_amdgcn_raw_buffer_load_b128(data, off[i], kt * 64, 0);
    st.s = __builtin_amdgcn_raw_buffer_load_b32(scale, soff, kt * 4, 0);
  }
  __device__ __forceinline__ void store(uint16_t* lds, const Stage4& st) const {
    const int r0 = threadIdx.x >> 2, c = threadIdx.x & 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(lds + (r0 + 128 * i) * LDK + c * 8) = st.r[i];
    *reinterpret_cast<uint32_t*>(lds + (r0 + 128 * (c & 1)) * LDK + BK) = st.s;
  }
};

template <class L> struct StageOf { using type = Stage; };
template <> struct StageOf<KMajorLoader8> { using type = Stage8; };
template <> struct StageOf<KMajorLoader8D> { using type = Stage8; };
template <> struct StageOf<KMajorLoader4> { using type = Stage4; };

// SWZ: the operand was moved by KMajorLoader8D (swizzled codes, scale
// words in thread order); otherwise by KMajorLoader8 (padded rows, scale
// word in the row's padding).
template <bool SWZ = false>
__device__ __forceinline__ i32x8 frag8(const uint16_t* lds, int ent0, int s) {
  const int lane = lane_id();
  u32x4 a, b;
  if constexpr (SWZ) {
    // 16-byte chunks 4s + h and 4s + 2 + h of the row
    const int e = ent0 + (lane & 31), h = lane >> 5;
    a = *reinterpret_cast<const u32x4*>(lds + e * BK + (((4 * s + h) ^ kswz(e)) << 3));
    b = *reinterpret_cast<const u32x4*>(lds + e * BK + (((4 * s + 2 + h) ^ kswz(e)) << 3));
  } else {
    const uint16_t* p = lds + (ent0 + (lane & 31)) * LDK + s * 32 + (lane >> 5) * 8;
    a = *reinterpret_cast<const u32x4*>(p);       // codes 16h .. 16h+15 of the step
    b = *reinterpret_cast<const u32x4*>(p + 16);  // codes 32+16h .. 32+16h+15
  }
  return i32x8{int(a[0]), int(a[1]), int(a[2]), int(a[3]), int(b[0]), int(b[1]), int(b[2]), int(b[3])};
}

// where KMajorLoader8D put row e's scale word (16-bit units from the operand)
__device__ __forceinline__ int scale_pos8(int e) { return kScaleWords8 + 2 * (8 * (e & 63) + (e >> 6)); }

// An E2M1 operand of the same MFMA (measured on gfx950): a lane of half h
// holds k = 32h .. 32h+31 of its row as 32 nibbles in registers 0-3, value
// 2j in the low nibble of byte j, i.e. 16 consecutive bytes of the row; its
// scale is that of k-block h, as for FP8 (the instruction reads 4 registers).
__device__ __forceinline__ i32x8 frag4(const uint16_t* lds, int ent0, int s) {
  const int lane = lane_id();
  const u32x4 a = *reinterpret_cast<const u32x4*>(lds + (ent0 + (lane & 31)) * LDK + s * 16 + (lane >> 5) * 8);
  return i32x8{int(a[0]), int(a[1]), int(a[2]), int(a[3]), 0, 0, 0, 0};
}

// fp32 scale of this lane's row for the slab: with fp32 block scales
// (kRuleF32) the slab's 4 scale bytes of a row are one float, the scale of
// its 128-code block
template <bool SWZ = false>
__device__ __forceinline__ float fscale8(const uint16_t* lds, int ent0) {
  const int e = ent0 + (lane_id() & 31);
  return *reinterpret_cast<const float*>(lds + (SWZ ? scale_pos8(e) : e * LDK + BK));
}

// s = m * 2^e with m in [1, 2) and e in E8M0's range [-127, 127]; a
// subnormal s (amax / 448 below 2^-126) takes e = -127 and m < 1
__device__ __forceinline__ void split_scale(float s, int& e, float& m) {
  const uint32_t u = __float_as_uint(s);
  const int be = int((u >> 23) & 0xFFu);
  if (be == 0) {
    e = -127;
    m = s * 1.7014118346046923e38f;  // * 2^127, exact
  } else {
    e = be - 127;
    m = __uint_as_float((u & 0x007FFFFFu) | 0x3F800000u);
  }
}

// One slab with fp32 block scales. The slab is one 128-deep block of both
// operands. A lane's accumulators are one P row and 16 Q columns of one
// 32-row group, which never straddles a 128-row weight block, so the
// block's scale product s_P[m] * s_Q[n-block] is one float per lane and
// sub-tile. Write it m_P m_Q 2^(e_P + e_Q): the MFMA applies 2^(e_P + e_Q)
// through its E8M0 scale operands, and the accumulators are kept in units of
// the current block's m_P m_Q (bounded, [1, 4)): each slab first rescales
// them by the previous block's m_P m_Q over this one's, and after the last
// slab mainloop_staged_fp8 multiplies by the last m_P m_Q.
template <bool SWZ = false>
__device__ __forceinline__ void mma_slab_fp8_f32s(const uint16_t* ldsP, const uint16_t* ldsQ, Acc& acc) {
  const int pm0 = wave_m() * WTM, qn0 = wave_n() * WTN;
  int pe[TM], qe[TN];
  float pmant[TM], qmant[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) split_scale(fscale8<SWZ>(ldsP, pm0 + 32 * i), pe[i], pmant[i]);
#pragma unroll
  for (int j = 0; j < TN; ++j) split_scale(fscale8<SWZ>(ldsQ, qn0 + 32 * j), qe[j], qmant[j]);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float r = (acc.mP[i] * acc.mQ[j]) * __builtin_amdgcn_rcpf(pmant[i] * qmant[j]);
#pragma unroll
      for (int q = 0; q < 16; ++q) acc.c[i][j][q] *= r;
    }
#pragma unroll
  for (int i = 0; i < TM; ++i) acc.mP[i] = pmant[i];
#pragma unroll
  for (int j = 0; j < TN; ++j) acc.mQ[j] = qmant[j];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    i32x8 qf[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) qf[j] = frag8<SWZ>(ldsQ, qn0 + 32 * j, s);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const i32x8 pf = frag8<SWZ>(ldsP, pm0 + 32 * i, s);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[j], pf, acc.c[i][j], 0, 0, 0, qe[j] + 127,
                                                                      0, pe[i] + 127);
    }
  }
}

// the accumulators back from units of the last block's m_P m_Q
__device__ __forceinline__ void finish_f32s(Acc& acc) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float f = acc.mP[i] * acc.mQ[j];
#pragma unroll
      for (int q = 0; q < 16; ++q) acc.c[i][j][q] *= f;
    }
}

// The slab's 4 scale bytes of this lane's row, one LDS word (byte 2s + h is
// the scale of k-block h of step s)
template <bool SWZ = false>
__device__ __forceinline__ uint32_t scale_word8(const uint16_t* lds, int ent0) {
  const int e = ent0 + (lane_id() & 31);
  return *reinterpret_cast<const uint32_t*>(lds + (SWZ ? scale_pos8(e) : e * LDK + BK));
}
__device__ __forceinline__ int scale_byte8(uint32_t w, int s) {
  return int((w >> (8 * (2 * s + (lane_id() >> 5)))) & 0xFFu);
}

template <bool W4 = false, bool F32S = false, bool SWZ = false>
__device__ __forceinline__ void mma_slab_fp8(const uint16_t* ldsP, const uint16_t* ldsQ, Acc& acc) {
  static_assert(!(W4 && SWZ), "FP4 weights go through registers");
  if constexpr (F32S) {
    static_assert(!W4, "fp32 block scales are for E4M3 operands");
    mma_slab_fp8_f32s<SWZ>(ldsP, ldsQ, acc);
    return;
  }
  const int pm0 = wave_m() * WTM, qn0 = wave_n() * WTN;
  // scale words of the slab: one LDS read per row block
  uint32_t qsw[TN], psw[TM];
#pragma unroll
  for (int j = 0; j < TN; ++j) qsw[j] = scale_word8<SWZ>(ldsQ, qn0 + 32 * j);
#pragma unroll
  for (int i = 0; i < TM; ++i) psw[i] = scale_word8<SWZ>(ldsP, pm0 + 32 * i);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    i32x8 qf[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) qf[j] = W4 ? frag4(ldsQ, qn0 + 32 * j, s) : frag8<SWZ>(ldsQ, qn0 + 32 * j, s);
    if constexpr (SWZ) {
      // straight-to-LDS slabs: the compiler's own order (the pipelined form
      // below costs registers these k loops do not have)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const i32x8 pf = frag8<SWZ>(ldsP, pm0 + 32 * i, s);
        const int ps = scale_byte8(psw[i], s);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[j], pf, acc.c[i][j], 0, 0, 0,
                                                                        scale_byte8(qsw[j], s), 0, ps);
      }
      continue;
    }
    // the P fragments are software-pipelined: row block i+1's read is issued
    // before row block i's MFMAs, so its LDS latency hides behind them
    i32x8 pf = frag8<SWZ>(ldsP, pm0, s);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      i32x8 pn;
      if (i + 1 < TM) pn = frag8<SWZ>(ldsP, pm0 + 32 * (i + 1), s);
      __builtin_amdgcn_sched_barrier(0);
      const int ps = scale_byte8(psw[i], s);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[j], pf, acc.c[i][j], W4 ? 4 : 0, 0, 0,
                                                                      scale_byte8(qsw[j], s), 0, ps);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < TM) pf = pn;
    }
  }
}

// One FP8 slab loaded straight into LDS (both operands KMajorLoader8D): slab
// kt out of stage `cur`, slab kt+1 into `nxt` (both compile-time objects).
template <bool F32S, class LP, class LQ>
__device__ __forceinline__ void fp8_direct_slab(LP& lp, LQ& lq, int kt, int nk, uint16_t* cur, uint16_t* nxt,
                                                Acc& acc, bool active) {
  if (kt + 1 < nk) {
    lp.dma(kt + 1, nxt);
    lq.dma(kt + 1, nxt + kOperandLds);
  }
  if (active) mma_slab_fp8<false, F32S, true>(cur, cur + kOperandLds, acc);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the slab's loads into LDS have landed (vmcnt(0))
  __syncthreads();
}

// Straight-to-LDS FP8 slabs 0 .. nk-1, slab 0 in stage 0, in whole pairs
// and a last odd slab (as direct_pairs).
template <bool F32S, class LP, class LQ>
__device__ __forceinline__ void fp8_direct_pairs(LP& lp, LQ& lq, int nk, Acc& acc, bool active) {
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    fp8_direct_slab<F32S>(lp, lq, kt, nk, g_stage0, g_stage1, acc, active);
    fp8_direct_slab<F32S>(lp, lq, kt + 1, nk, g_stage1, g_stage0, acc, active);
  }
  if (kt < nk) fp8_direct_slab<F32S>(lp, lq, kt, nk, g_stage0, g_stage1, acc, active);
}

// The FP8 k loop with slab 0 already fetched into sp, sq (row-tile walks).
template <bool F32S = false, class LP = KMajorLoader8, class LQ = KMajorLoader8>
__device__ __forceinline__ void mainloop_staged_fp8(LP& lp, LQ& lq, int nk, Acc& acc, bool active,
                                                    typename StageOf<LP>::type& sp,
                                                    typename StageOf<LQ>::type& sq) {
  constexpr bool W4 = std::is_same<LQ, KMajorLoader4>::value;
  static_assert(LP::kDirect == LQ::kDirect, "both operands or neither load straight into LDS");
  if (nk <= 0) return;
  lp.store(g_stage0, sp);
  lq.store(g_stage0 + kOperandLds, sq);
  __syncthreads();
  if constexpr (kBothDirect<LP, LQ>) {
    fp8_direct_pairs<F32S>(lp, lq, nk, acc, active);
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      uint16_t* cur = stage_buf(kt & 1);
      uint16_t* nxt = stage_buf((kt + 1) & 1);
      const bool more = kt + 1 < nk;
      if (more) {
        lp.fetch(kt + 1, sp);
        lq.fetch(kt + 1, sq);
      }
      if (active) mma_slab_fp8<W4, F32S>(cur, cur + kOperandLds, acc);
      // unconditional (after the last slab it rewrites stale data into the idle
      // buffer): a conditional block here lets the compiler sink the MFMAs
      // below it, with every fragment of the slab live at once
      lp.store(nxt, sp);
      lq.store(nxt + kOperandLds, sq);
      __syncthreads();
    }
  }
  if constexpr (F32S) finish_f32s(acc);
}

// The FP8 k loop of a tile that loads its own slab 0.
template <bool F32S = false, class LP, class LQ>
__device__ __forceinline__ void mainloop_fp8(LP& lp, LQ& lq, int nk, Acc& acc, bool active = true) {
  if (nk <= 0) return;
  if constexpr (kBothDirect<LP, LQ>) {
    lp.dma(0, g_stage0);
    lq.dma(0, g_stage0 + kOperandLds);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    fp8_direct_pairs<F32S>(lp, lq, nk, acc, active);
    if constexpr (F32S) finish_f32s(acc);
  } else {
    Stage8 sp, sq;
    lp.fetch(0, sp);
    lq.fetch(0, sq);
    mainloop_staged_fp8<F32S>(lp, lq, nk, acc, active, sp, sq);
  }
}

// ------------------------------------------------------------------ LDS-staged epilogue
// After the k loop the operand buffers are free. The accumulators of the
// waves of one column half (wave_n() in {2h, 2h+1}) are written there as fp32
// F[m][c], m < 256, c < 128 (this half's columns, in tile order).
constexpr int FLD = 128 + 4;  // fp32 row stride (the pad spreads rows over banks)
static_assert(128 * FLD * 4 <= kStageLds * 2, "fp32 staging of 128 rows must fit one operand stage");
// row m of the fp32 staging (rows [0, 128) in stage 0, [128, 256) in stage 1)
__device__ __forceinline__ float* frow(int m) {
  return reinterpret_cast<float*>(m < BM / 2 ? g_stage0 : g_stage1) + (m & (BM / 2 - 1)) * FLD;
}
constexpr int kRowPass = kThreads / 16;  // rows per pass when 16 threads share a row

__device__ __forceinline__ void stage_half(const Acc& acc, int half) {
  if ((wave_n() >> 1) != half) return;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = lane_row(tm);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = lane_col(tn, g) - half * 128;
        const f32x16& a = acc.c[tm][tn];
        const f32x4 v = {a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
        *reinterpret_cast<f32x4*>(frow(m) + c) = v;
      }
  }
}

// Plain bf16 store of the tile into a row-major [*, ld] output starting at
// (row0, col0); rows beyond `rows` and columns beyond `cols` are not written.
// With a row map, tile row m goes to output row rowmap[row0 + m] instead.
// Every wave rounds its accumulators to bf16 (round to nearest even, as the
// output would be) into a [256][256 + 8] LDS image (8-byte writes, two per
// bank pair at most); then thread t copies 16-byte pieces (column chunk
// t % 32) of rows t/32 + 16*j, so each row goes out as one 512-byte run.
constexpr int LDT = BN + 8;
static_assert((BM / 2) * LDT <= kStageLds, "half of the bf16 tile image must fit one operand stage");
// row m of the bf16 tile image (rows [0, 128) in stage 0, [128, 256) in stage 1)
__device__ __forceinline__ uint16_t* img_row(int m) {
  return (m < BM / 2 ? g_stage0 : g_stage1) + (m & (BM / 2 - 1)) * LDT;
}

// store_tile in two halves: stage_image writes the bf16 image (and loads the
// row map, so its latency overlaps the image writes) and waits; copy_image
// writes the image out and waits. Callers may issue other loads between the
// two, so that their waits do not include the image's stores.
__device__ __forceinline__ void stage_image(const Acc& acc, int64_t row0, int rows,
                                            const int32_t* rowmap, int32_t* s_map) {
  if (rowmap && int(threadIdx.x) < rows) s_map[threadIdx.x] = rowmap[row0 + threadIdx.x];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = lane_row(tm);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc.c[tm][tn];
        const u32x2 v = {pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
        *reinterpret_cast<u32x2*>(img_row(m) + lane_col(tn, g)) = v;
      }
  }
  __syncthreads();
}

// The image's rows out to global memory with streaming (nontemporal) stores:
// every output of these GEMMs (the down GEMM's and dX's rows, summed by a
// combine; the weight gradients) is written once and not read again by the
// next tiles, and cached stores displaced the operand rows that the
// concurrent tiles share in L2 (the weight-gradient GEMMs ran 6 % slower).
__device__ __forceinline__ void copy_image(uint16_t* out, int64_t ld, int64_t row0,
                                           int64_t col0, int rows, int cols, const int32_t* rowmap,
                                           const int32_t* s_map) {
  const int c = (threadIdx.x & 31) * 8;
  if (c < cols) {
    for (int m = threadIdx.x >> 5; m < rows; m += kThreads / 32) {
      const int64_t orow = rowmap ? int64_t(s_map[m]) : row0 + m;
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(img_row(m) + c),
                                  reinterpret_cast<u32x4*>(out + orow * ld + col0 + c));
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void store_tile(const Acc& acc, uint16_t* out, int64_t ld,
                                           int64_t row0, int64_t col0, int rows, int cols) {
  stage_image(acc, row0, rows, nullptr, nullptr);
  copy_image(out, ld, row0, col0, rows, cols, nullptr, nullptr);
}

// ------------------------------------------------------------------ scheduling

// Tile of a persistent walk, remapped so that XCD x (= blockIdx % 8 under
// round-robin dispatch) owns a contiguous block of tile ids in every round.
__device__ __forceinline__ int64_t first_tile() {
  const int G = gridDim.x, b = blockIdx.x;
  if ((G & 7) == 0) return int64_t(b & 7) * (G >> 3) + (b >> 3);
  return b;
}

// s_pref[e] = sum_{e' < e} ceil(counts[e'] / BM), e = 0..E (E <= 1024).
__device__ void tile_prefix(const int32_t* counts, int E, int32_t* s_pref, int32_t* s_tmp) {
  constexpr int kPerT = (1024 + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  int32_t loc[kPerT];
  int32_t sum = 0;
#pragma unroll
  for (int q = 0; q < kPerT; ++q) {
    const int e = tid * kPerT + q;
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
  for (int q = 0; q < kPerT; ++q) {
    const int e = tid * kPerT + q;
    if (e < E) s_pref[e] = run;
    run += loc[q];
  }
  if (tid == kThreads - 1) s_pref[E] = s_tmp[tid];
  __syncthreads();
}

// expert e with s_pref[e] <= gm < s_pref[e+1]
__device__ __forceinline__ int find_expert(const int32_t* s_pref, int E, int32_t gm) {
  int lo = 0, hi = E;
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

__device__ __forceinline__ RowTile decode_row_tile(int64_t t, int NT, const int32_t* s_pref, int E,
                                                   const int32_t* counts, const int32_t* offsets) {
  RowTile r;
  // the search reads LDS into vector registers; the result is the same in
  // every lane, and saying so keeps the tile's bases in scalar registers
  r.e = __builtin_amdgcn_readfirstlane(find_expert(s_pref, E, int32_t(t / NT)));
  const int32_t m0 = __builtin_amdgcn_readfirstlane(s_pref[r.e]);
  const int32_t mtiles = __builtin_amdgcn_readfirstlane(s_pref[r.e + 1]) - m0;
  // an expert's tiles are walked n-tile by n-tile: all its m-tiles of one
  // weight panel are neighbours in the walk (so they run together and share
  // the panel in L2), and a cut between two rounds or two XCDs re-reads
  // activation rows rather than weight panels
  const int32_t l = int32_t(t - int64_t(m0) * NT);
  r.nt = l / mtiles;
  const int mt = l - r.nt * mtiles;
  r.row0 = int64_t(offsets[r.e]) + int64_t(mt) * BM;
  r.rows = min(BM, counts[r.e] - mt * BM);
  return r;
}

__device__ __forceinline__ void store4_bf16(uint16_t* p, float a, float b, float c, float d) {
  u32x2 v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<u32x2*>(p) = v;
}
// the same as a streaming (nontemporal) store: for data no later kernel of
// the step reads soon, which then does not displace operands in the caches
__device__ __forceinline__ void store4_bf16_nt(uint16_t* p, float a, float b, float c, float d) {
  __builtin_nontemporal_store(u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)}, reinterpret_cast<u32x2*>(p));
}


#define MOE_ROW_SCHED                                                          \
  __shared__ int32_t s_pref[1025];                                             \
  __shared__ int32_t s_tmp[kThreads];                                          \
  tile_prefix(p.counts, E, s_pref, s_tmp);

// Persistent walk over row tiles. With PREFETCH the next tile's loaders are
// set up and its first k-slab fetched into registers before the current
// tile's epilogue runs, so that fetch's latency is spent on the epilogue
// (kernels whose epilogue needs the registers turn it off). setup(t, state)
// configures lp and lq for tile t; epi(state, acc) must not use lp or lq.
struct TileState {
  RowTile rt;
  float w;  // routing weight of tile row threadIdx.x (kernels that need it)
};

template <bool FP8, bool Q_MN, bool PREFETCH, bool F32S = false, class LP, class LQ, class Setup, class Epi>
__device__ __forceinline__ void row_tile_walk(int64_t total, int nk, LP& lp, LQ& lq, Setup&& setup,
                                              Epi&& epi) {
  typename StageOf<LP>::type sp;
  typename StageOf<LQ>::type sq;
  TileState cur, nxt;
  int64_t t = first_tile();
  if (PREFETCH && t < total) {
    setup(t, cur);
    lp.fetch(0, sp);
    lq.fetch(0, sq);
  }
  while (t < total) {
    if (!PREFETCH) {
      setup(t, cur);
      lp.fetch(0, sp);
      lq.fetch(0, sq);
    }
    Acc acc;
    acc.zero();
    const bool active = wave_m() * WTM < cur.rt.rows;
    if constexpr (FP8)
      mainloop_staged_fp8<F32S>(lp, lq, nk, acc, active, sp, sq);
    else
      mainloop_staged<false, Q_MN>(lp, lq, nk, acc, active, sp, sq);
    t += gridDim.x;
    if (PREFETCH && t < total) {
      setup(t, nxt);
      lp.fetch(0, sp);
      lq.fetch(0, sq);
    }
    epi(cur, acc);
    if (PREFETCH) cur = nxt;
  }
}

// ================================================================== forward GEMM1
// C[r][q] = x[tok(r)] . W13[e][wrow(q)],  K = H. Q rows are arranged so that
// each wave's two sub-tiles are (gate, up) of the same 32 intermediate
// indices; the epilogue forms a = silu(g) * u and stores g and u (for the
// backward) and w * a (routing weight folded in: the down GEMM then needs no
// scale, and the dW2 GEMM reads the weighted activation directly).
namespace g1 {
constexpr int IPT = BN / 2;  // intermediate indices per tile (128)
// Q row q -> row of W13[e]
__device__ __forceinline__ int w13_row(int q, int nt, int I) {
  const int wn = q / WTN;         // wave column
  const int s = (q % WTN) >> 5;   // 0 gate, 1 up
  const int i = nt * IPT + wn * 32 + (q & 31);
  return s * I + i;
}
}  // namespace g1

// An operand in memory: bf16 elements (scales == nullptr) or E4M3 codes with
// per-(row, 32-block) E8M0 scales.
struct Operand {
  const void* data;
  const uint8_t* scales;
};

// Row length in 16-bit units (a bf16 element, or two E4M3 codes): the k loop
// runs over slabs of 64 such units in both cases.
template <bool FP8>
__device__ __forceinline__ int row_units(int K) { return FP8 ? K / 2 : K; }

template <bool FP8, bool W4 = false, bool F32S = false>
__global__ __launch_bounds__(kThreads) void gemm1_swiglu_kernel(GemmProblem p, Operand X, Operand W,
                                                                uint16_t* __restrict__ h13,
                                                                uint16_t* __restrict__ act) {
  __shared__ float s_w[BM];
  const int E = int(p.E), H = int(p.H), I = int(p.I), k = int(p.k);
  MOE_ROW_SCHED
  const int NT = (2 * I) / BN;
  const int KU = row_units<FP8>(H);
  const int KW = W4 ? KU / 2 : KU;  // weight row in 16-bit units
  const int64_t total = int64_t(s_pref[E]) * NT;
  KLoaderD<FP8> lp;
  typename std::conditional<W4, KMajorLoader4, KLoaderD<FP8>>::type lq;
  auto setup = [&](int64_t t, TileState& st) {
    const RowTile rt = decode_row_tile(t, NT, s_pref, E, p.counts, p.offsets);
    st.rt = rt;
    if constexpr (FP8) {
      lp.set_base(static_cast<const uint16_t*>(X.data), p.T * KU, X.scales, p.T * (H / 32));
      lq.set_base(static_cast<const uint16_t*>(W.data) + int64_t(rt.e) * 2 * I * KW, 2 * I * KW,
                  W.scales + int64_t(rt.e) * 2 * I * (H / 32), 2 * I * (H / 32));
    } else {
      lp.set_base(static_cast<const uint16_t*>(X.data), p.T * KU);
      lq.set_base(static_cast<const uint16_t*>(W.data) + int64_t(rt.e) * 2 * I * KU, 2 * I * KU);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = KMajorLoader::row_of_thread(i);
      const int mc = m < rt.rows ? m : rt.rows - 1;  // past-the-end rows reuse a real row
      lp.set_row(i, int64_t(p.src_of[rt.row0 + mc] / k) * KU);
      if constexpr (!W4) lq.set_row(i, int64_t(g1::w13_row(m, rt.nt, I)) * KU);
    }
    if constexpr (W4) {
#pragma unroll
      for (int i = 0; i < KMajorLoader4::kRows; ++i)
        lq.set_row(i, int64_t(g1::w13_row(KMajorLoader4::row_of_thread(i), rt.nt, I)) * KW);
    }
    // routing weight of tile row t: loaded now, used after the k loop
    st.w = threadIdx.x < BM ? p.wrow[rt.row0 + min(int(threadIdx.x), rt.rows - 1)] : 0.f;
  };
  auto epi = [&](const TileState& st, const Acc& acc) {
    const RowTile& rt = st.rt;
    if (threadIdx.x < BM) s_w[threadIdx.x] = st.w;
    // half h holds g and u of intermediate indices nt*128 + h*64 + [0, 64):
    // staged column (i/32)*64 + i%32 is g, +32 is u.
    const int io = (threadIdx.x & 15) * 4;  // 4 intermediate indices per thread
    const int gc = (io >> 5) * 64 + (io & 31);
    for (int h = 0; h < 2; ++h) {
      stage_half(acc, h);
      __syncthreads();
      const int i = rt.nt * g1::IPT + h * 64 + io;
      for (int m = threadIdx.x >> 4; m < rt.rows; m += kRowPass) {
        const int64_t r = rt.row0 + m;
        const float w = s_w[m];
        const f32x4 gv = *reinterpret_cast<const f32x4*>(frow(m) + gc);
        const f32x4 uv = *reinterpret_cast<const f32x4*>(frow(m) + gc + 32);
        float av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) av[q] = w * (gv[q] * sigmoidf_fast(gv[q]) * uv[q]);
        if (h13) {  // read again only by the backward's dH epilogue
          store4_bf16_nt(h13 + r * 2 * I + i, gv[0], gv[1], gv[2], gv[3]);
          store4_bf16_nt(h13 + r * 2 * I + I + i, uv[0], uv[1], uv[2], uv[3]);
        }
        store4_bf16(act + r * I + i, av[0], av[1], av[2], av[3]);
      }
      __syncthreads();
    }
  };
  row_tile_walk<FP8, false, true, F32S>(total, KU / 64, lp, lq, setup, epi);
}

// ================================================================== forward GEMM2
// O[r][h] = (w a)[r] . W2[e][h],  K = I.
template <bool FP8, bool W4 = false, bool F32S = false>
__global__ __launch_bounds__(kThreads) void gemm2_kernel(GemmProblem p, Operand A, Operand W,
                                                         uint16_t* __restrict__ out) {
  const int E = int(p.E), H = int(p.H), I = int(p.I);
  MOE_ROW_SCHED
  const int NT = H / BN;
  const int KU = row_units<FP8>(I);
  const int KW = W4 ? KU / 2 : KU;  // weight row in 16-bit units
  const int64_t total = int64_t(s_pref[E]) * NT;
  KLoaderD<FP8> lp;
  typename std::conditional<W4, KMajorLoader4, KLoaderD<FP8>>::type lq;
  auto setup = [&](int64_t t, TileState& st) {
    const RowTile rt = decode_row_tile(t, NT, s_pref, E, p.counts, p.offsets);
    st.rt = rt;
    if constexpr (FP8) {
      lp.set_base(static_cast<const uint16_t*>(A.data) + rt.row0 * KU, int64_t(rt.rows) * KU,
                  A.scales + rt.row0 * (I / 32), int64_t(rt.rows) * (I / 32));
      lq.set_base(static_cast<const uint16_t*>(W.data) + (int64_t(rt.e) * H + int64_t(rt.nt) * BN) * KW,
                  int64_t(BN) * KW, W.scales + (int64_t(rt.e) * H + int64_t(rt.nt) * BN) * (I / 32),
                  int64_t(BN) * (I / 32));
    } else {
      lp.set_base(static_cast<const uint16_t*>(A.data) + rt.row0 * KU, int64_t(rt.rows) * KU);
      lq.set_base(static_cast<const uint16_t*>(W.data) + (int64_t(rt.e) * H + int64_t(rt.nt) * BN) * KU,
                  int64_t(BN) * KU);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = KMajorLoader::row_of_thread(i);
      lp.set_row(i, int64_t(m < rt.rows ? m : rt.rows - 1) * KU);
      if constexpr (!W4) lq.set_row(i, int64_t(m) * KU);
    }
    if constexpr (W4) {
#pragma unroll
      for (int i = 0; i < KMajorLoader4::kRows; ++i) lq.set_row(i, int64_t(KMajorLoader4::row_of_thread(i)) * KW);
    }
  };
  // k == 1: each row is its token's whole result, written to the token row
  const int32_t* rowmap = p.k == 1 ? p.src_of : nullptr;
  __shared__ int32_t s_map[BM];
  auto copy = [&](const TileState& st) {
    copy_image(out, H, st.rt.row0, int64_t(st.rt.nt) * BN, st.rt.rows, BN, rowmap, s_map);
  };
  auto epi = [&](const TileState& st, const Acc& acc) {
    stage_image(acc, st.rt.row0, st.rt.rows, rowmap, s_map);
    copy(st);
  };
  row_tile_walk<FP8, false, true, F32S>(total, KU / 64, lp, lq, setup, epi);
}

// ------------------------------------------------------------------ row functions

// A row function maps k (a row of an expert segment) to a memory row:
// index(k) directly, or in two steps, load(k) (which may read an index
// array) and row(raw), so that a loader can issue the loads early and use
// them later.
struct DirectRows {  // memory row k of a row-major tensor
  using Raw = int32_t;
  int32_t ld;            // elements between rows
  int32_t nrows;         // k-rows past this contribute zeros (nrows >= 1)
  __device__ __forceinline__ int32_t index(int k) const { return k < nrows ? k : nrows - 1; }
  __device__ __forceinline__ bool valid(int k) const { return k < nrows; }
  __device__ __forceinline__ Raw load(int k) const { return index(k); }
  __device__ __forceinline__ int32_t row(Raw r) const { return r; }
};

// floor(2^32 / k) (2^32 - 1 for k = 1): with it, n / k for 0 <= n < 2^31 is
// q = mulhi(n, m) or q + 1. m is short of 2^32 / k by less than 1, so n m / 2^32
// is short of n / k by less than n / 2^32 < 1/2 and q is the quotient or one less;
// one comparison of the remainder fixes it.
__host__ __device__ inline uint32_t div_magic(uint32_t k) {
  return k == 1 ? 0xFFFFFFFFu : uint32_t((uint64_t(1) << 32) / k);
}
__device__ __forceinline__ uint32_t div_by(uint32_t n, uint32_t k, uint32_t m) {
  const uint32_t q = uint32_t((uint64_t(n) * m) >> 32);
  return q + (n - q * k >= k ? 1u : 0u);
}

struct TokenRows {  // k-th row of an expert segment -> its token's row
  using Raw = int32_t;
  int32_t ld;            // elements between token rows
  const int32_t* src;    // src_of + segment start
  int rows;              // segment length (>= 1)
  int kk;                // experts per token
  uint32_t kmagic;       // div_magic(kk)
  __device__ __forceinline__ bool valid(int k) const { return k < rows; }
  __device__ __forceinline__ Raw load(int k) const { return src[k < rows ? k : rows - 1]; }
  // a pair index (>= 0) -> its token
  __device__ __forceinline__ int32_t row(Raw r) const { return int32_t(div_by(uint32_t(r), uint32_t(kk), kmagic)); }
};

// ================================================================== backward dH
// dA_u[r][i] = dY[tok(r)] . W2[e][:, i]  (K = H; W2 read mn-major), then per
// element, with g, u from the saved [g | u]:
//   a = silu(g) u,  dw partial += dA_u a,  dA = w dA_u,
//   dg = dA u sig(g) (1 + g (1 - sig(g))),  du = dA silu(g).
// dwpart[r][2*nt + h] holds the partial sum of dA_u * a over column half h.
int dh_num_parts(int64_t I) { return int((I + BN - 1) / BN) * 2; }

// In the FP8 variant W2 arrives transposed, [E, I, H] (k-major rows i).

// The dH epilogue of one row tile: dA_u (the accumulators) with the saved
// [g | u] rows gives dh13 = [dg | du] and the routing-weight partials. A
// thread handles 8 rows in batches of kDhRows (fewer rows per batch leave
// more registers to the k loop); the [g | u] loads of the next batch go out
// before the current batch's math, so their latency hides behind it.
template <int kDhRows>
__device__ __forceinline__ void dh_epilogue(const TileState& st, const Acc& acc, int I, int nparts, float* s_w,
                                            const uint16_t* __restrict__ h13, uint16_t* __restrict__ dh13,
                                            float* __restrict__ dwpart) {
  constexpr int kDhBatches = 8 / kDhRows;
  const RowTile& rt = st.rt;
  const int ncols = min(BN, I - rt.nt * BN);
  if (threadIdx.x < BM) s_w[threadIdx.x] = st.w;
  // half h holds dA_u of intermediate indices nt*256 + h*128 + [0, 128).
  // Thread t works on 8 of them (c) for tile rows t/16 + 32*j, j < 8.
  const int c = (threadIdx.x & 15) * 8;
  for (int h = 0; h < 2; ++h) {
    const bool col_ok = h * 128 + c < ncols;
    const int i = rt.nt * BN + h * 128 + (col_ok ? c : 0);
    // [g | u] is read once: streaming (nontemporal) loads keep it out of the caches
    auto request = [&](int bt, u32x4 (&gq)[kDhRows], u32x4 (&uq)[kDhRows]) {
#pragma unroll
      for (int j = 0; j < kDhRows; ++j) {
        const int m = min((int(threadIdx.x) >> 4) + kRowPass * (kDhRows * bt + j), rt.rows - 1);
        const uint16_t* src = h13 + (rt.row0 + m) * 2 * I + i;
        gq[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        uq[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + I));
      }
    };
    stage_half(acc, h);
    u32x4 gn[kDhRows], un[kDhRows];
    request(0, gn, un);
    __syncthreads();
    for (int bt = 0; bt < kDhBatches; ++bt) {
      u32x4 gq[kDhRows], uq[kDhRows];
#pragma unroll
      for (int j = 0; j < kDhRows; ++j) {
        gq[j] = gn[j];
        uq[j] = un[j];
      }
      if (bt + 1 < kDhBatches) request(bt + 1, gn, un);
#pragma unroll
      for (int j = 0; j < kDhRows; ++j) {
        const int m = (threadIdx.x >> 4) + kRowPass * (kDhRows * bt + j);
        const bool row_ok = m < rt.rows;
        float dws = 0.f;
        if (row_ok && col_ok) {
          const int64_t r = rt.row0 + m;
          const float w = s_w[m];
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(frow(m) + c);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(frow(m) + c + 4);
          u32x4 dgq, duq;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float dgp[2], dup[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const float gv = hh ? bf16_hi(gq[j][q]) : bf16_lo(gq[j][q]);
              const float uv = hh ? bf16_hi(uq[j][q]) : bf16_lo(uq[j][q]);
              const int e8 = 2 * q + hh;
              const float dau = e8 < 4 ? d0[e8] : d1[e8 - 4];
              const float sg_ = sigmoidf_fast(gv);
              const float sl = gv * sg_;  // silu(g)
              dws += dau * sl * uv;
              const float da = w * dau;
              dgp[hh] = da * uv * sg_ * (1.f + gv * (1.f - sg_));
              dup[hh] = da * sl;
            }
            dgq[q] = pack_bf16x2(dgp[0], dgp[1]);
            duq[q] = pack_bf16x2(dup[0], dup[1]);
          }
          __builtin_nontemporal_store(dgq, reinterpret_cast<u32x4*>(dh13 + r * 2 * I + i));
          __builtin_nontemporal_store(duq, reinterpret_cast<u32x4*>(dh13 + r * 2 * I + I + i));
        }
        // sum over the 16 threads of this row (lanes 16g .. 16g+15)
        dws += __shfl_xor(dws, 8);
        dws += __shfl_xor(dws, 4);
        dws += __shfl_xor(dws, 2);
        dws += __shfl_xor(dws, 1);
        if (row_ok && (threadIdx.x & 15) == 0) dwpart[(rt.row0 + m) * nparts + 2 * rt.nt + h] = dws;
      }
    }
    __syncthreads();
  }
}

// The FP8 dH (W2 arrives as transposed codes), both operands straight into
// LDS; its own tile loop, no prefetch across tiles.
// Its epilogue is the one of dh_epilogue with four rows per batch, written
// inline: called as that function the FP8 kernels spill 34-35 registers.
template <bool F32S, bool FP8 = true>  // FP8 stays a template parameter for row_units<FP8>
__device__ __forceinline__ void dh_fp8_tiles(const GemmProblem& p, const Operand& DY, const Operand& W,
                                             const uint16_t* __restrict__ h13, uint16_t* __restrict__ dh13,
                                             float* __restrict__ dwpart) {
  __shared__ float s_w[BM];
  const int E = int(p.E), H = int(p.H), I = int(p.I), k = int(p.k);
  MOE_ROW_SCHED
  const int NT = (I + BN - 1) / BN;  // the last n-tile may hold 128 columns
  const int nparts = 2 * NT;
  const int64_t total = int64_t(s_pref[E]) * NT;
  for (int64_t t = first_tile(); t < total; t += gridDim.x) {
    const RowTile rt = decode_row_tile(t, NT, s_pref, E, p.counts, p.offsets);
    const int KU = row_units<FP8>(H);
    KMajorLoader8D lp;
    lp.set_base(static_cast<const uint16_t*>(DY.data), p.T * KU, DY.scales, p.T * (H / 32));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = KMajorLoader::row_of_thread(i);
      const int mc = m < rt.rows ? m : rt.rows - 1;
      lp.set_row(i, int64_t(p.src_of[rt.row0 + mc] / k) * KU);
    }
    const int ncols = min(BN, I - rt.nt * BN);
    const float w_row = threadIdx.x < BM ? p.wrow[rt.row0 + min(int(threadIdx.x), rt.rows - 1)] : 0.f;
    Acc acc;
    acc.zero();
    {
      // rows i of W2^T past the (partial) last n-tile reuse row I-1; their
      // columns are never stored
      KMajorLoader8D lq;
      lq.set_base(static_cast<const uint16_t*>(W.data) + (int64_t(rt.e) * I + int64_t(rt.nt) * BN) * KU,
                  int64_t(ncols) * KU, W.scales + (int64_t(rt.e) * I + int64_t(rt.nt) * BN) * (H / 32),
                  int64_t(ncols) * (H / 32));
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        lq.set_row(i, int64_t(min(KMajorLoader::row_of_thread(i), ncols - 1)) * KU);
      mainloop_fp8<F32S>(lp, lq, KU / 64, acc, wave_m() * WTM < rt.rows);
    }
    if (threadIdx.x < BM) s_w[threadIdx.x] = w_row;
    // half h holds dA_u of intermediate indices nt*256 + h*128 + [0, 128).
    // Thread t works on 8 of them (c) for tile rows t/16 + 32*j, j < 8, in
    // two batches of four rows; each batch's [g | u] pieces are requested
    // together (the first batch's before the staging barrier).
    const int c = (threadIdx.x & 15) * 8;
    for (int h = 0; h < 2; ++h) {
      const bool col_ok = h * 128 + c < ncols;
      const int i = rt.nt * BN + h * 128 + (col_ok ? c : 0);
      stage_half(acc, h);
      for (int bt = 0; bt < 2; ++bt) {
        u32x4 gq[4], uq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = min((int(threadIdx.x) >> 4) + kRowPass * (4 * bt + j), rt.rows - 1);
          const uint16_t* src = h13 + (rt.row0 + m) * 2 * I + i;
          gq[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
          uq[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + I));
        }
        if (bt == 0) __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = (threadIdx.x >> 4) + kRowPass * (4 * bt + j);
          const bool row_ok = m < rt.rows;
          float dws = 0.f;
          if (row_ok && col_ok) {
            const int64_t r = rt.row0 + m;
            const float w = s_w[m];
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(frow(m) + c);
            const f32x4 d1 = *reinterpret_cast<const f32x4*>(frow(m) + c + 4);
            u32x4 dgq, duq;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float dgp[2], dup[2];
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                const float gv = hh ? bf16_hi(gq[j][q]) : bf16_lo(gq[j][q]);
                const float uv = hh ? bf16_hi(uq[j][q]) : bf16_lo(uq[j][q]);
                const int e8 = 2 * q + hh;
                const float dau = e8 < 4 ? d0[e8] : d1[e8 - 4];
                const float sg_ = sigmoidf_fast(gv);
                const float sl = gv * sg_;  // silu(g)
                dws += dau * sl * uv;
                const float da = w * dau;
                dgp[hh] = da * uv * sg_ * (1.f + gv * (1.f - sg_));
                dup[hh] = da * sl;
              }
              dgq[q] = pack_bf16x2(dgp[0], dgp[1]);
              duq[q] = pack_bf16x2(dup[0], dup[1]);
            }
            __builtin_nontemporal_store(dgq, reinterpret_cast<u32x4*>(dh13 + r * 2 * I + i));
            __builtin_nontemporal_store(duq, reinterpret_cast<u32x4*>(dh13 + r * 2 * I + I + i));
          }
          // sum over the 16 threads of this row (lanes 16g .. 16g+15)
          dws += __shfl_xor(dws, 8);
          dws += __shfl_xor(dws, 4);
          dws += __shfl_xor(dws, 2);
          dws += __shfl_xor(dws, 1);
          if (row_ok && (threadIdx.x & 15) == 0) dwpart[(rt.row0 + m) * nparts + 2 * rt.nt + h] = dws;
        }
      }
      __syncthreads();
    }
  }
}

// The bf16 dH: own tile loop, the loaders scoped to the tile and no prefetch
// across tiles (the epilogue needs the registers); the gathered dY rows and
// the mn-major W2 load straight into LDS.
__device__ __forceinline__ void dh_bf16_tiles(const GemmProblem& p, const Operand& DY, const Operand& W,
                                              const uint16_t* __restrict__ h13, uint16_t* __restrict__ dh13,
                                              float* __restrict__ dwpart) {
  __shared__ float s_w[BM];
  const int E = int(p.E), H = int(p.H), I = int(p.I), k = int(p.k);
  MOE_ROW_SCHED
  const int NT = (I + BN - 1) / BN;  // the last n-tile may hold 128 columns
  const int nparts = 2 * NT;
  const int64_t total = int64_t(s_pref[E]) * NT;
  for (int64_t t = first_tile(); t < total; t += gridDim.x) {
    const RowTile rt = decode_row_tile(t, NT, s_pref, E, p.counts, p.offsets);
    KMajorLoaderD lp;
    lp.set_base(static_cast<const uint16_t*>(DY.data), p.T * H);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = KMajorLoader::row_of_thread(i);
      const int mc = m < rt.rows ? m : rt.rows - 1;
      lp.set_row(i, int64_t(p.src_of[rt.row0 + mc] / k) * H);
    }
    const int ncols = min(BN, I - rt.nt * BN);
    MNMajorLoaderD<DirectRows> lq;
    lq.set_base(static_cast<const uint16_t*>(W.data) + int64_t(rt.e) * H * I + int64_t(rt.nt) * BN,
                int64_t(H) * I - int64_t(rt.nt) * BN);
    lq.fn.ld = I;
    lq.fn.nrows = H;
    lq.nchunks = ncols / 8;
    lq.prime(0);
    TileState st;
    st.rt = rt;
    st.w = threadIdx.x < BM ? p.wrow[rt.row0 + min(int(threadIdx.x), rt.rows - 1)] : 0.f;
    Acc acc;
    acc.zero();
    mainloop_direct<false, true>(lp, lq, H / 64, acc, wave_m() * WTM < rt.rows);
    dh_epilogue<1>(st, acc, I, nparts, s_w, h13, dh13, dwpart);
  }
}

template <bool FP8, bool F32S = false>
__global__ __launch_bounds__(kThreads) void gemm_dh_kernel(GemmProblem p, Operand DY, Operand W,
                                                           const uint16_t* __restrict__ h13,
                                                           uint16_t* __restrict__ dh13,
                                                           float* __restrict__ dwpart) {
  if constexpr (FP8)
    dh_fp8_tiles<F32S>(p, DY, W, h13, dh13, dwpart);
  else
    dh_bf16_tiles(p, DY, W, h13, dh13, dwpart);
}

// ================================================================== backward dX
// dXr[r][h] = [dg | du][r] . W13[e][:, h]  (K = 2I; W13 read mn-major).
// In the FP8 variant W13 arrives transposed, [E, H, 2I] (k-major rows h).
template <bool FP8, bool F32S = false>
__global__ __launch_bounds__(kThreads) void gemm_dx_kernel(GemmProblem p, Operand DH, Operand W,
                                                           uint16_t* __restrict__ out) {
  const int E = int(p.E), H = int(p.H), I = int(p.I);
  MOE_ROW_SCHED
  const int NT = H / BN;
  const int KU = row_units<FP8>(2 * I);
  const int64_t total = int64_t(s_pref[E]) * NT;
  KLoaderD<FP8> lp;
  typename std::conditional<FP8, KMajorLoader8, MNMajorLoaderD<DirectRows>>::type lq;
  auto setup = [&](int64_t t, TileState& st) {
    const RowTile rt = decode_row_tile(t, NT, s_pref, E, p.counts, p.offsets);
    st.rt = rt;
    if constexpr (FP8)
      lp.set_base(static_cast<const uint16_t*>(DH.data) + rt.row0 * KU, int64_t(rt.rows) * KU,
                  DH.scales + rt.row0 * (2 * I / 32), int64_t(rt.rows) * (2 * I / 32));
    else
      lp.set_base(static_cast<const uint16_t*>(DH.data) + rt.row0 * KU, int64_t(rt.rows) * KU);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = KMajorLoader::row_of_thread(i);
      lp.set_row(i, int64_t(m < rt.rows ? m : rt.rows - 1) * KU);
    }
    if constexpr (FP8) {
      lq.set_base(static_cast<const uint16_t*>(W.data) + (int64_t(rt.e) * H + int64_t(rt.nt) * BN) * KU,
                  int64_t(BN) * KU, W.scales + (int64_t(rt.e) * H + int64_t(rt.nt) * BN) * (2 * I / 32),
                  int64_t(BN) * (2 * I / 32));
#pragma unroll
      for (int i = 0; i < kPer; ++i) lq.set_row(i, int64_t(KMajorLoader::row_of_thread(i)) * KU);
    } else {
      lq.set_base(static_cast<const uint16_t*>(W.data) + int64_t(rt.e) * 2 * I * H + int64_t(rt.nt) * BN,
                  int64_t(2 * I) * H - int64_t(rt.nt) * BN);
      lq.fn.ld = H;
      lq.fn.nrows = 2 * I;
      lq.prime(0);
    }
  };
  // k == 1: each row is its token's whole result, written to the token row
  const int32_t* rowmap = p.k == 1 ? p.src_of : nullptr;
  __shared__ int32_t s_map[BM];
  auto copy = [&](const TileState& st) {
    copy_image(out, H, st.rt.row0, int64_t(st.rt.nt) * BN, st.rt.rows, BN, rowmap, s_map);
  };
  auto epi = [&](const TileState& st, const Acc& acc) {
    stage_image(acc, st.rt.row0, st.rt.rows, rowmap, s_map);
    copy(st);
  };
  row_tile_walk<FP8, !FP8, true, F32S>(total, KU / 64, lp, lq, setup, epi);
}

// ================================================================== weight gradients
// dW13[e][c][h] = sum_{r in seg e} dH13[r][c] x[tok(r)][h]
// dW2[e][h][i]  = sum_{r in seg e} dY[tok(r)][h] (w a)[r][i]
// The reduction runs over the expert's rows (K = rows_e, the ragged last
// slab zero-filled); an expert without rows produces an exact-zero tile.
// ------------------------------------------------------------------ dW schedule
// A weight-gradient tile's k loop runs over its expert's rows. With balanced
// routing the tiles cost the same and the static XCD-aware walk of the other
// GEMMs is best (every XCD works on a contiguous run of tiles, so concurrent
// tiles share their expert's rows in L2). Under skewed routing (largest
// expert above twice the mean) tiles differ in cost by an order of
// magnitude; then experts are ranked by descending row count (ties by id)
// and workgroups take tiles from a queue (a word in device memory, zero at
// launch), heaviest expert first, so short tiles fill in behind long ones.
// Thread 0 takes its next ticket as soon as a tile starts, so the atomic's
// round trip overlaps the tile's own first loads. Tile indices are 32-bit
// and pass through readfirstlane, so the tile's buffer resources stay in
// scalar registers.

// Fills s_order (experts by descending count) and returns whether the
// routing is skewed. Same result in every workgroup.
__device__ bool dw_expert_order(const int32_t* counts, int E, int32_t* s_cnt, int32_t* s_order, int32_t* s_flag) {
  // s_cnt padded to a multiple of 4 with -1, which ranks below every count
  const int E4 = (E + 3) >> 2;
  for (int e = threadIdx.x; e < 4 * E4; e += kThreads) s_cnt[e] = e < E ? counts[e] : -1;
  __syncthreads();
  const i32x4* c4 = reinterpret_cast<const i32x4*>(s_cnt);
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const int c = s_cnt[e];
    int r = 0;
    for (int q = 0; q < E4; ++q) {
      const i32x4 v = c4[q];
#pragma unroll
      for (int u = 0; u < 4; ++u) r += (v[u] > c || (v[u] == c && 4 * q + u < e)) ? 1 : 0;
    }
    s_order[r] = e;
  }
  if (threadIdx.x < 64) {  // wave 0: the total and the largest count
    int64_t sum = 0;
    int mx = 0;
    for (int j = threadIdx.x; j < E; j += 64) {
      sum += s_cnt[j];
      mx = max(mx, s_cnt[j]);
    }
    for (int o = 32; o > 0; o >>= 1) {
      sum += __shfl_xor(sum, o);
      mx = max(mx, __shfl_xor(mx, o));
    }
    if (threadIdx.x == 0) *s_flag = (int64_t(mx) * E > 2 * sum) ? 1 : 0;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_flag) != 0;
}

// Split-K for the hottest experts under skewed routing. A tile's k loop
// runs over its expert's rows, so under skew the tiles of the hottest
// experts can outlast a workgroup's share of all the work. With `avg` the
// rows one workgroup would run if all tiles were spread over 256 of them (a
// fixed nominal count, so that the plan, and with it the fp32 summation
// order, does not depend on the grid), an expert with rows >= 1024 and
// 4 * rows > 3 * avg is cut into S = min(kMaxSplit, ceil(2 * rows / avg))
// row ranges of `chunk` rows (a multiple of 128), walking the experts in
// the queue order above while the fp32 partial-tile budget lasts
// (kSplitSlots tiles, at most kMaxSplitExperts experts). A split item
// writes its fp32 partial tile to the workspace; a second kernel adds the S
// partials of each split tile in split order and stores the tile, so the
// result does not depend on the order the items ran in. Workgroup 0 writes
// the plan for that kernel.
constexpr int kMaxSplit = 4;
constexpr int kMaxSplitExperts = 16;
constexpr int kSplitSlots = 320;  // fp32 partial tiles of 256 x 256
constexpr int kSplitMinRows = 1024;
constexpr int kNominalWGs = 256;

struct DwPlan {
  int nsplit;                      // split experts: queue ranks 0 .. nsplit-1
  int split_last;                  // 1: their items after the unsplit ones (tail split)
  int e[kMaxSplitExperts];         // their expert ids
  int S[kMaxSplitExperts];         // their split counts
  int chunk[kMaxSplitExperts];     // rows per split
  int slot0[kMaxSplitExperts];     // first partial slot (tile t, split s: slot0 + t * S + s)
  int item0[kMaxSplitExperts + 1]; // prefix of the split experts' items
};
static_assert(sizeof(DwPlan) <= sizeof(int32_t) * kSplitWords, "the plan fits its workspace words");
static_assert(kSplitFloats == int64_t(kSplitSlots) * BM * BN, "the partial buffer holds kSplitSlots tiles");

// One work item of a weight-gradient GEMM: tile `local` of expert e over the
// expert's rows [k0, k0 + klen) (S == 1: all of them).
struct DwItem {
  int e, local;
  int s, S;
  int k0, klen, chunk;
  int slot;
};

// the split plan (thread 0; every workgroup computes the same)
__device__ void dw_plan(const int32_t* s_cnt, const int32_t* s_order, int E, int per_expert, DwPlan* plan) {
  if (threadIdx.x != 0) return;
  int64_t sum = 0;
  for (int j = 0; j < E; ++j) sum += s_cnt[j];
  const int64_t avg = max(int64_t(1), int64_t(per_expert) * sum / kNominalWGs);
  int used = 0, n = 0;
  plan->item0[0] = 0;
  while (n < kMaxSplitExperts && n < E) {
    const int e = s_order[n];
    const int rows = s_cnt[e];
    if (rows < kSplitMinRows || 4 * int64_t(rows) <= 3 * avg) break;
    const int want = int(min(int64_t(kMaxSplit), (2 * int64_t(rows) + avg - 1) / avg));
    const int chunk = ((rows + want - 1) / want + 127) / 128 * 128;
    const int S = (rows + chunk - 1) / chunk;
    if (S < 2 || used + per_expert * S > kSplitSlots) break;
    plan->e[n] = e;
    plan->S[n] = S;
    plan->chunk[n] = chunk;
    plan->slot0[n] = used;
    plan->item0[n + 1] = plan->item0[n] + per_expert * S;
    used += per_expert * S;
    ++n;
  }
  plan->nsplit = n;
  plan->split_last = 0;
}

// Split for the last round under balanced routing. The n = E * per_expert
// tiles cost about the same, so the walk takes ceil(n / G) tile times on G
// workgroups, with the last round only x / G full (x = n mod G). Cutting x
// tiles into two row halves and running the whole tiles first (longest
// first) finishes in floor(n / G) + 1/2 tile times when x <= G / 2. The
// tiles of the ceil(x / per_expert) heaviest experts are cut (each half a
// multiple of 128 rows, at least kSplitMinRows); only when floor(n / G) is 1
// to 3 (a saving of an eighth to a quarter) and every cut expert has the
// rows. G is the nominal 256, as in dw_plan. nsplit = 0: no split.
__device__ void dw_tail_plan(const int32_t* s_cnt, const int32_t* s_order, int E, int per_expert, DwPlan* plan) {
  if (threadIdx.x != 0) return;
  plan->nsplit = 0;
  plan->split_last = 1;
  plan->item0[0] = 0;
  const int n = E * per_expert;
  const int r = n / kNominalWGs, x = n - r * kNominalWGs;
  if (r < 1 || r > 3 || x == 0 || 2 * x > kNominalWGs) return;
  const int nexp = (x + per_expert - 1) / per_expert;
  if (nexp > kMaxSplitExperts || nexp > E || nexp * per_expert * 2 > kSplitSlots) return;
  for (int j = 0; j < nexp; ++j) {
    const int e = s_order[j];
    const int rows = s_cnt[e];
    const int chunk = ((rows + 1) / 2 + 127) / 128 * 128;
    if (chunk < kSplitMinRows || (rows + chunk - 1) / chunk != 2) return;
    plan->e[j] = e;
    plan->S[j] = 2;
    plan->chunk[j] = chunk;
    plan->slot0[j] = j * per_expert * 2;
    plan->item0[j + 1] = (j + 1) * per_expert * 2;
  }
  plan->nsplit = nexp;
}

// Runs body(item) over every work item of a weight-gradient GEMM with
// per_expert tiles per expert. Balanced routing: the static walk over
// (expert, tile), unless dw_tail_plan cuts the last round's tiles. Skewed:
// workgroups take items from one queue (queue[0]), the split experts' items
// first, then the other experts heaviest first. Tail split: the whole tiles
// and then the halves are dealt out in eight contiguous shares, XCD x
// (= blockIdx % 8) taking items from its own share through queue[x], so
// that the tiles one XCD runs at the same time share expert rows in its L2
// (the static walk's locality, which a single queue loses); a workgroup
// whose share is done takes items from the next XCDs' shares. s_flag and
// s_next are distinct LDS words. Workgroup 0 writes the plan (nsplit = 0:
// no split tiles) to plan_out.
template <class Body>
__device__ __forceinline__ void dw_for_each_item(const int32_t* counts, int E, int per_expert, int32_t* queue,
                                                 int32_t* plan_out, int32_t* s_cnt, int32_t* s_order,
                                                 int32_t* s_flag, int32_t* s_next, DwPlan* plan, Body&& body) {
  const bool skewed = dw_expert_order(counts, E, s_cnt, s_order, s_flag);
  if (skewed)
    dw_plan(s_cnt, s_order, E, per_expert, plan);
  else
    dw_tail_plan(s_cnt, s_order, E, per_expert, plan);
  __syncthreads();
  const int nsplit = __builtin_amdgcn_readfirstlane(plan->nsplit);
  if (blockIdx.x == 0) {
    const int32_t* w = reinterpret_cast<const int32_t*>(plan);
    for (int i = threadIdx.x; i < int(sizeof(DwPlan) / sizeof(int32_t)); i += kThreads) plan_out[i] = w[i];
  }
  const int split_items = __builtin_amdgcn_readfirstlane(plan->item0[nsplit]);
  const int whole_items = (E - nsplit) * per_expert;
  // split item us (us < split_items) or whole item v
  auto run = [&](bool split, int idx) {
    DwItem it;
    if (split) {
      int r = 0;
      while (r + 1 < nsplit && plan->item0[r + 1] <= idx) ++r;
      r = __builtin_amdgcn_readfirstlane(r);
      const int S = __builtin_amdgcn_readfirstlane(plan->S[r]);
      const int within = idx - __builtin_amdgcn_readfirstlane(plan->item0[r]);
      it.e = __builtin_amdgcn_readfirstlane(plan->e[r]);
      it.local = within / S;
      it.s = within % S;
      it.S = S;
      it.chunk = __builtin_amdgcn_readfirstlane(plan->chunk[r]);
      it.k0 = it.s * it.chunk;
      it.klen = min(it.chunk, __builtin_amdgcn_readfirstlane(counts[it.e]) - it.k0);
      it.slot = __builtin_amdgcn_readfirstlane(plan->slot0[r]) + it.local * S + it.s;
    } else {
      it.e = __builtin_amdgcn_readfirstlane(s_order[nsplit + idx / per_expert]);
      it.local = idx % per_expert;
      it.s = 0;
      it.S = 1;
      it.k0 = 0;
      it.klen = __builtin_amdgcn_readfirstlane(counts[it.e]);
      it.chunk = it.klen;
      it.slot = 0;
    }
    body(it);
  };
  if (skewed) {
    const int total = split_items + whole_items;
    int32_t ticket = 0;  // thread 0 only
    if (threadIdx.x == 0) ticket = atomicAdd(queue, 1);
    for (;;) {
      if (threadIdx.x == 0) *s_next = ticket;
      __syncthreads();
      const int u = __builtin_amdgcn_readfirstlane(*s_next);
      __syncthreads();
      if (u >= total) break;
      if (threadIdx.x == 0) ticket = atomicAdd(queue, 1);
      run(u < split_items, u < split_items ? u : u - split_items);
    }
  } else if (nsplit > 0) {
    // share x: whole items [W x / 8, W (x+1) / 8), then split items [S x / 8, S (x+1) / 8)
    int x = int(blockIdx.x & 7), tries = 0;
    int32_t ticket = 0;  // thread 0 only
    if (threadIdx.x == 0) ticket = atomicAdd(queue + x, 1);
    for (;;) {
      if (threadIdx.x == 0) *s_next = ticket;
      __syncthreads();
      const int j = __builtin_amdgcn_readfirstlane(*s_next);
      __syncthreads();
      const int w0 = whole_items * x / 8, w1 = whole_items * (x + 1) / 8;
      const int s0 = split_items * x / 8, s1 = split_items * (x + 1) / 8;
      if (j >= (w1 - w0) + (s1 - s0)) {  // share x is done: the next one
        if (++tries == 8) break;
        x = (x + 1) & 7;
        if (threadIdx.x == 0) ticket = atomicAdd(queue + x, 1);
        continue;
      }
      if (threadIdx.x == 0) ticket = atomicAdd(queue + x, 1);
      run(j >= w1 - w0, j < w1 - w0 ? w0 + j : s0 + j - (w1 - w0));
    }
  } else {
    for (int t = int(first_tile()); t < E * per_expert; t += gridDim.x) run(false, t);
  }
}

// Stores a weight-gradient tile (rows [row0, row0 + 256), columns
// [col0, col0 + cols) of the row-major [*, ld] output) when the item covers
// all of the expert's rows, else writes its fp32 partial, a row-major
// 256 x 256 tile, to its slot.
__device__ __forceinline__ void dw_store(const Acc& acc, const DwItem& it, uint16_t* out, int64_t ld,
                                         int64_t row0, int64_t col0, int cols, float* partial) {
  if (it.S == 1) {
    store_tile(acc, out, ld, row0, col0, BM, cols);
    return;
  }
  float* mine = partial + int64_t(it.slot) * (BM * BN);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    float* row = mine + lane_row(tm) * BN;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc.c[tm][tn];
        *reinterpret_cast<f32x4*>(row + lane_col(tn, g)) = f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
      }
  }
}

// The split tiles of a weight-gradient GEMM: tile b (b < nsplit * per_expert)
// is tile b % per_expert of split expert b / per_expert; each element is the
// sum of its S partials in split order, rounded to bf16 and stored to the
// expert's row-major [*, ld] block of `out` (expert stride `estride`; NT
// tiles per tile row). A unit is 2048 consecutive elements of one tile, 8
// per thread.
constexpr int kSumThreads = 256;
constexpr int kSumUnits = BM * BN / (8 * kSumThreads);
constexpr int kSumGrid = 1024;
__global__ __launch_bounds__(kSumThreads) void dw_split_sum_kernel(const int32_t* __restrict__ plan_words,
                                                                   const float* __restrict__ partial,
                                                                   int per_expert, int NT, uint16_t* __restrict__ out,
                                                                   int64_t estride, int ld) {
  const DwPlan* plan = reinterpret_cast<const DwPlan*>(plan_words);
  const int units = plan->nsplit * per_expert * kSumUnits;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int b = u / kSumUnits, piece = u % kSumUnits;
    const int r = b / per_expert, local = b % per_expert;
    const int S = plan->S[r];
    const int idx = piece * (8 * kSumThreads) + 8 * int(threadIdx.x);
    const int m = idx / BN, c = idx % BN;
    const int mt = local / NT, nt = local % NT;
    if (c >= ld - nt * BN) continue;  // past the output's last column
    const float* src = partial + int64_t(plan->slot0[r] + local * S) * (BM * BN) + idx;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < S; ++q) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(src + int64_t(q) * (BM * BN));
      const f32x4 d = *reinterpret_cast<const f32x4*>(src + int64_t(q) * (BM * BN) + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] += a[i];
        hi[i] += d[i];
      }
    }
    const u32x4 v = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                     pack_bf16x2(hi[2], hi[3])};
    uint16_t* dst = out + int64_t(plan->e[r]) * estride + (int64_t(mt) * BM + m) * ld + int64_t(nt) * BN + c;
    *reinterpret_cast<u32x4*>(dst) = v;
  }
}

#define MOE_DW_SMEM                                                            \
  __shared__ __attribute__((aligned(16))) int32_t s_cnt[1024];                 \
  __shared__ int32_t s_order[1024];                                            \
  __shared__ int32_t s_flag;                                                   \
  __shared__ int32_t s_next;                                                   \
  __shared__ DwPlan s_plan;

__global__ __launch_bounds__(kThreads) void gemm_dw13_kernel(GemmProblem p, const uint16_t* __restrict__ dh13,
                                                             const uint16_t* __restrict__ x,
                                                             uint16_t* __restrict__ dW13, int32_t* queue,
                                                             float* __restrict__ partial, int32_t* plan_out) {
  MOE_DW_SMEM
  const int H = int(p.H), I = int(p.I);
  const int MT = (2 * I) / BM, NT = H / BN;
  const uint32_t kmagic = div_magic(uint32_t(p.k));
  dw_for_each_item(p.counts, int(p.E), MT * NT, queue, plan_out, s_cnt, s_order, &s_flag, &s_next, &s_plan,
                   [&](const DwItem& it) {
    const int nt = it.local % NT;
    const int mt = it.local / NT;
    const int rows = it.klen;  // this item's rows of the expert, from row it.k0
    const int64_t off = int64_t(__builtin_amdgcn_readfirstlane(p.offsets[it.e])) + it.k0;
    MNMajorLoaderD<DirectRows> lp;
    lp.set_base(dh13 + off * 2 * I + int64_t(mt) * BM, int64_t(rows) * 2 * I - int64_t(mt) * BM);
    lp.fn.ld = 2 * I;
    lp.fn.nrows = rows;
    MNMajorLoaderD<TokenRows> lq;
    lq.set_base(x + int64_t(nt) * BN, p.T * H - int64_t(nt) * BN);
    lq.fn.ld = H;
    lq.fn.src = p.src_of + off;
    lq.fn.rows = rows;
    lq.fn.kk = int(p.k);
    lq.fn.kmagic = kmagic;
    if (rows > 0) {  // an empty expert runs no k loop and stores zeros
      lp.prime(0);
      lq.prime(0);
    }
    Acc acc;
    acc.zero();
    mainloop_direct<true, true>(lp, lq, (rows + BK - 1) / BK, acc);
    dw_store(acc, it, dW13 + int64_t(it.e) * 2 * I * H, H, int64_t(mt) * BM, int64_t(nt) * BN, BN, partial);
  });
}

__global__ __launch_bounds__(kThreads) void gemm_dw2_kernel(GemmProblem p, const uint16_t* __restrict__ dy,
                                                            const uint16_t* __restrict__ act,
                                                            uint16_t* __restrict__ dW2, int32_t* queue,
                                                            float* __restrict__ partial, int32_t* plan_out) {
  MOE_DW_SMEM
  const int H = int(p.H), I = int(p.I);
  const int MT = H / BM, NT = (I + BN - 1) / BN;  // the last n-tile may hold 128 columns
  const uint32_t kmagic = div_magic(uint32_t(p.k));
  dw_for_each_item(p.counts, int(p.E), MT * NT, queue, plan_out, s_cnt, s_order, &s_flag, &s_next, &s_plan,
                   [&](const DwItem& it) {
    const int nt = it.local % NT;
    const int mt = it.local / NT;
    const int rows = it.klen;  // this item's rows of the expert, from row it.k0
    const int64_t off = int64_t(__builtin_amdgcn_readfirstlane(p.offsets[it.e])) + it.k0;
    MNMajorLoaderD<TokenRows> lp;
    lp.set_base(dy + int64_t(mt) * BM, p.T * H - int64_t(mt) * BM);
    lp.fn.ld = H;
    lp.fn.src = p.src_of + off;
    lp.fn.rows = rows;
    lp.fn.kk = int(p.k);
    lp.fn.kmagic = kmagic;
    MNMajorLoaderD<DirectRows> lq;
    lq.set_base(act + off * I + int64_t(nt) * BN, int64_t(rows) * I - int64_t(nt) * BN);
    lq.fn.ld = I;
    lq.fn.nrows = rows;
    const int ncols = min(BN, I - nt * BN);
    lq.nchunks = ncols / 8;
    if (rows > 0) {  // an empty expert runs no k loop and stores zeros
      lp.prime(0);
      lq.prime(0);
    }
    Acc acc;
    acc.zero();
    mainloop_direct<true, true>(lp, lq, (rows + BK - 1) / BK, acc);
    dw_store(acc, it, dW2 + int64_t(it.e) * H * I, I, int64_t(mt) * BM, int64_t(nt) * BN, ncols, partial);
  });
}

// ================================================================== launchers

// ------------------------------------------------------------------ FP8 weight gradients
// dW[e][m][n] = sum over the expert's rows r of P'[m][r] Q'[n][r], with P'
// and Q' the operands quantized along the expert's rows (launch_quant_tokens
// layout: per expert, codes [C][Kp_e] with Kp_e = rows rounded up to 128 and
// zero codes past the rows, experts packed in order, one scale byte per
// (column, 32 rows)). Both operands are k-major there, so the tiles run the
// FP8 k loop of the forward GEMMs over Kp_e / 128 slabs; the schedule is the
// weight-gradient schedule above. MP % 256 == 0; NQ % 128 == 0 (a last
// n-tile of 128 columns reuses row NQ - 1 for the rest, never stored).

// s_kb[e] = sum over e' < e of ceil(counts[e'] / 128), e = 0..E (E <= 1024)
__device__ void block_prefix128(const int32_t* counts, int E, int32_t* s_kb, int32_t* s_tmp) {
  const int tid = threadIdx.x;
  int32_t loc[2], sum = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * tid + q;
    loc[q] = e < E ? (counts[e] + 127) / 128 : 0;
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
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * tid + q;
    if (e < E) s_kb[e] = run;
    run += loc[q];
  }
  if (tid == kThreads - 1) s_kb[E] = s_tmp[tid];
  __syncthreads();
}
static_assert(2 * kThreads >= 1024, "block_prefix128 takes two experts per thread");

__global__ __launch_bounds__(kThreads) void gemm_dw_fp8_kernel(GemmProblem p, const uint8_t* __restrict__ pcodes,
                                                               const uint8_t* __restrict__ pscales, int MP,
                                                               const uint8_t* __restrict__ qcodes,
                                                               const uint8_t* __restrict__ qscales, int NQ,
                                                               uint16_t* __restrict__ dW, int32_t* queue,
                                                               float* __restrict__ partial, int32_t* plan_out) {
  MOE_DW_SMEM
  __shared__ int32_t s_kb[1025];
  const int E = int(p.E);
  block_prefix128(p.counts, E, s_kb, s_cnt);  // s_cnt as scratch: the schedule refills it
  const int MT = MP / BM, NT = (NQ + BN - 1) / BN;
  dw_for_each_item(p.counts, E, MT * NT, queue, plan_out, s_cnt, s_order, &s_flag, &s_next, &s_plan,
                   [&](const DwItem& it) {
    const int nt = it.local % NT;
    const int mt = it.local / NT;
    const int e = it.e;
    const int64_t poff = int64_t(__builtin_amdgcn_readfirstlane(s_kb[e])) * 128;
    const int64_t kp = int64_t(__builtin_amdgcn_readfirstlane(s_kb[e + 1] - s_kb[e])) * 128;  // Kp_e
    // this item's codes [k0, kend) of each row (k0 a multiple of 128; the
    // last split runs to Kp_e, over the zero codes past the rows)
    const int64_t kend = it.S == 1 ? kp : min(kp, int64_t(it.k0) + it.chunk);
    const int kb = int((kend - it.k0) / 128);
    const int KU = int(kp / 2);  // row stride in 16-bit units
    const int ncols = min(BN, NQ - nt * BN);
    const int64_t pb = int64_t(MP) * poff + int64_t(mt) * BM * kp + it.k0;  // byte of P row 0, code k0
    const int64_t qb = int64_t(NQ) * poff + int64_t(nt) * BN * kp + it.k0;
    KMajorLoader8 lp, lq;  // through registers: straight into LDS this kernel spills 67 VGPRs
    lp.set_base(reinterpret_cast<const uint16_t*>(pcodes + pb), int64_t(BM) * KU - it.k0 / 2, pscales + pb / 32,
                int64_t(BM) * kp / 32 - it.k0 / 32);
    lq.set_base(reinterpret_cast<const uint16_t*>(qcodes + qb), int64_t(ncols) * KU - it.k0 / 2, qscales + qb / 32,
                int64_t(ncols) * kp / 32 - it.k0 / 32);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = KMajorLoader::row_of_thread(i);
      lp.set_row(i, int64_t(m) * KU);
      lq.set_row(i, int64_t(min(m, ncols - 1)) * KU);
    }
    Acc acc;
    acc.zero();
    mainloop_fp8(lp, lq, kb, acc);  // an empty expert runs no slab and stores zeros
    dw_store(acc, it, dW + int64_t(e) * MP * NQ, NQ, int64_t(mt) * BM, int64_t(nt) * BN, ncols, partial);
  });
}

static int grid_for(int64_t tiles, int num_cus) {
  int64_t g = int64_t(num_cus);  // one 512-thread workgroup per CU (LDS-bound)
  if (tiles < g) g = tiles;
  if (g < 1) g = 1;
  return int(g);
}

static int64_t row_tiles_upper(const GemmProblem& p) { return (p.T * p.k + BM - 1) / BM + p.E; }

hipError_t launch_gemm1_swiglu(const GemmProblem& p, GemmOperand x, GemmOperand W13, uint16_t* h13,
                               uint16_t* act, hipStream_t st, KernelTimer* timer) {
  const int grid = grid_for(row_tiles_upper(p) * (2 * p.I / BN), p.num_cus);
  const Operand X{x.data, x.scales}, W{W13.data, W13.scales};
  if (W13.fp4) {
    TimedLaunch tl(timer, "gemm1_swiglu_fp8_fp4", st);
    hipLaunchKernelGGL((gemm1_swiglu_kernel<true, true>), dim3(grid), dim3(kThreads), 0, st, p, X, W, h13, act);
  } else if (x.f32s) {
    TimedLaunch tl(timer, "gemm1_swiglu_fp8f32", st);
    hipLaunchKernelGGL((gemm1_swiglu_kernel<true, false, true>), dim3(grid), dim3(kThreads), 0, st, p, X, W, h13,
                       act);
  } else if (x.scales) {
    TimedLaunch tl(timer, "gemm1_swiglu_fp8", st);
    hipLaunchKernelGGL(gemm1_swiglu_kernel<true>, dim3(grid), dim3(kThreads), 0, st, p, X, W, h13, act);
  } else {
    TimedLaunch tl(timer, "gemm1_swiglu", st);
    hipLaunchKernelGGL(gemm1_swiglu_kernel<false>, dim3(grid), dim3(kThreads), 0, st, p, X, W, h13, act);
  }
  return hipGetLastError();
}

hipError_t launch_gemm2(const GemmProblem& p, GemmOperand act, GemmOperand W2, uint16_t* out_rows,
                        hipStream_t st, KernelTimer* timer) {
  const int grid = grid_for(row_tiles_upper(p) * (p.H / BN), p.num_cus);
  const Operand A{act.data, act.scales}, W{W2.data, W2.scales};
  if (W2.fp4) {
    TimedLaunch tl(timer, "gemm2_fp8_fp4", st);
    hipLaunchKernelGGL((gemm2_kernel<true, true>), dim3(grid), dim3(kThreads), 0, st, p, A, W, out_rows);
  } else if (act.f32s) {
    TimedLaunch tl(timer, "gemm2_fp8f32", st);
    hipLaunchKernelGGL((gemm2_kernel<true, false, true>), dim3(grid), dim3(kThreads), 0, st, p, A, W, out_rows);
  } else if (act.scales) {
    TimedLaunch tl(timer, "gemm2_fp8", st);
    hipLaunchKernelGGL(gemm2_kernel<true>, dim3(grid), dim3(kThreads), 0, st, p, A, W, out_rows);
  } else {
    TimedLaunch tl(timer, "gemm2", st);
    hipLaunchKernelGGL(gemm2_kernel<false>, dim3(grid), dim3(kThreads), 0, st, p, A, W, out_rows);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_dh(const GemmProblem& p, GemmOperand dy, GemmOperand W2, const uint16_t* h13,
                          uint16_t* dh13, float* dwpart, hipStream_t st, KernelTimer* timer) {
  const int grid = grid_for(row_tiles_upper(p) * ((p.I + BN - 1) / BN), p.num_cus);
  const Operand D{dy.data, dy.scales}, W{W2.data, W2.scales};
  if (dy.f32s) {
    TimedLaunch tl(timer, "gemm_dh_dswiglu_fp8f32", st);
    hipLaunchKernelGGL((gemm_dh_kernel<true, true>), dim3(grid), dim3(kThreads), 0, st, p, D, W, h13, dh13, dwpart);
  } else if (dy.scales) {
    TimedLaunch tl(timer, "gemm_dh_dswiglu_fp8", st);
    hipLaunchKernelGGL(gemm_dh_kernel<true>, dim3(grid), dim3(kThreads), 0, st, p, D, W, h13, dh13, dwpart);
  } else {
    TimedLaunch tl(timer, "gemm_dh_dswiglu", st);
    hipLaunchKernelGGL(gemm_dh_kernel<false>, dim3(grid), dim3(kThreads), 0, st, p, D, W, h13, dh13, dwpart);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const GemmProblem& p, GemmOperand dh13, GemmOperand W13, uint16_t* dx_rows,
                          hipStream_t st, KernelTimer* timer) {
  const int grid = grid_for(row_tiles_upper(p) * (p.H / BN), p.num_cus);
  const Operand D{dh13.data, dh13.scales}, W{W13.data, W13.scales};
  if (dh13.f32s) {
    TimedLaunch tl(timer, "gemm_dx_fp8f32", st);
    hipLaunchKernelGGL((gemm_dx_kernel<true, true>), dim3(grid), dim3(kThreads), 0, st, p, D, W, dx_rows);
  } else if (dh13.scales) {
    TimedLaunch tl(timer, "gemm_dx_fp8", st);
    hipLaunchKernelGGL(gemm_dx_kernel<true>, dim3(grid), dim3(kThreads), 0, st, p, D, W, dx_rows);
  } else {
    TimedLaunch tl(timer, "gemm_dx", st);
    hipLaunchKernelGGL(gemm_dx_kernel<false>, dim3(grid), dim3(kThreads), 0, st, p, D, W, dx_rows);
  }
  return hipGetLastError();
}

__global__ void zero_words_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

hipError_t launch_zero_queues(int32_t* queues, hipStream_t st, KernelTimer* timer) {
  TimedLaunch tl(timer, "zero_queues", st);
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, st, queues, kQueueWords);
  return hipGetLastError();
}

static hipError_t launch_dw_split_sum(const int32_t* plan, const float* partial, int per_expert, int NT,
                                      uint16_t* out, int64_t estride, int ld, hipStream_t st, KernelTimer* timer,
                                      const char* name) {
  TimedLaunch tl(timer, name, st);
  hipLaunchKernelGGL(dw_split_sum_kernel, dim3(kSumGrid), dim3(kSumThreads), 0, st, plan, partial, per_expert, NT,
                     out, estride, ld);
  return hipGetLastError();
}

hipError_t launch_gemm_dw13(const GemmProblem& p, const uint16_t* dh13, const uint16_t* x, uint16_t* dW13,
                            int32_t* queue, float* partial, int32_t* plan, hipStream_t st, KernelTimer* timer) {
  const int MT = int(2 * p.I / BM), NT = int(p.H / BN);
  const int grid = grid_for(p.E * MT * NT, p.num_cus);
  {
    TimedLaunch tl(timer, "gemm_dw13", st);
    hipLaunchKernelGGL(gemm_dw13_kernel, dim3(grid), dim3(kThreads), 0, st, p, dh13, x, dW13, queue, partial, plan);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dw_split_sum(plan, partial, MT * NT, NT, dW13, 2 * p.I * p.H, int(p.H), st, timer,
                             "dw13_split_sum");
}

hipError_t launch_gemm_dw2(const GemmProblem& p, const uint16_t* dy, const uint16_t* act, uint16_t* dW2,
                           int32_t* queue, float* partial, int32_t* plan, hipStream_t st, KernelTimer* timer) {
  const int MT = int(p.H / BM), NT = int((p.I + BN - 1) / BN);
  const int grid = grid_for(p.E * MT * NT, p.num_cus);
  {
    TimedLaunch tl(timer, "gemm_dw2", st);
    hipLaunchKernelGGL(gemm_dw2_kernel, dim3(grid), dim3(kThreads), 0, st, p, dy, act, dW2, queue, partial, plan);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dw_split_sum(plan, partial, MT * NT, NT, dW2, p.H * p.I, int(p.I), st, timer, "dw2_split_sum");
}

hipError_t launch_gemm_dw_fp8(const GemmProblem& p, const uint8_t* pcodes, const uint8_t* pscales, int MP,
                              const uint8_t* qcodes, const uint8_t* qscales, int NQ, uint16_t* dW, int32_t* queue,
                              float* partial, int32_t* plan, hipStream_t st, KernelTimer* timer, const char* name,
                              const char* sum_name) {
  const int MT = MP / BM, NT = (NQ + BN - 1) / BN;
  const int grid = grid_for(p.E * MT * NT, p.num_cus);
  {
    TimedLaunch tl(timer, name, st);
    hipLaunchKernelGGL(gemm_dw_fp8_kernel, dim3(grid), dim3(kThreads), 0, st, p, pcodes, pscales, MP, qcodes,
                       qscales, NQ, dW, queue, partial, plan);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dw_split_sum(plan, partial, MT * NT, NT, dW, int64_t(MP) * NQ, NQ, st, timer, sum_name);
}

}  // namespace moe
