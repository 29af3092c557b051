// Expert-contiguous permutation of the routed (token, slot) pairs.
//
// Routing indices become a token reorder in which every expert's rows are
// contiguous and indexed by group offsets, the first stage of the fused
// pipeline (kongchang.com explainer, grouped-GEMM note). Integer work, so
// the result is exact and deterministic: the rows of one expert keep the
// ascending order of the flat pair index f = t*k + j.
//
// Three launches:
//   permute_hist    per chunk of kChunk pairs, per-expert counts (LDS integer
//                   atomics: the totals do not depend on their order); column E
//                   counts ids outside [0, E)
//   permute_scan    one workgroup: per-expert totals, exclusive prefix over
//                   experts (offsets) and each chunk's starting row per expert
//   permute_scatter per chunk again, in pair order: the rank of a pair among
//                   the equal ids before it comes from wavefront ballots
//                   (lanes with the same id found bit by bit), per-wave counts
//                   in LDS and a running per-chunk count, then
//                   row_of[f] = start + rank and src_of[row] = f (and, for
//                   the layer, the pair's routing weight at its row).
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kPermThreads = 256;
constexpr int kPermItems = 4;
constexpr int kChunk = kPermThreads * kPermItems;  // 1024 pairs per workgroup
static_assert(kChunk == kPermChunk, "the router's fused histogram uses the same chunks");
constexpr int kPermWaves = kPermThreads / kWave;

__global__ __launch_bounds__(kPermThreads) void permute_hist(const int32_t* __restrict__ idx,
                                                             int64_t n, int E,
                                                             int32_t* __restrict__ chunk_hist) {
  extern __shared__ int32_t hist[];  // E + 1
  for (int e = threadIdx.x; e <= E; e += kPermThreads) hist[e] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * kChunk;
  for (int it = 0; it < kPermItems; ++it) {
    const int64_t f = base + int64_t(it) * kPermThreads + threadIdx.x;
    if (f < n) {
      int e = idx[f];
      if (e < 0 || e >= E) e = E;
      atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  int32_t* out = chunk_hist + int64_t(blockIdx.x) * (E + 1);
  for (int e = threadIdx.x; e <= E; e += kPermThreads) out[e] = hist[e];
}

// One workgroup of 1024 threads. chunk_hist [nchunk][E+1] is turned in place
// into each chunk's first row per expert; counts/offsets written; status word
// set when any id was out of range. The chunk axis is cut into S segments so
// that S*(E+1) threads share the per-expert running sums: pass 1 sums each
// segment, the segment prefixes and expert offsets follow in LDS, pass 2
// rewrites each segment's chunks as running starts.
__global__ __launch_bounds__(1024) void permute_scan(int32_t* __restrict__ chunk_hist, int nchunk,
                                                     int E, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ status) {
  __shared__ int32_t seg[1025];  // [S][E+1] segment sums (S * (E+1) <= 1025)
  __shared__ int32_t tot[1025];
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int W = E + 1;                      // columns (column E = invalid ids)
  const int S = max(1, 1024 / W);           // segments of the chunk axis
  const int cps = (nchunk + S - 1) / S;     // chunks per segment
  // work item w = sg * W + e: segment sg of column e (E = 1024 gives one
  // segment and 1025 items, so thread 0 also takes item 1024)
  for (int w = tid; w < S * W; w += 1024) {
    const int e = w % W, sg = w / W;
    const int c0 = min(nchunk, sg * cps), c1 = min(nchunk, c0 + cps);
    int32_t sum = 0;
    for (int c = c0; c < c1; ++c) sum += chunk_hist[int64_t(c) * W + e];
    seg[w] = sum;
  }
  __syncthreads();
  for (int x = tid; x < W; x += 1024) {
    int32_t run = 0;
    for (int q = 0; q < S; ++q) run += seg[q * W + x];
    tot[x] = run;
  }
  __syncthreads();
  // exclusive scan of tot[0..E) (E <= 1024): Hillis-Steele on a copy
  int32_t v = tid < E ? tot[tid] : 0;
  part[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const int32_t excl = part[tid] - v;  // exclusive prefix at tid
  if (tid < E) {
    counts[tid] = v;
    offsets[tid] = excl;
    tot[tid] = excl;  // reused below as the expert's first row
  }
  if (tid == E - 1) offsets[E] = part[tid];
  if (tid == 0) status[0] = tot[E] > 0 ? 8 /* MOE_ERR_ROUTING */ : 0;
  __syncthreads();
  for (int w = tid; w < S * W; w += 1024) {
    const int e = w % W, sg = w / W;
    if (e == E) continue;
    const int c0 = min(nchunk, sg * cps), c1 = min(nchunk, c0 + cps);
    int32_t run = tot[e];
    for (int q = 0; q < sg; ++q) run += seg[q * W + e];
    for (int c = c0; c < c1; ++c) {
      int32_t* p = chunk_hist + int64_t(c) * W + e;
      const int32_t x = *p;
      *p = run;
      run += x;
    }
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter(
    const int32_t* __restrict__ idx, int64_t n, int E, int id_bits,
    const int32_t* __restrict__ chunk_start, int32_t* __restrict__ row_of,
    int32_t* __restrict__ src_of, const float* __restrict__ topk_w, float* __restrict__ wrow) {
  extern __shared__ int32_t sm[];
  int32_t* running = sm;                // [E+1]  rows already placed in this chunk
  int32_t* wave_cnt = sm + (E + 1);     // [kPermWaves][E+1]
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  for (int i = tid; i < (E + 1) * (1 + kPermWaves); i += kPermThreads) sm[i] = 0;
  const int32_t* start = chunk_start + int64_t(blockIdx.x) * (E + 1);
  const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * kChunk;
  for (int it = 0; it < kPermItems; ++it) {
    const int64_t f = base + int64_t(it) * kPermThreads + tid;
    const bool in_range = f < n;
    int e = E;
    if (in_range) {
      e = idx[f];
      if (e < 0 || e >= E) e = E;
    }
    // peers: lanes of this wave holding the same id (and in range)
    uint64_t peers = __ballot(in_range);
    if (!in_range) peers = ~peers;
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(bit);
      peers &= bit ? ones : ~ones;
    }
    const int rank_in_wave = __popcll(peers & lanes_below);
    const bool leader = rank_in_wave == 0;
    if (in_range && leader) wave_cnt[wave * (E + 1) + e] = __popcll(peers);
    __syncthreads();
    if (in_range) {
      int32_t before = running[e];
      for (int w = 0; w < wave; ++w) before += wave_cnt[w * (E + 1) + e];
      if (e < E) {
        const int32_t row = start[e] + before + rank_in_wave;
        row_of[f] = row;
        src_of[row] = static_cast<int32_t>(f);
        if (wrow) wrow[row] = topk_w[f];
      } else {
        row_of[f] = -1;
      }
    }
    __syncthreads();
    if (in_range && leader) {
      atomicAdd(&running[e], __popcll(peers));
      wave_cnt[wave * (E + 1) + e] = 0;
    }
    __syncthreads();
  }
}

int permute_num_chunks(int64_t n) { return int((n + kChunk - 1) / kChunk); }

size_t permute_scratch_bytes(int64_t n, int E) {
  // [status word, padded to 256 B][chunk table nchunk x (E+1) int32]
  const int64_t nchunk = permute_num_chunks(n);
  return 256 + size_t(nchunk > 0 ? nchunk : 1) * size_t(E + 1) * 4;
}

hipError_t launch_permute(const int32_t* idx, int64_t n, int E, int32_t* counts,
                          int32_t* offsets, int32_t* row_of, int32_t* src_of, void* scratch,
                          hipStream_t st, KernelTimer* timer, const float* topk_w, float* wrow) {
  return launch_permute_split(idx, n, E, counts, offsets, row_of, src_of, static_cast<int32_t*>(scratch),
                              reinterpret_cast<int32_t*>(static_cast<char*>(scratch) + 256), st, timer, topk_w,
                              wrow);
}

hipError_t launch_permute_split(const int32_t* idx, int64_t n, int E, int32_t* counts, int32_t* offsets,
                                int32_t* row_of, int32_t* src_of, int32_t* status, int32_t* chunk_tab,
                                hipStream_t st, KernelTimer* timer, const float* topk_w, float* wrow,
                                bool hist_done) {
  const int nchunk = permute_num_chunks(n);
  int id_bits = 0;
  while ((1 << id_bits) <= E) ++id_bits;  // ids 0..E (E marks invalid) fit
  if (nchunk > 0 && !hist_done) {
    TimedLaunch t(timer, "permute_hist", st);
    hipLaunchKernelGGL(permute_hist, dim3(nchunk), dim3(kPermThreads), (E + 1) * 4, st, idx, n,
                       E, chunk_tab);
  }
  {
    TimedLaunch t(timer, "permute_scan", st);
    hipLaunchKernelGGL(permute_scan, dim3(1), dim3(1024), 0, st, chunk_tab, nchunk, E, counts,
                       offsets, status);
  }
  if (nchunk > 0) {
    TimedLaunch t(timer, "permute_scatter", st);
    hipLaunchKernelGGL(permute_scatter, dim3(nchunk), dim3(kPermThreads),
                       (E + 1) * (1 + kPermWaves) * 4, st, idx, n, E, id_bits, chunk_tab, row_of,
                       src_of, topk_w, wrow);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- fixed scratch
// The chunk table of launch_permute in a file-scope device array, for
// callers that cannot allocate (see permute_static_scratch). Each device the
// library runs on holds its own copy until the process ends; every call on a
// device uses the same copy, so calls that overlap on one device race.
// Nothing in it needs to start at zero: permute_hist writes every entry of
// the table before permute_scan or permute_scatter reads it.
static __device__ __align__(256) int32_t scratch[kStaticPermuteWords];

namespace {
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t permute_static_scratch(int32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the array's device address on the current device (the host-side name
    // is only a stand-in and must never reach a kernel)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
