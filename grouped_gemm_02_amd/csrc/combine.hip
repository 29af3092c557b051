// Weighted top-k combine as a gather-reduce without atomics.
//
// Expert outputs are aggregated back per token (kongchang.com explainer,
// first paragraph on MoE structure; MarkTechPost article, "How does the fused
// kernel work?": combine). The routing weight is already folded into each
// permuted row by the down GEMM's epilogue, so
//   out[t] = sum_{j = 0..k-1} rows[row_of[t*k + j]]
// in fp32, slots in ascending j, one bf16 rounding at the end; dropped pairs
// (row_of = -1) add nothing. Each token owns its output row, so there is no
// atomic and the result is bitwise reproducible. The same kernel reduces the
// dX rows in the backward and, there, also sums the routing-weight-gradient
// partials of each pair in a fixed order.
//
// HBM-bound: per token it reads k rows of H bf16 and writes one row. Both
// go through streaming (nontemporal) accesses: the rows are read once, and
// the output is not read again inside the layer, so neither is kept in the
// caches (measured 12-16 % faster than cached accesses).
//
// With k = 1 the down and dX GEMMs write each row straight to its token
// (the sum has one term, so the result is the same bits); launch_combine is
// then called with rows == nullptr and only writes the zero rows of dropped
// tokens and the routing-weight gradients.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kCombThreads = 256;

// One workgroup per token; thread t covers bf16 columns [8t, 8t+8) + 2048*s.
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const uint16_t* __restrict__ rows, const int32_t* __restrict__ row_of, int k, int H,
    uint16_t* __restrict__ out, const float* __restrict__ dwpart, int nparts,
    float* __restrict__ d_topk_w) {
  const int64_t t = blockIdx.x;
  const int32_t* ro = row_of + t * k;
  for (int c0 = threadIdx.x * 8; c0 < H; c0 += kCombThreads * 8) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int32_t r = ro[j];
      if (r < 0) continue;
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rows + int64_t(r) * H + c0));
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[2 * d] += bf16_lo(v[d]);
        acc[2 * d + 1] += bf16_hi(v[d]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(acc[2 * d], acc[2 * d + 1]);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + t * H + c0));
  }
  if (dwpart != nullptr) {
    for (int j = threadIdx.x; j < k; j += kCombThreads) {
      const int32_t r = ro[j];
      float s = 0.f;
      if (r >= 0) {
        const float* pp = dwpart + int64_t(r) * nparts;
        for (int c = 0; c < nparts; ++c) s += pp[c];
      }
      d_topk_w[t * k + j] = s;
    }
  }
}

// k == 1, rows already in out: one thread per token zeroes the row of a
// dropped token and sums its routing-weight-gradient partials.
__global__ __launch_bounds__(kCombThreads) void top1_finish_kernel(const int32_t* __restrict__ row_of, int64_t T,
                                                                   int H, uint16_t* __restrict__ out,
                                                                   const float* __restrict__ dwpart, int nparts,
                                                                   float* __restrict__ d_topk_w) {
  const int64_t t = int64_t(blockIdx.x) * kCombThreads + threadIdx.x;
  if (t >= T) return;
  const int32_t r = row_of[t];
  if (r < 0) {
    for (int c0 = 0; c0 < H; c0 += 8) *reinterpret_cast<u32x4*>(out + t * H + c0) = u32x4{0u, 0u, 0u, 0u};
  }
  if (dwpart != nullptr) {
    float s = 0.f;
    if (r >= 0)
      for (int c = 0; c < nparts; ++c) s += dwpart[int64_t(r) * nparts + c];
    d_topk_w[t] = s;
  }
}

hipError_t launch_combine(const uint16_t* rows, const int32_t* row_of, int64_t T, int k, int64_t H,
                          uint16_t* out, const float* dwpart, int nparts, float* d_topk_w,
                          hipStream_t st, KernelTimer* timer, const char* name) {
  if (T <= 0) return hipSuccess;
  TimedLaunch tl(timer, name, st);
  if (rows == nullptr) {  // k == 1: see top1_finish_kernel
    hipLaunchKernelGGL(top1_finish_kernel, dim3(unsigned((T + kCombThreads - 1) / kCombThreads)),
                       dim3(kCombThreads), 0, st, row_of, T, int(H), out, dwpart, nparts, d_topk_w);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned(T)), dim3(kCombThreads), 0, st, rows, row_of, k,
                     int(H), out, dwpart, nparts, d_topk_w);
  return hipGetLastError();
}

}  // namespace moe
