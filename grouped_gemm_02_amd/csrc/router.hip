// Router step before the layer: softmax over a token's expert logits, the k
// largest, and the routing weights (optionally renormalised over the k), plus
// its backward to the logits. The pages keep the router outside the measured
// layer and name that, together with uniform random routing, as the
// benchmark's idealisation (ic.work analysis, section on the benchmark's
// idealised assumptions); this step makes a router-inclusive, skew-aware
// measurement possible.
//
// One wave per token; lane l holds the logits of experts l + 64 i (E <= 1024,
// so at most 16 per lane; the kernels are instantiated for 2, 4 and 16). Experts are selected one at a time by a wave-wide
// arg-max over the logits not yet taken (ties to the lower expert id), which
// orders them by descending logit exactly. Sums and maxima are butterfly
// reductions in a fixed order, so results are reproducible.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kRouteWaves = 4;

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// (v, id) of the largest v, ties to the smaller id, in every lane
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(id, off);
    if (ov > v || (ov == v && oi < id)) {
      v = ov;
      id = oi;
    }
  }
}

// Routes token t (one wave): the k experts with the largest logits in
// descending order (ties to the lower id) and their weights. Slot j ends in
// lane j % 64, register j / 64: sel_i[i] (expert) and sel_w[i] (weight) for
// j = lane + 64 i < k. PER logits per lane: E <= 64 * PER.
template <int PER>
__device__ __forceinline__ void route_token(const float* __restrict__ z, int E, int k, int renorm, int (&sel_i)[PER],
                                            float (&sel_w)[PER]) {
  constexpr int kRouteMaxPer = PER;
  const int lane = lane_id();
  float v[kRouteMaxPer];
#pragma unroll
  for (int i = 0; i < kRouteMaxPer; ++i) v[i] = lane + 64 * i < E ? z[lane + 64 * i] : -INFINITY;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRouteMaxPer; ++i) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kRouteMaxPer; ++i) s += lane + 64 * i < E ? expf(v[i] - m) : 0.f;
  s = wave_sum(s);
  // selection: slot j is kept by lane j % 64 in its register j / 64
  uint32_t taken = 0;
  float sel_v[kRouteMaxPer];
  float first = 0.f;  // the largest selected logit
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kRouteMaxPer; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) first = bv;
#pragma unroll
    for (int i = 0; i < kRouteMaxPer; ++i)
      if (j == lane + 64 * i) {
        sel_v[i] = bv;
        sel_i[i] = bi;
      }
  }
  float den = s, ref = m;
  if (renorm) {  // softmax of the selected logits
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < kRouteMaxPer; ++i)
      if (lane + 64 * i < k) d += expf(sel_v[i] - first);
    den = wave_sum(d);
    ref = first;
  }
#pragma unroll
  for (int i = 0; i < kRouteMaxPer; ++i)
    if (lane + 64 * i < k) sel_w[i] = expf(sel_v[i] - ref) / den;
}

template <int PER>
__global__ __launch_bounds__(64 * kRouteWaves) void route_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                                 int k, int renorm, int32_t* __restrict__ idx,
                                                                 float* __restrict__ w) {
  const int64_t t = int64_t(blockIdx.x) * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;  // the whole wave
  int sel_i[PER];
  float sel_w[PER];
  route_token<PER>(logits + t * E, E, k, renorm, sel_i, sel_w);
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = lane + 64 * i;
    if (j < k) {
      idx[t * k + j] = sel_i[i];
      w[t * k + j] = sel_w[i];
    }
  }
}

// The router fused with the permutation's first pass: one wave per token
// as route_kernel, and each selected pair f is also counted in its chunk's
// row of the chunk table (chunks of kPermChunk pairs: the counts
// permute_scan reads). The table starts at zero (zero_table_kernel); the
// counts are integer atomics, so the table does not depend on their order.
// Column E (ids outside [0, E)) stays 0: the router names experts in [0, E).
__global__ void zero_table_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0;
}

template <int PER>
__global__ __launch_bounds__(64 * kRouteWaves) void route_hist_kernel(const float* __restrict__ logits, int64_t T,
                                                                      int E, int k, int renorm,
                                                                      int32_t* __restrict__ idx,
                                                                      float* __restrict__ w,
                                                                      int32_t* __restrict__ chunk_hist) {
  const int64_t t = int64_t(blockIdx.x) * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;  // the whole wave
  int sel_i[PER];
  float sel_w[PER];
  route_token<PER>(logits + t * E, E, k, renorm, sel_i, sel_w);
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = lane + 64 * i;
    if (j < k) {
      const int64_t f = t * k + j;
      idx[f] = sel_i[i];
      w[f] = sel_w[i];
      atomicAdd(chunk_hist + (f / kPermChunk) * (E + 1) + sel_i[i], 1);
    }
  }
}

// d_logits of L given dL/dw (w, idx from route_kernel). Renormalised:
// dL/dz_S = w (dw - <w, dw>), zero elsewhere. Otherwise, with p = softmax(z)
// and G = dw scattered onto the selected experts: dL/dz = p (G - <p, G>).
// Each lane gathers the values of its own experts, then writes them: every
// element of the row is written once.
template <int PER>
__global__ __launch_bounds__(64 * kRouteWaves) void route_bwd_kernel(const float* __restrict__ logits, int64_t T,
                                                                     int E, int k, int renorm,
                                                                     const int32_t* __restrict__ idx,
                                                                     const float* __restrict__ w,
                                                                     const float* __restrict__ dw,
                                                                     float* __restrict__ dz) {
  constexpr int kRouteMaxPer = PER;
  const int64_t t = int64_t(blockIdx.x) * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  float g[kRouteMaxPer];  // G (or the renormalised gradient) of experts lane + 64 i
#pragma unroll
  for (int i = 0; i < kRouteMaxPer; ++i) g[i] = 0.f;
  float c = 0.f;  // <w, dw> over the selection
  for (int j0 = 0; j0 < k; j0 += 64) {
    const int j = j0 + lane;
    const float wj = j < k ? w[t * k + j] : 0.f;
    const float dj = j < k ? dw[t * k + j] : 0.f;
    c += wj * dj;
  }
  c = wave_sum(c);
  for (int j0 = 0; j0 < k; j0 += 64) {
    const int j = j0 + lane;
    const int ej = j < k ? idx[t * k + j] : -1;
    const float vj = j < k ? (renorm ? w[t * k + j] * (dw[t * k + j] - c) : dw[t * k + j]) : 0.f;
    const int n = min(64, k - j0);
    for (int q = 0; q < n; ++q) {  // slot j0 + q: its expert's lane takes the value
      const int e = __shfl(ej, q);
      const float val = __shfl(vj, q);
#pragma unroll
      for (int i = 0; i < kRouteMaxPer; ++i)
        if (e == lane + 64 * i) g[i] = val;
    }
  }
  float* out = dz + t * E;
  if (renorm) {
#pragma unroll
    for (int i = 0; i < kRouteMaxPer; ++i)
      if (lane + 64 * i < E) out[lane + 64 * i] = g[i];
    return;
  }
  const float* z = logits + t * E;
  float v[kRouteMaxPer];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRouteMaxPer; ++i) {
    v[i] = lane + 64 * i < E ? z[lane + 64 * i] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
  m = wave_max(m);
  float s = 0.f, pg = 0.f;
#pragma unroll
  for (int i = 0; i < kRouteMaxPer; ++i) {
    v[i] = lane + 64 * i < E ? expf(v[i] - m) : 0.f;  // unnormalised p
    s += v[i];
    pg += v[i] * g[i];
  }
  s = wave_sum(s);
  pg = wave_sum(pg) / s;
#pragma unroll
  for (int i = 0; i < kRouteMaxPer; ++i)
    if (lane + 64 * i < E) out[lane + 64 * i] = v[i] / s * (g[i] - pg);
}

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int renorm, int32_t* idx, float* w,
                        hipStream_t st, KernelTimer* timer) {
  if (T <= 0) return hipSuccess;
  TimedLaunch tl(timer, "route", st);
  const dim3 grid(unsigned((T + kRouteWaves - 1) / kRouteWaves)), block(64 * kRouteWaves);
  if (E <= 128)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, st, logits, T, E, k, renorm, idx, w);
  else if (E <= 256)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, st, logits, T, E, k, renorm, idx, w);
  else
    hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, st, logits, T, E, k, renorm, idx, w);
  return hipGetLastError();
}

hipError_t launch_route_hist(const float* logits, int64_t T, int E, int k, int renorm, int32_t* idx, float* w,
                             int32_t* chunk_hist, hipStream_t st, KernelTimer* timer) {
  if (T <= 0) return hipSuccess;
  const int64_t words = (T * k + kPermChunk - 1) / kPermChunk * (E + 1);
  {
    TimedLaunch tl(timer, "route_table_zero", st);
    const int64_t g = (words + 255) / 256;
    hipLaunchKernelGGL(zero_table_kernel, dim3(static_cast<unsigned>(g < 1024 ? g : 1024)), dim3(256), 0, st,
                       chunk_hist, words);
  }
  TimedLaunch tl(timer, "route_hist", st);
  const dim3 grid(static_cast<unsigned>((T + kRouteWaves - 1) / kRouteWaves)), block(64 * kRouteWaves);
  if (E <= 128)
    hipLaunchKernelGGL(route_hist_kernel<2>, grid, block, 0, st, logits, T, E, k, renorm, idx, w, chunk_hist);
  else if (E <= 256)
    hipLaunchKernelGGL(route_hist_kernel<4>, grid, block, 0, st, logits, T, E, k, renorm, idx, w, chunk_hist);
  else
    hipLaunchKernelGGL(route_hist_kernel<16>, grid, block, 0, st, logits, T, E, k, renorm, idx, w, chunk_hist);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const float* logits, int64_t T, int E, int k, int renorm, const int32_t* idx,
                            const float* w, const float* dw, float* dz, hipStream_t st, KernelTimer* timer) {
  if (T <= 0) return hipSuccess;
  TimedLaunch tl(timer, "route_bwd", st);
  const dim3 grid(unsigned((T + kRouteWaves - 1) / kRouteWaves)), block(64 * kRouteWaves);
  if (E <= 128)
    hipLaunchKernelGGL(route_bwd_kernel<2>, grid, block, 0, st, logits, T, E, k, renorm, idx, w, dw, dz);
  else if (E <= 256)
    hipLaunchKernelGGL(route_bwd_kernel<4>, grid, block, 0, st, logits, T, E, k, renorm, idx, w, dw, dz);
  else
    hipLaunchKernelGGL(route_bwd_kernel<16>, grid, block, 0, st, logits, T, E, k, renorm, idx, w, dw, dz);
  return hipGetLastError();
}

}  // namespace moe
