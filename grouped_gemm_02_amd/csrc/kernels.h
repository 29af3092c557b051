// Host-side launcher declarations for the MoE layer's HIP kernels, and the
// optional per-kernel event timer used by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Records one (start, stop) HIP event pair per launch when enabled.
struct KernelTimer {
  virtual void begin(const char* name, hipStream_t st) = 0;
  virtual void end(hipStream_t st) = 0;
  virtual ~KernelTimer() {}
};

struct TimedLaunch {
  KernelTimer* t;
  hipStream_t st;
  TimedLaunch(KernelTimer* timer, const char* name, hipStream_t s) : t(timer), st(s) {
    if (t) t->begin(name, st);
  }
  ~TimedLaunch() {
    if (t) t->end(st);
  }
};

// ---------------------------------------------------------------- permute
constexpr int kPermChunk = 1024;  // pairs per chunk of the permutation's passes
int permute_num_chunks(int64_t n);
size_t permute_scratch_bytes(int64_t n, int E);
// When wrow != nullptr also wrow[row_of[f]] = topk_w[f].
hipError_t launch_permute(const int32_t* idx, int64_t n, int E, int32_t* counts,
                          int32_t* offsets, int32_t* row_of, int32_t* src_of, void* scratch,
                          hipStream_t st, KernelTimer* timer, const float* topk_w = nullptr,
                          float* wrow = nullptr);

// The same with the status word and the chunk table given apart. With
// hist_done the table already holds the chunks' per-expert counts (the
// router's fused pass wrote them) and the histogram launch is skipped.
hipError_t launch_permute_split(const int32_t* idx, int64_t n, int E, int32_t* counts, int32_t* offsets,
                                int32_t* row_of, int32_t* src_of, int32_t* status, int32_t* chunk_tab,
                                hipStream_t st, KernelTimer* timer, const float* topk_w = nullptr,
                                float* wrow = nullptr, bool hist_done = false);
// A fixed chunk table in device memory the library owns (no allocation):
// kStaticPermuteWords int32 per device, found once per device with
// hipGetSymbolAddress; *out is its address on the current device.
constexpr int64_t kStaticPermuteWords = int64_t(1) << 20;  // 4 MiB
constexpr int kMaxDevices = 64;
hipError_t permute_static_scratch(int32_t** out);

// ---------------------------------------------------------------- combine
// y[t] = sum_j rows[row_of[t*k+j]]  (bf16 rows of width H, fp32 sum, ascending j)
// and, when dwpart != nullptr, d_topk_w[f] = sum_c dwpart[row_of[f]*nparts + c].
// rows == nullptr (k == 1 only): the rows are already in y; zero the rows of
// dropped tokens and reduce d_topk_w.
hipError_t launch_combine(const uint16_t* rows, const int32_t* row_of, int64_t T, int k, int64_t H,
                          uint16_t* out, const float* dwpart, int nparts, float* d_topk_w,
                          hipStream_t st, KernelTimer* timer, const char* name);

// ---------------------------------------------------------------- grouped GEMMs
struct GemmProblem {
  int64_t T, H, I, E, k;
  int num_cus;  // persistent grid cap in CUs
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* src_of;
  const float* topk_w;
  const float* wrow;  // routing weight of each permuted row
};

// A GEMM operand: bf16 elements (scales == nullptr) or E4M3 codes with
// E8M0 scales per (row, 32-block along the reduction axis).
struct GemmOperand {
  const void* data;
  const uint8_t* scales;
  bool fp4 = false;  // E2M1 codes, two per byte (weights of the FP8 x FP4 forward)
  bool f32s = false;  // scales are fp32 per (row, 128-block) (kRuleF32), not E8M0 bytes
};
// forward
hipError_t launch_gemm1_swiglu(const GemmProblem& p, GemmOperand x, GemmOperand W13, uint16_t* h13,
                               uint16_t* act, hipStream_t st, KernelTimer* timer);
hipError_t launch_gemm2(const GemmProblem& p, GemmOperand act, GemmOperand W2, uint16_t* out_rows,
                        hipStream_t st, KernelTimer* timer);
// backward (FP8: W2 as [E, I, H] and W13 as [E, H, 2I], i.e. transposed)
int dh_num_parts(int64_t I);
hipError_t launch_gemm_dh(const GemmProblem& p, GemmOperand dy, GemmOperand W2, const uint16_t* h13,
                          uint16_t* dh13, float* dwpart, hipStream_t st, KernelTimer* timer);
hipError_t launch_gemm_dx(const GemmProblem& p, GemmOperand dh13, GemmOperand W13, uint16_t* dx_rows,
                          hipStream_t st, KernelTimer* timer);
// weight gradients; each takes kQueuesPerGemm zeroed queue words (tile counters), the
// fp32 partial tiles of split items (kSplitFloats floats, shared: the
// weight-gradient GEMMs run one after the other) and kSplitWords words of its
// own for the split plan, which the GEMM writes and its split-sum kernel
// (launched right after it by the same call) reads
constexpr int kQueuesPerGemm = 8;  // one per XCD (the tail split); the skew queue is the first
constexpr int kNumQueues = 2 * kQueuesPerGemm;
constexpr int kSplitWords = 256;
constexpr int kQueueWords = kNumQueues + 2 * kSplitWords;  // queues, then the plan words of both GEMMs
constexpr int64_t kSplitFloats = int64_t(320) * 256 * 256;
hipError_t launch_zero_queues(int32_t* queues, hipStream_t st, KernelTimer* timer);
hipError_t launch_gemm_dw13(const GemmProblem& p, const uint16_t* dh13, const uint16_t* x, uint16_t* dW13,
                            int32_t* queue, float* partial, int32_t* plan, hipStream_t st, KernelTimer* timer);
hipError_t launch_gemm_dw2(const GemmProblem& p, const uint16_t* dy, const uint16_t* act, uint16_t* dW2,
                           int32_t* queue, float* partial, int32_t* plan, hipStream_t st, KernelTimer* timer);

// ---------------------------------------------------------------- FP8 quantization
constexpr int kRulePow2 = 0;  // smallest 2^e with 448 * 2^e >= amax
constexpr int kRuleMx = 1;    // 2^(floor(log2 amax) - 8)
// fp32 scale s = amax / 448, codes of fl32(v * fl32(448 / amax)) (128 or
// 128x128 blocks); the scale array holds one float per (row, 128 values):
// the bytes the E8M0 layout gives that row's four 32-blocks
constexpr int kRuleF32 = 2;
// bf16 [rows, K] -> E4M3 codes [rows, K] + E8M0 scales [rows, K/32]; block 32 or 128
hipError_t launch_quant_rows(const uint16_t* in, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                             int block, int rule, hipStream_t st, KernelTimer* timer, const char* name);
// bf16 W [E, R, C] in 128x128 tiles -> plain codes [E, R, C] and/or transposed codes [E, C, R]
// (either output may be null), each with scales per (output row, 32-block); blockwise rule: one
// exponent per tile, MX rule: per 32 values of an output row
hipError_t launch_quant_weights(const uint16_t* W, int64_t E, int R, int C, uint8_t* pcodes, uint8_t* pscales,
                                uint8_t* tcodes, uint8_t* tscales, int rule, hipStream_t st, KernelTimer* timer);

// bf16 [rows, C] -> E2M1 codes [rows, C/2] (two per byte, the even value in the
// low nibble) + E8M0 scales [rows, C/32], 32-blocks along the rows, MX rule for E2M1
hipError_t launch_quant_fp4_rows(const uint16_t* in, int64_t rows, int C, uint8_t* codes, uint8_t* scales,
                                 hipStream_t st, KernelTimer* timer);

// The FP8 weight-gradient operands: rows of every expert quantized along the
// rows (codes [C][Kp_e] per expert, Kp_e = rows rounded up to 128, experts
// packed in order; one scale byte per (column, 32 rows)). src_of == nullptr:
// expert rows are rows offsets[e] + r of `in`; else token rows src_of[..] / kk.
// rcodes/rscales (optional): also the launch_quant_rows output of the rows
// (each source row must occur once: a direct operand, or kk == 1).
hipError_t launch_quant_tokens(const uint16_t* in, int64_t ld, int C, const int32_t* counts, const int32_t* offsets,
                               int E, int64_t M, const int32_t* src_of, int kk, uint8_t* codes, uint8_t* scales,
                               int rule, hipStream_t st, KernelTimer* timer, const char* name,
                               uint8_t* rcodes = nullptr, uint8_t* rscales = nullptr);
// FP8 weight gradients from those operands: dW[e] (P rows x Q rows, bf16,
// row-major [MP][NQ]) = sum over the expert's rows of P'[m][r] Q'[n][r]
hipError_t launch_gemm_dw_fp8(const GemmProblem& p, const uint8_t* pcodes, const uint8_t* pscales, int MP,
                              const uint8_t* qcodes, const uint8_t* qscales, int NQ, uint16_t* dW, int32_t* queue,
                              float* partial, int32_t* plan, hipStream_t st, KernelTimer* timer, const char* name,
                              const char* sum_name);

// ---------------------------------------------------------------- router
// logits fp32 [T, E] -> idx int32 [T, k] (descending logit, ties to the lower
// id), w fp32 [T, k] (softmax probabilities, renormalised over the k if
// renorm); the backward writes dz fp32 [T, E] = dL/dlogits from dw = dL/dw.
hipError_t launch_route(const float* logits, int64_t T, int E, int k, int renorm, int32_t* idx, float* w,
                        hipStream_t st, KernelTimer* timer);
// the router and the permutation's histogram pass in one launch: writes idx,
// w and the chunk table [nchunk][E+1] of launch_permute_split (hist_done)
hipError_t launch_route_hist(const float* logits, int64_t T, int E, int k, int renorm, int32_t* idx, float* w,
                             int32_t* chunk_hist, hipStream_t st, KernelTimer* timer);
hipError_t launch_route_bwd(const float* logits, int64_t T, int E, int k, int renorm, const int32_t* idx,
                            const float* w, const float* dw, float* dz, hipStream_t st, KernelTimer* timer);

}  // namespace moe
