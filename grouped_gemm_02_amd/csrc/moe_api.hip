// C ABI of the MoE expert layer: validation, buffer layout, launch order.
// Declarations and the contract of every entry point are in include/moe.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ------------------------------------------------------------ shape checks

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_NULL;
  if (s->precision < MOE_BF16 || s->precision > MOE_FP8_BWD_F32) return MOE_ERR_PRECISION;
  if (s->T < 0 || s->E < 1 || s->E > 1024 || s->k < 1 || s->k > s->E) return MOE_ERR_SHAPE;
  if (s->H < 256 || s->H > 16384 || s->H % 256 != 0) return MOE_ERR_SHAPE;
  if (s->I < 128 || s->I > 8192 || s->I % 128 != 0) return MOE_ERR_SHAPE;
  if (s->T * s->k >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (s->T * s->H >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;  // 32-bit row offsets into x, dY
  if (s->T * s->k * s->I >= (int64_t(1) << 30)) return MOE_ERR_SHAPE;  // 32-bit byte offsets into [g | u] rows
  if (s->num_cus < 0 || s->reserved != 0) return MOE_ERR_SHAPE;
  if ((s->flags & ~MOE_FLAG_FP8_WGRAD) != 0) return MOE_ERR_PRECISION;
  if ((s->flags & MOE_FLAG_FP8_WGRAD) != 0) {
    if (s->precision == MOE_BF16 || s->precision == MOE_FP8_FP4) return MOE_ERR_PRECISION;  // no FP8 backward
    // the row-axis quantizer has the power-of-two and MX rules only
    if (s->precision == MOE_FP8_BLOCK_F32 || s->precision == MOE_FP8_BWD_F32) return MOE_ERR_UNSUPPORTED;
    // 32-bit offsets inside a weight-gradient tile's 256 rows of Kp codes
    if (s->T * s->k >= (int64_t(1) << 23)) return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool fp8_forward(const moe_shape& s) {
  return s.precision == MOE_FP8_BLOCK || s.precision == MOE_MXFP8 || s.precision == MOE_FP8_FP4 ||
         s.precision == MOE_FP8_BLOCK_F32;
}
bool fp8_backward(const moe_shape& s) {
  return s.precision == MOE_FP8_BLOCK || s.precision == MOE_MXFP8 || s.precision == MOE_FP8_BWD ||
         s.precision == MOE_FP8_BLOCK_F32 || s.precision == MOE_FP8_BWD_F32;
}
bool fp4_weights(const moe_shape& s) { return s.precision == MOE_FP8_FP4; }
// blockwise with fp32 block scales
bool f32_scales(const moe_shape& s) { return s.precision == MOE_FP8_BLOCK_F32 || s.precision == MOE_FP8_BWD_F32; }
// activation block (32 or 128 values along the reduction axis) and scale rule
bool mx_acts(const moe_shape& s) { return s.precision == MOE_MXFP8 || s.precision == MOE_FP8_FP4; }
int act_block(const moe_shape& s) { return mx_acts(s) ? 32 : 128; }
int scale_rule(const moe_shape& s) { return mx_acts(s) ? kRuleMx : (f32_scales(s) ? kRuleF32 : kRulePow2); }
bool fp8_wgrad(const moe_shape& s) { return (s.flags & MOE_FLAG_FP8_WGRAD) != 0; }
// an upper bound of the sum over experts of rows rounded up to 128
int64_t wgrad_rows_cap(const moe_shape& s) { return 128 * ((s.T * s.k) / 128 + s.E); }

// bytes of E4M3 codes [rows, K] and of their scale bytes [rows, K/32]
size_t codes_bytes(int64_t rows, int64_t K) { return align_up(size_t(rows) * size_t(K)); }
size_t scale_bytes(int64_t rows, int64_t K) { return align_up(size_t(rows) * size_t(K / 32)); }

// ------------------------------------------------------------ buffer layouts

struct FwdLayout {
  size_t perm;     // permutation scratch (status word first)
  size_t rows;     // bf16 [Tk, H] weighted expert outputs
  size_t inf;      // saved-like area used when no saved buffer is given
  size_t xq, xs;   // FP8 forward: x codes [T, H], scales [T, H/32]
  size_t aq, as;   // FP8 forward: w*silu(g)*u codes [Tk, I], scales [Tk, I/32]
  size_t total;
};

moe_wq_layout wq_layout(const moe_shape& s) {
  moe_wq_layout L;
  L.w13 = L.w13_scale = L.w2 = L.w2_scale = SIZE_MAX;
  L.w2t = L.w2t_scale = L.w13t = L.w13t_scale = SIZE_MAX;
  size_t o = 0;
  const int64_t E = s.E, H = s.H, I = s.I;
  if (fp8_forward(s)) {
    const int64_t div = fp4_weights(s) ? 2 : 1;  // FP4: two codes per byte
    L.w13 = o;       o += codes_bytes(E * 2 * I, H / div);
    L.w13_scale = o; o += scale_bytes(E * 2 * I, H);
    L.w2 = o;        o += codes_bytes(E * H, I / div);
    L.w2_scale = o;  o += scale_bytes(E * H, I);
  }
  if (fp8_backward(s)) {
    L.w2t = o;        o += codes_bytes(E * I, H);
    L.w2t_scale = o;  o += scale_bytes(E * I, H);
    L.w13t = o;       o += codes_bytes(E * H, 2 * I);
    L.w13t_scale = o; o += scale_bytes(E * H, 2 * I);
  }
  L.total = o;
  return L;
}

moe_saved_layout saved_layout(const moe_shape& s) {
  const int64_t Tk = s.T * s.k;
  moe_saved_layout L;
  size_t o = 0;
  L.counts = o;  o = align_up(o + size_t(s.E) * 4);
  L.offsets = o; o = align_up(o + size_t(s.E + 1) * 4);
  L.row_of = o;  o = align_up(o + size_t(Tk) * 4);
  L.src_of = o;  o = align_up(o + size_t(Tk) * 4);
  L.wrow = o;    o = align_up(o + size_t(Tk) * 4);
  L.h13 = o;     o = align_up(o + size_t(Tk) * size_t(2 * s.I) * 2);
  L.act = o;     o = align_up(o + size_t(Tk) * size_t(s.I) * 2);
  L.total = o;
  return L;
}

FwdLayout fwd_layout(const moe_shape& s) {
  const int64_t Tk = s.T * s.k;
  FwdLayout L;
  size_t o = 0;
  L.perm = o; o = align_up(o + permute_scratch_bytes(Tk, int(s.E)));
  L.rows = o; o = align_up(o + size_t(Tk) * size_t(s.H) * 2);
  L.inf = o;  o = align_up(o + saved_layout(s).total);
  L.xq = L.xs = L.aq = L.as = 0;
  if (fp8_forward(s)) {
    L.xq = o; o += codes_bytes(s.T, s.H);
    L.xs = o; o += scale_bytes(s.T, s.H);
    L.aq = o; o += codes_bytes(Tk, s.I);
    L.as = o; o += scale_bytes(Tk, s.I);
  }
  L.total = o;
  return L;
}

struct BwdLayout {
  size_t queues;   // int32: tile queues, then the split plans, of the weight-gradient GEMMs
  size_t partial;  // fp32 partial tiles of split weight-gradient items
  size_t dh13, dwpart, dxrows;
  size_t dyq, dys;  // FP8 backward: dY codes [T, H], scales [T, H/32]
  size_t dhq, dhs;  // FP8 backward: [dg | du] codes [Tk, 2I], scales [Tk, 2I/32]
  // FP8 weight gradients: operands quantized along tokens (codes, scales) of
  // [dg | du], x, dY and w*silu(g)*u
  size_t wgd, wgds, wgx, wgxs, wgy, wgys, wga, wgas;
  size_t total;
};

BwdLayout bwd_layout(const moe_shape& s) {
  const int64_t Tk = s.T * s.k;
  BwdLayout L;
  size_t o = 0;
  L.queues = o; o = align_up(o + size_t(kQueueWords) * 4);
  L.partial = o; o = align_up(o + size_t(kSplitFloats) * 4);
  L.dh13 = o;   o = align_up(o + size_t(Tk) * size_t(2 * s.I) * 2);
  L.dwpart = o; o = align_up(o + size_t(Tk) * size_t(dh_num_parts(s.I)) * 4);
  L.dxrows = o; o = align_up(o + size_t(Tk) * size_t(s.H) * 2);
  L.dyq = L.dys = L.dhq = L.dhs = 0;
  if (fp8_backward(s)) {
    L.dyq = o; o += codes_bytes(s.T, s.H);
    L.dys = o; o += scale_bytes(s.T, s.H);
    L.dhq = o; o += codes_bytes(Tk, 2 * s.I);
    L.dhs = o; o += scale_bytes(Tk, 2 * s.I);
  }
  L.wgd = L.wgds = L.wgx = L.wgxs = L.wgy = L.wgys = L.wga = L.wgas = 0;
  if (fp8_wgrad(s)) {
    const int64_t K = wgrad_rows_cap(s);
    L.wgd = o; o += codes_bytes(2 * s.I, K);
    L.wgds = o; o += scale_bytes(2 * s.I, K);
    L.wgx = o; o += codes_bytes(s.H, K);
    L.wgxs = o; o += scale_bytes(s.H, K);
    L.wgy = o; o += codes_bytes(s.H, K);
    L.wgys = o; o += scale_bytes(s.H, K);
    L.wga = o; o += codes_bytes(s.I, K);
    L.wgas = o; o += scale_bytes(s.I, K);
  }
  L.total = o;
  return L;
}

// ------------------------------------------------------------ device info

struct DevInfo {
  bool checked = false;
  bool gfx950 = false;
  int cus = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

moe_status device_info(int* cus_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_LAUNCH;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_LAUNCH;
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.checked = true;
  }
  if (!d.gfx950) return MOE_ERR_ARCH;
  *cus_out = d.cus;
  return MOE_OK;
}

// ------------------------------------------------------------ kernel timing

struct EventTimer : KernelTimer {
  struct Rec {
    std::string name;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void begin(const char* name, hipStream_t st) override {
    Rec r{name, get(), get()};
    if (r.a) (void)hipEventRecord(r.a, st);
    recs.push_back(r);
  }
  void end(hipStream_t st) override {
    if (!recs.empty() && recs.back().b) (void)hipEventRecord(recs.back().b, st);
  }
};

std::mutex g_timer_mu;
bool g_timing = false;
EventTimer g_timer;

KernelTimer* timer() { return g_timing ? &g_timer : nullptr; }

moe_status launch_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}
template <class T>
const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

int effective_cus(const moe_shape& s, int dev_cus) {
  return (s.num_cus > 0 && s.num_cus < dev_cus) ? s.num_cus : dev_cus;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: shape violates H%256, I%128, 1<=k<=E or size limits";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case MOE_ERR_PRECISION: return "MOE_ERR_PRECISION: unknown precision";
    case MOE_ERR_ARCH: return "MOE_ERR_ARCH: current device is not gfx950";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than required";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: HIP launch or runtime call failed";
    case MOE_ERR_ROUTING: return "MOE_ERR_ROUTING: an expert id was outside [0, E)";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: not implemented by this library";
  }
  return "unknown moe_status";
}

moe_status moe_workspace_size(const moe_shape* s, size_t* fwd_ws, size_t* saved_bytes,
                              size_t* bwd_ws) {
  const moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (fwd_ws) *fwd_ws = fwd_layout(*s).total;
  if (saved_bytes) *saved_bytes = saved_layout(*s).total;
  if (bwd_ws) *bwd_ws = bwd_layout(*s).total;
  return MOE_OK;
}

moe_status moe_get_saved_layout(const moe_shape* s, moe_saved_layout* out) {
  const moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!out) return MOE_ERR_NULL;
  *out = saved_layout(*s);
  return MOE_OK;
}

size_t moe_permute_scratch_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return permute_scratch_bytes(s->T * s->k, int(s->E));
}

moe_status moe_permute(const moe_shape* s, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* row_of, int32_t* src_of, void* scratch,
                       void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  const int64_t Tk = s->T * s->k;
  if (!counts || !offsets || !scratch || (Tk > 0 && (!topk_idx || !row_of || !src_of)))
    return MOE_ERR_NULL;
  if (!aligned16(scratch)) return MOE_ERR_ALIGN;
  int cus = 0;
  if ((st = device_info(&cus)) != MOE_OK) return st;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  return launch_status(launch_permute(topk_idx, Tk, int(s->E), counts, offsets, row_of, src_of,
                                      scratch, static_cast<hipStream_t>(stream), timer()));
}

moe_status moe_permute_noalloc(const moe_shape* s, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                               int32_t* row_of, int32_t* src_of, int32_t* status, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  const int64_t Tk = s->T * s->k;
  if (!counts || !offsets || !status || (Tk > 0 && (!topk_idx || !row_of || !src_of))) return MOE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(status) & 3u) != 0) return MOE_ERR_ALIGN;
  // the chunk table must fit the library's fixed array
  if (int64_t(permute_num_chunks(Tk)) * (s->E + 1) > kStaticPermuteWords) return MOE_ERR_WORKSPACE;
  int cus = 0;
  if ((st = device_info(&cus)) != MOE_OK) return st;
  int32_t* table = nullptr;
  if (permute_static_scratch(&table) != hipSuccess) return MOE_ERR_LAUNCH;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  return launch_status(launch_permute_split(topk_idx, Tk, int(s->E), counts, offsets, row_of, src_of, status,
                                            table, static_cast<hipStream_t>(stream), timer()));
}

moe_status moe_get_wq_layout(const moe_shape* s, moe_wq_layout* out) {
  const moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!out) return MOE_ERR_NULL;
  *out = wq_layout(*s);
  return MOE_OK;
}

moe_status moe_quantize_weights(const moe_shape* s, const void* W13, const void* W2, void* wq,
                                void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->precision == MOE_BF16) return MOE_OK;
  if (!W13 || !W2 || !wq) return MOE_ERR_NULL;
  if (!aligned16(W13) || !aligned16(W2) || !aligned16(wq)) return MOE_ERR_ALIGN;
  int cus = 0;
  if ((st = device_info(&cus)) != MOE_OK) return st;
  const moe_wq_layout L = wq_layout(*s);
  const uint16_t* w13 = static_cast<const uint16_t*>(W13);
  const uint16_t* w2 = static_cast<const uint16_t*>(W2);
  const int H = int(s->H), I = int(s->I), rule = scale_rule(*s);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lk(g_timer_mu);
  KernelTimer* tm = timer();
  if (fp4_weights(*s)) {  // forward only: W13 along H, W2 along I
    hipError_t e = launch_quant_fp4_rows(w13, s->E * 2 * I, H, at<uint8_t>(wq, L.w13), at<uint8_t>(wq, L.w13_scale),
                                         hs, tm);
    if (e != hipSuccess) return MOE_ERR_LAUNCH;
    return launch_status(launch_quant_fp4_rows(w2, s->E * H, I, at<uint8_t>(wq, L.w2), at<uint8_t>(wq, L.w2_scale),
                                               hs, tm));
  }
  const bool fwd = fp8_forward(*s);
  hipError_t e = launch_quant_weights(w13, s->E, 2 * I, H, fwd ? at<uint8_t>(wq, L.w13) : nullptr,
                                      fwd ? at<uint8_t>(wq, L.w13_scale) : nullptr, at<uint8_t>(wq, L.w13t),
                                      at<uint8_t>(wq, L.w13t_scale), rule, hs, tm);
  if (e != hipSuccess) return MOE_ERR_LAUNCH;
  e = launch_quant_weights(w2, s->E, H, I, fwd ? at<uint8_t>(wq, L.w2) : nullptr,
                           fwd ? at<uint8_t>(wq, L.w2_scale) : nullptr, at<uint8_t>(wq, L.w2t),
                           at<uint8_t>(wq, L.w2t_scale), rule, hs, tm);
  return launch_status(e);
}

moe_status moe_quantize_rows(const moe_shape* s, const void* in, int64_t rows, int64_t K, void* codes,
                             void* scales, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->precision == MOE_BF16) return MOE_ERR_PRECISION;
  if (rows < 0 || K < 128 || K > 65536 || K % 128 != 0 || rows * K >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!in || !codes || !scales) return MOE_ERR_NULL;
  if (!aligned16(in) || !aligned16(codes)) return MOE_ERR_ALIGN;
  if (f32_scales(*s) && (reinterpret_cast<uintptr_t>(scales) & 3u) != 0) return MOE_ERR_ALIGN;
  int cus = 0;
  if ((st = device_info(&cus)) != MOE_OK) return st;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  return launch_status(launch_quant_rows(static_cast<const uint16_t*>(in), rows, int(K), static_cast<uint8_t*>(codes),
                                         static_cast<uint8_t*>(scales), act_block(*s), scale_rule(*s),
                                         static_cast<hipStream_t>(stream), timer(), "quant_rows"));
}

moe_status moe_quantize_tokens(const moe_shape* s, const void* in, int64_t ld, int64_t C, const int32_t* counts,
                               const int32_t* offsets, const int32_t* src_of, void* codes, void* scales,
                               void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->precision == MOE_BF16) return MOE_ERR_PRECISION;
  if (f32_scales(*s)) return MOE_ERR_UNSUPPORTED;  // the row-axis reading has pow2 and MX scales only
  if (C < 128 || C > 65536 || C % 128 != 0 || ld < C || ld % 8 != 0) return MOE_ERR_SHAPE;
  if (s->T * s->k >= (int64_t(1) << 23)) return MOE_ERR_SHAPE;
  if (s->T == 0) return MOE_OK;
  if (!in || !counts || !offsets || !codes || !scales) return MOE_ERR_NULL;
  if (!aligned16(in) || !aligned16(codes)) return MOE_ERR_ALIGN;
  int cus = 0;
  if ((st = device_info(&cus)) != MOE_OK) return st;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  return launch_status(launch_quant_tokens(static_cast<const uint16_t*>(in), ld, int(C), counts, offsets,
                                           int(s->E), s->T * s->k, src_of, src_of ? int(s->k) : 1,
                                           static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                                           scale_rule(*s), static_cast<hipStream_t>(stream), timer(),
                                           "quant_tokens"));
}

}  // extern "C"

namespace {

// The forward; with logits != nullptr the router runs first, fused with the
// permutation's histogram pass, and writes topk_idx and topk_w.
moe_status fwd_impl(const moe_shape* s, const void* x, const float* logits, int32_t renorm, int32_t* topk_idx,
                    float* topk_w, const void* W13, const void* W2, const void* wq, void* y, void* saved, void* ws,
                    size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->precision == MOE_BF16 && wq) return MOE_ERR_PRECISION;
  const bool f8 = fp8_forward(*s);
  const int64_t Tk = s->T * s->k;
  // the FP8 forwards read only the quantized weights
  if ((!f8 && (!W13 || !W2)) || !ws || (f8 && !wq) ||
      (s->T > 0 && (!x || !topk_idx || !topk_w || !y)))
    return MOE_ERR_NULL;
  const void* ptrs[] = {x, topk_idx, topk_w, W13, W2, y, saved, ws, wq, logits};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_ALIGN;
  const FwdLayout FL = fwd_layout(*s);
  if (ws_bytes < FL.total) return MOE_ERR_WORKSPACE;
  int cus = 0;
  if ((st = device_info(&cus)) != MOE_OK) return st;

  const moe_saved_layout SL = saved_layout(*s);
  void* sv = saved ? saved : at<char>(ws, FL.inf);
  int32_t* counts = at<int32_t>(sv, SL.counts);
  int32_t* offsets = at<int32_t>(sv, SL.offsets);
  int32_t* row_of = at<int32_t>(sv, SL.row_of);
  int32_t* src_of = at<int32_t>(sv, SL.src_of);
  float* wrow = at<float>(sv, SL.wrow);
  uint16_t* h13 = saved ? at<uint16_t>(sv, SL.h13) : nullptr;
  uint16_t* act = at<uint16_t>(sv, SL.act);
  uint16_t* rows = at<uint16_t>(ws, FL.rows);
  hipStream_t hs = static_cast<hipStream_t>(stream);

  std::lock_guard<std::mutex> lk(g_timer_mu);
  KernelTimer* tm = timer();
  int32_t* perm_status = at<int32_t>(ws, FL.perm);
  int32_t* chunk_tab = at<int32_t>(ws, FL.perm + 256);
  hipError_t e = hipSuccess;
  if (logits) {
    e = launch_route_hist(logits, s->T, int(s->E), int(s->k), renorm, topk_idx, topk_w, chunk_tab, hs, tm);
    if (e != hipSuccess) return MOE_ERR_LAUNCH;
  }
  e = launch_permute_split(topk_idx, Tk, int(s->E), counts, offsets, row_of, src_of, perm_status, chunk_tab, hs, tm,
                           topk_w, wrow, logits != nullptr);
  if (e != hipSuccess || s->T == 0) return launch_status(e);
  GemmProblem gp{s->T, s->H, s->I, s->E, s->k, effective_cus(*s, cus), counts, offsets, src_of, topk_w, wrow};
  GemmOperand gx{x, nullptr}, gw13{W13, nullptr}, ga{act, nullptr}, gw2{W2, nullptr};
  if (f8) {
    const moe_wq_layout WL = wq_layout(*s);
    const int blk = act_block(*s), rule = scale_rule(*s);
    uint8_t* xq = at<uint8_t>(ws, FL.xq);
    uint8_t* xs = at<uint8_t>(ws, FL.xs);
    if ((e = launch_quant_rows(static_cast<const uint16_t*>(x), s->T, int(s->H), xq, xs, blk, rule, hs, tm,
                               "quant_x")) != hipSuccess)
      return MOE_ERR_LAUNCH;
    const bool w4 = fp4_weights(*s), f32 = f32_scales(*s);
    gx = GemmOperand{xq, xs, false, f32};
    gw13 = GemmOperand{at<uint8_t>(wq, WL.w13), at<uint8_t>(wq, WL.w13_scale), w4, f32};
    gw2 = GemmOperand{at<uint8_t>(wq, WL.w2), at<uint8_t>(wq, WL.w2_scale), w4, f32};
  }
  if ((e = launch_gemm1_swiglu(gp, gx, gw13, h13, act, hs, tm)) != hipSuccess) return MOE_ERR_LAUNCH;
  if (f8) {
    uint8_t* aq = at<uint8_t>(ws, FL.aq);
    uint8_t* as = at<uint8_t>(ws, FL.as);
    if ((e = launch_quant_rows(act, Tk, int(s->I), aq, as, act_block(*s), scale_rule(*s), hs, tm,
                               "quant_act")) != hipSuccess)
      return MOE_ERR_LAUNCH;
    ga = GemmOperand{aq, as, false, f32_scales(*s)};
  }
  // top-1: the down GEMM writes y's rows directly; the combine only zeroes
  // the rows of dropped tokens
  const bool direct = s->k == 1;
  if ((e = launch_gemm2(gp, ga, gw2, direct ? static_cast<uint16_t*>(y) : rows, hs, tm)) != hipSuccess)
    return MOE_ERR_LAUNCH;
  e = launch_combine(direct ? nullptr : rows, row_of, s->T, int(s->k), s->H, static_cast<uint16_t*>(y), nullptr, 0,
                     nullptr, hs, tm, "combine_y");
  return launch_status(e);
}

}  // namespace

extern "C" {

moe_status moe_fwd(const moe_shape* s, const void* x, const int32_t* topk_idx,
                   const float* topk_w, const void* W13, const void* W2, const void* wq,
                   void* y, void* saved, void* ws, size_t ws_bytes, void* stream) {
  // read only: without logits fwd_impl writes neither routing buffer
  return fwd_impl(s, x, nullptr, 0, const_cast<int32_t*>(topk_idx), const_cast<float*>(topk_w), W13, W2, wq, y,
                  saved, ws, ws_bytes, stream);
}

moe_status moe_fwd_logits(const moe_shape* s, const void* x, const float* logits, int32_t renorm,
                          int32_t* topk_idx, float* topk_w, const void* W13, const void* W2, const void* wq,
                          void* y, void* saved, void* ws, size_t ws_bytes, void* stream) {
  if (s && s->T > 0 && !logits) return MOE_ERR_NULL;
  return fwd_impl(s, x, s && s->T > 0 ? logits : nullptr, renorm, topk_idx, topk_w, W13, W2, wq, y, saved, ws,
                  ws_bytes, stream);
}

moe_status moe_bwd(const moe_shape* s, const void* dy, const void* x, const int32_t* topk_idx,
                   const float* topk_w, const void* W13, const void* W2, const void* wq,
                   const void* saved, void* dx, float* d_topk_w, void* dW13, void* dW2, void* ws,
                   size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->precision == MOE_BF16 && wq) return MOE_ERR_PRECISION;
  if (s->precision == MOE_FP8_FP4) return MOE_ERR_PRECISION;  // an inference forward: no backward
  const bool f8 = fp8_backward(*s);
  (void)topk_idx;  // the permutation comes from `saved`
  // the FP8 backwards read only the quantized weights
  if ((!f8 && (!W13 || !W2)) || !saved || !dW13 || !dW2 || !ws || (f8 && !wq) ||
      (s->T > 0 && (!dy || !x || !topk_w || !dx || !d_topk_w)))
    return MOE_ERR_NULL;
  const void* ptrs[] = {dy, x, topk_idx, topk_w, W13, W2, saved, dx, d_topk_w, dW13, dW2, ws, wq};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_ALIGN;
  const BwdLayout BL = bwd_layout(*s);
  if (ws_bytes < BL.total) return MOE_ERR_WORKSPACE;
  int cus = 0;
  if ((st = device_info(&cus)) != MOE_OK) return st;

  const moe_saved_layout SL = saved_layout(*s);
  const int32_t* counts = at<int32_t>(saved, SL.counts);
  const int32_t* offsets = at<int32_t>(saved, SL.offsets);
  const int32_t* row_of = at<int32_t>(saved, SL.row_of);
  const int32_t* src_of = at<int32_t>(saved, SL.src_of);
  const float* wrow = at<float>(saved, SL.wrow);
  const uint16_t* h13 = at<uint16_t>(saved, SL.h13);
  const uint16_t* act = at<uint16_t>(saved, SL.act);
  uint16_t* dh13 = at<uint16_t>(ws, BL.dh13);
  float* dwpart = at<float>(ws, BL.dwpart);
  uint16_t* dxrows = at<uint16_t>(ws, BL.dxrows);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const uint16_t* dy16 = static_cast<const uint16_t*>(dy);
  const uint16_t* x16 = static_cast<const uint16_t*>(x);

  std::lock_guard<std::mutex> lk(g_timer_mu);
  KernelTimer* tm = timer();
  GemmProblem gp{s->T, s->H, s->I, s->E, s->k, effective_cus(*s, cus), counts, offsets, src_of, topk_w, wrow};
  int32_t* queues = at<int32_t>(ws, BL.queues);
  int32_t* plan13 = queues + kNumQueues;  // split plans of the two weight-gradient GEMMs
  int32_t* plan2 = plan13 + kSplitWords;
  float* partial = at<float>(ws, BL.partial);
  hipError_t e = launch_zero_queues(queues, hs, tm);
  if (e != hipSuccess) return MOE_ERR_LAUNCH;
  const bool wg8 = fp8_wgrad(*s);
  const int64_t Tk = s->T * s->k;
  const int I = int(s->I), H = int(s->H), E = int(s->E), kk = int(s->k), rule = scale_rule(*s);
  if (s->T > 0) {
    GemmOperand gdy{dy, nullptr}, gw2{W2, nullptr}, gdh{dh13, nullptr}, gw13{W13, nullptr};
    if (f8) {
      const moe_wq_layout WL = wq_layout(*s);
      uint8_t* dyq = at<uint8_t>(ws, BL.dyq);
      uint8_t* dys = at<uint8_t>(ws, BL.dys);
      if (wg8 && kk == 1) {
        // each token row occurs once among the expert rows: one pass gives
        // dY's codes along H (for dH) and along the expert rows (for dW2)
        e = launch_quant_tokens(dy16, H, H, counts, offsets, E, Tk, src_of, kk, at<uint8_t>(ws, BL.wgy),
                                at<uint8_t>(ws, BL.wgys), rule, hs, tm, "quant_wg_dy", dyq, dys);
      } else {
        e = launch_quant_rows(dy16, s->T, H, dyq, dys, act_block(*s), rule, hs, tm, "quant_dy");
      }
      if (e != hipSuccess) return MOE_ERR_LAUNCH;
      const bool f32 = f32_scales(*s);
      gdy = GemmOperand{dyq, dys, false, f32};
      gw2 = GemmOperand{at<uint8_t>(wq, WL.w2t), at<uint8_t>(wq, WL.w2t_scale), false, f32};
      gw13 = GemmOperand{at<uint8_t>(wq, WL.w13t), at<uint8_t>(wq, WL.w13t_scale), false, f32};
    }
    if ((e = launch_gemm_dh(gp, gdy, gw2, h13, dh13, dwpart, hs, tm)) != hipSuccess) return MOE_ERR_LAUNCH;
    if (f8) {
      uint8_t* dhq = at<uint8_t>(ws, BL.dhq);
      uint8_t* dhs = at<uint8_t>(ws, BL.dhs);
      if (wg8)  // [dg | du] along 2I (for dX) and along the expert rows (for dW13) in one pass
        e = launch_quant_tokens(dh13, 2 * I, 2 * I, counts, offsets, E, Tk, nullptr, 1, at<uint8_t>(ws, BL.wgd),
                                at<uint8_t>(ws, BL.wgds), rule, hs, tm, "quant_wg_dh13", dhq, dhs);
      else
        e = launch_quant_rows(dh13, Tk, 2 * I, dhq, dhs, act_block(*s), rule, hs, tm, "quant_dh13");
      if (e != hipSuccess) return MOE_ERR_LAUNCH;
      gdh = GemmOperand{dhq, dhs, false, f32_scales(*s)};
    }
    const bool direct = s->k == 1;  // top-1: dX rows go straight to dx
    if ((e = launch_gemm_dx(gp, gdh, gw13, direct ? static_cast<uint16_t*>(dx) : dxrows, hs, tm)) != hipSuccess)
      return MOE_ERR_LAUNCH;
    if ((e = launch_combine(direct ? nullptr : dxrows, row_of, s->T, int(s->k), s->H, static_cast<uint16_t*>(dx), dwpart,
                            dh_num_parts(s->I), d_topk_w, hs, tm, "combine_dx_dw")) != hipSuccess)
      return MOE_ERR_LAUNCH;
  }
  if (wg8) {
    // [dg | du] (and, for top-1, dY) were quantized along the expert rows
    // above; with no tokens every expert is empty and no operand is read
    uint8_t* wgd = at<uint8_t>(ws, BL.wgd);
    uint8_t* wgds = at<uint8_t>(ws, BL.wgds);
    uint8_t* wgx = at<uint8_t>(ws, BL.wgx);
    uint8_t* wgxs = at<uint8_t>(ws, BL.wgxs);
    uint8_t* wgy = at<uint8_t>(ws, BL.wgy);
    uint8_t* wgys = at<uint8_t>(ws, BL.wgys);
    uint8_t* wga = at<uint8_t>(ws, BL.wga);
    uint8_t* wgas = at<uint8_t>(ws, BL.wgas);
    if ((e = launch_quant_tokens(x16, H, H, counts, offsets, E, Tk, src_of, kk, wgx, wgxs, rule, hs, tm,
                                 "quant_wg_x")) != hipSuccess ||
        (e = launch_gemm_dw_fp8(gp, wgd, wgds, 2 * I, wgx, wgxs, H, static_cast<uint16_t*>(dW13), queues, partial,
                                plan13, hs, tm, "gemm_dw13_fp8", "dw13_split_sum")) != hipSuccess)
      return MOE_ERR_LAUNCH;
    if (kk != 1 && (e = launch_quant_tokens(dy16, H, H, counts, offsets, E, Tk, src_of, kk, wgy, wgys, rule, hs,
                                            tm, "quant_wg_dy")) != hipSuccess)
      return MOE_ERR_LAUNCH;
    if ((e = launch_quant_tokens(act, I, I, counts, offsets, E, Tk, nullptr, 1, wga, wgas, rule, hs, tm,
                                 "quant_wg_act")) != hipSuccess)
      return MOE_ERR_LAUNCH;
    e = launch_gemm_dw_fp8(gp, wgy, wgys, H, wga, wgas, I, static_cast<uint16_t*>(dW2), queues + kQueuesPerGemm, partial,
                           plan2, hs, tm, "gemm_dw2_fp8", "dw2_split_sum");
    return launch_status(e);
  }
  if ((e = launch_gemm_dw13(gp, dh13, x16, static_cast<uint16_t*>(dW13), queues, partial, plan13, hs, tm)) !=
      hipSuccess)
    return MOE_ERR_LAUNCH;
  e = launch_gemm_dw2(gp, dy16, act, static_cast<uint16_t*>(dW2), queues + kQueuesPerGemm, partial, plan2, hs, tm);
  return launch_status(e);
}

moe_status moe_route(const moe_shape* s, const float* logits, int32_t renorm, int32_t* topk_idx, float* topk_w,
                     void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_NULL;
  int cus = 0;
  if ((st = device_info(&cus)) != MOE_OK) return st;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  return launch_status(launch_route(logits, s->T, int(s->E), int(s->k), renorm != 0, topk_idx, topk_w,
                                    static_cast<hipStream_t>(stream), timer()));
}

moe_status moe_route_bwd(const moe_shape* s, const float* logits, const int32_t* topk_idx, const float* topk_w,
                         const float* d_topk_w, int32_t renorm, float* d_logits, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w || !d_topk_w || !d_logits) return MOE_ERR_NULL;
  int cus = 0;
  if ((st = device_info(&cus)) != MOE_OK) return st;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  return launch_status(launch_route_bwd(logits, s->T, int(s->E), int(s->k), renorm != 0, topk_idx, topk_w, d_topk_w,
                                        d_logits, static_cast<hipStream_t>(stream), timer()));
}

moe_status moe_read_status(const void* fwd_ws, int32_t* out, void* stream) {
  if (!fwd_ws || !out) return MOE_ERR_NULL;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(out, fwd_ws, sizeof(int32_t), hipMemcpyDeviceToHost, hs) != hipSuccess)
    return MOE_ERR_LAUNCH;
  if (hipStreamSynchronize(hs) != hipSuccess) return MOE_ERR_LAUNCH;
  return MOE_OK;
}

moe_status moe_set_kernel_timing(int enable) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  g_timing = enable != 0;
  return MOE_OK;
}

moe_status moe_kernel_timing_collect(moe_kernel_time* out, int32_t max, int32_t* n_out) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  std::vector<moe_kernel_time> agg;
  moe_status st = MOE_OK;
  for (auto& r : g_timer.recs) {
    float ms = 0.f;
    if (!r.a || !r.b || hipEventSynchronize(r.b) != hipSuccess ||
        hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = MOE_ERR_LAUNCH;
    }
    size_t i = 0;
    for (; i < agg.size(); ++i)
      if (r.name == agg[i].name) break;
    if (i == agg.size()) {
      moe_kernel_time kt;
      std::memset(&kt, 0, sizeof(kt));
      std::strncpy(kt.name, r.name.c_str(), sizeof(kt.name) - 1);
      agg.push_back(kt);
    }
    agg[i].launches += 1;
    agg[i].total_ms += ms;
    if (r.a) g_timer.pool.push_back(r.a);
    if (r.b) g_timer.pool.push_back(r.b);
  }
  g_timer.recs.clear();
  int32_t n = 0;
  for (size_t i = 0; i < agg.size() && n < max; ++i) out[n++] = agg[i];
  if (n_out) *n_out = n;
  return st;
}

}  // extern "C"
