// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_host_sanitizers.py with the
// sanitizers on the host code only). Every call here is refused, or answered,
// before any device work: shape and precision checks, NULL and alignment
// checks, workspace sizes, layouts, status strings and the empty timing record.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/moe.h"

static int g_fail = 0;
#define EXPECT(cond)                                               \
  do {                                                             \
    if (!(cond)) {                                                 \
      std::fprintf(stderr, "FAILED %s:%d %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                    \
    }                                                              \
  } while (0)

static moe_shape shape(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int prec = MOE_BF16, int flags = 0) {
  moe_shape s;
  std::memset(&s, 0, sizeof(s));
  s.T = T; s.H = H; s.I = I; s.E = E; s.k = k;
  s.precision = prec;
  s.flags = flags;
  return s;
}

int main() {
  void* const P = reinterpret_cast<void*>(uintptr_t(1) << 20);  // aligned stand-in, never dereferenced
  void* const Q = reinterpret_cast<void*>((uintptr_t(1) << 20) + 8);  // misaligned stand-in
  for (int p = MOE_BF16; p <= MOE_FP8_BWD_F32; ++p) {
    moe_shape s = shape(16384, 2048, 768, 128, 8, p);
    size_t f = 0, sv = 0, b = 0;
    EXPECT(moe_workspace_size(&s, &f, &sv, &b) == MOE_OK);
    EXPECT(f > 0 && sv > 0 && b > 0);
    moe_saved_layout sl;
    EXPECT(moe_get_saved_layout(&s, &sl) == MOE_OK && sl.total == sv);
    moe_wq_layout wl;
    EXPECT(moe_get_wq_layout(&s, &wl) == MOE_OK);
    EXPECT(moe_permute_scratch_bytes(&s) > 256);
    // NULL weights / workspace, misaligned tensors, small workspaces
    EXPECT(moe_fwd(&s, P, (const int32_t*)P, (const float*)P, P, P, p == MOE_BF16 ? nullptr : P, P, P, nullptr, 1u << 30,
                   nullptr) == MOE_ERR_NULL);
    EXPECT(moe_fwd(&s, Q, (const int32_t*)P, (const float*)P, P, P, p == MOE_BF16 ? nullptr : P, P, P, P, f, nullptr) ==
           MOE_ERR_ALIGN);
    EXPECT(moe_fwd(&s, P, (const int32_t*)P, (const float*)P, P, P, p == MOE_BF16 ? nullptr : P, P, P, P, f - 1,
                   nullptr) == MOE_ERR_WORKSPACE);
    EXPECT(moe_fwd_logits(&s, P, nullptr, 1, (int32_t*)P, (float*)P, P, P, p == MOE_BF16 ? nullptr : P, P, P, P, f,
                          nullptr) == MOE_ERR_NULL);
    if (p != MOE_FP8_FP4) {
      EXPECT(moe_bwd(&s, P, P, (const int32_t*)P, (const float*)P, P, P, p == MOE_BF16 ? nullptr : P, nullptr, P,
                     (float*)P, P, P, P, b, nullptr) == MOE_ERR_NULL);
      EXPECT(moe_bwd(&s, P, P, (const int32_t*)P, (const float*)P, P, P, p == MOE_BF16 ? nullptr : P, P, P, (float*)P,
                     P, P, P, b - 1, nullptr) == MOE_ERR_WORKSPACE);
    } else {
      EXPECT(moe_bwd(&s, P, P, (const int32_t*)P, (const float*)P, P, P, P, P, P, (float*)P, P, P, P, b, nullptr) ==
             MOE_ERR_PRECISION);
    }
    if (p == MOE_BF16) {
      EXPECT(moe_quantize_rows(&s, P, 4, 256, P, P, nullptr) == MOE_ERR_PRECISION);
      EXPECT(moe_fwd(&s, P, (const int32_t*)P, (const float*)P, P, P, P, P, P, P, f, nullptr) == MOE_ERR_PRECISION);
    } else {
      EXPECT(moe_quantize_rows(&s, P, 4, 100, P, P, nullptr) == MOE_ERR_SHAPE);
      EXPECT(moe_quantize_rows(&s, Q, 4, 256, P, P, nullptr) == MOE_ERR_ALIGN);
    }
  }
  // shapes outside the limits, unknown precisions and flags
  const int64_t bad[][5] = {{16384, 2048, 768, 128, 0}, {16384, 2048, 768, 128, 129}, {16384, 2000, 768, 128, 8},
                            {16384, 2048, 700, 128, 8}, {-1, 2048, 768, 128, 8},      {1 << 28, 2048, 768, 128, 8},
                            {16384, 2048, 768, 2000, 8}, {1 << 20, 4096, 768, 128, 1}};
  for (const auto& d : bad) {
    moe_shape s = shape(d[0], d[1], d[2], d[3], d[4]);
    EXPECT(moe_workspace_size(&s, nullptr, nullptr, nullptr) == MOE_ERR_SHAPE);
  }
  moe_shape s = shape(16384, 2048, 768, 128, 8, 7);
  EXPECT(moe_workspace_size(&s, nullptr, nullptr, nullptr) == MOE_ERR_PRECISION);
  s = shape(16384, 2048, 768, 128, 8, MOE_FP8_BLOCK, 2);
  EXPECT(moe_workspace_size(&s, nullptr, nullptr, nullptr) == MOE_ERR_PRECISION);
  s = shape(16384, 2048, 768, 128, 8, MOE_FP8_BLOCK_F32, MOE_FLAG_FP8_WGRAD);
  EXPECT(moe_workspace_size(&s, nullptr, nullptr, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_workspace_size(nullptr, nullptr, nullptr, nullptr) == MOE_ERR_NULL);
  // the allocation-free permutation past its table limit
  s = shape((1 << 20) / 8 + 1024, 256, 128, 1024, 8);
  EXPECT(moe_permute_noalloc(&s, (const int32_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P,
                             nullptr) == MOE_ERR_WORKSPACE);
  EXPECT(moe_permute(&s, (const int32_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, Q, nullptr) ==
         MOE_ERR_ALIGN);
  // status strings and the empty timing record
  for (int st = 0; st <= 10; ++st) EXPECT(moe_status_string(moe_status(st)) != nullptr);
  std::vector<moe_kernel_time> kt(4);
  int32_t n = -1;
  EXPECT(moe_set_kernel_timing(0) == MOE_OK);
  EXPECT(moe_kernel_timing_collect(kt.data(), 4, &n) == MOE_OK && n == 0);
  EXPECT(moe_read_status(nullptr, &n, nullptr) == MOE_ERR_NULL);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("abi host checks passed\n");
  return 0;
}
