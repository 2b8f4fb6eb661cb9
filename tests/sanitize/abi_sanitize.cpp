// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every call below fails validation (or only
// sizes a workspace) before any HIP call, so the library's host code is
// exercised with no GPU.  Built from the library sources (host side only)
// by tests/test_abi_sanitize.py; exits nonzero on the first mismatch.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/lq.h"

static int failures = 0;
#define EXPECT(call, code)                                                              \
  do {                                                                                  \
    const lq_status st_ = (call);                                                       \
    if (st_ != (code)) {                                                                \
      std::fprintf(stderr, "%s:%d %s -> %d, expected %d (%s)\n", __FILE__, __LINE__,    \
                   #call, st_, (code), lq_last_error());                                \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

int main() {
  // fake device addresses, never dereferenced
  void* P = reinterpret_cast<void*>(uintptr_t{0x10000000});
  void* MIS = reinterpret_cast<void*>(uintptr_t{0x10000002});
  const uint32_t* W = static_cast<const uint32_t*>(P);
  const float* F = static_cast<const float*>(P);
  float* O = static_cast<float*>(P);
  for (int c = -1; c < 10; ++c)
    if (std::strlen(lq_status_string(c)) == 0) ++failures;
  // lq_gemv and lq_gemv_noalloc
  EXPECT(lq_gemv(nullptr, 8, 64, 4, F, F, 1, O, nullptr, 0, nullptr), LQ_ERR_NULL);
  EXPECT(lq_gemv(W, 8, 64, 4, F, F, 0, O, nullptr, 0, nullptr), LQ_ERR_SHAPE);
  EXPECT(lq_gemv(W, 8, 64, 4, F, F, 17, O, nullptr, 0, nullptr), LQ_ERR_SHAPE);
  EXPECT(lq_gemv(W, 8, 64, 1, F, F, 1, O, nullptr, 0, nullptr), LQ_ERR_SHAPE);
  EXPECT(lq_gemv(W, 8, 96, 3, F, F, 1, O, nullptr, 0, nullptr), LQ_ERR_ALIGN);
  EXPECT(lq_gemv(W, 8, 66, 4, F, F, 1, O, nullptr, 0, nullptr), LQ_ERR_SHAPE);
  EXPECT(lq_gemv(static_cast<const uint32_t*>(MIS), 8, 64, 4, F, F, 1, O, nullptr, 0, nullptr),
         LQ_ERR_ALIGN);
  EXPECT(lq_gemv(W, int64_t{1} << 40, 64, 4, F, F, 1, O, nullptr, 0, nullptr), LQ_ERR_SHAPE);
  EXPECT(lq_gemv(W, 8, int64_t{1} << 40, int64_t{1} << 35, F, F, 1, O, nullptr, 0, nullptr),
         LQ_ERR_SHAPE);
  EXPECT(lq_gemv(W, 8192, 68096, 2128, F, F, 1, O, nullptr, 0, nullptr), LQ_ERR_WORKSPACE);
  EXPECT(lq_gemv_noalloc(W, 4096, 1 << 21, 1 << 16, F, F, 1, O, nullptr), LQ_ERR_WORKSPACE);
  EXPECT(lq_gemv_noalloc(nullptr, 8, 64, 4, F, F, 1, O, nullptr), LQ_ERR_NULL);
  size_t n = 0;
  for (int64_t B = 1; B <= 16; ++B) {
    EXPECT(lq_gemv_workspace_size(28672, 19456, B, &n), LQ_OK);
    EXPECT(lq_gemv_workspace_size(8192, 68096, B, &n), LQ_OK);
    EXPECT(lq_gemv_workspace_size(1, 4, B, &n), LQ_OK);
    EXPECT(lq_gemv_workspace_size(4096, int64_t{1} << 24, B, &n), LQ_OK);
  }
  EXPECT(lq_gemv_workspace_size(8, 64, 0, &n), LQ_ERR_SHAPE);
  EXPECT(lq_gemv_workspace_size(8, 64, 1, nullptr), LQ_ERR_NULL);
  // lift, Kronecker lift, layer, GEMM, decode-weights product
  EXPECT(lq_lift_activations(P, LQ_BF16, 1, 100, P, LQ_BF16, 128, F, 8, 19, P, LQ_F32, nullptr),
         LQ_ERR_SHAPE);
  EXPECT(lq_lift_activations(P, 7, 1, 1024, P, LQ_BF16, 128, F, 8, 19, P, LQ_F32, nullptr),
         LQ_ERR_DTYPE);
  EXPECT(lq_lift_activations(P, LQ_BF16, 1, 1024, P, LQ_BF16, 64, F, 8, 19, P, LQ_F32, nullptr),
         LQ_ERR_UNSUPPORTED);
  EXPECT(lq_lift_kron_workspace_size(512, 8192, &n), LQ_OK);
  EXPECT(lq_lift_kron(P, LQ_BF16, 1, 8192, 63, F, F, F, F, F, 16, 40, P, LQ_F32, P, n, nullptr),
         LQ_ERR_SHAPE);
  EXPECT(lq_layer_b1_workspace_size(28672, 8192, 8, 19, &n), LQ_OK);
  EXPECT(lq_layer_b1(P, LQ_BF16, 8192, P, LQ_F16, 128, F, 8, 19, W, 28672, 640, F, O, P, n,
                     nullptr),
         LQ_ERR_DTYPE);
  EXPECT(lq_gemm(W, 8192, 20480, 640, F, P, LQ_F32, 512, O, nullptr), LQ_ERR_DTYPE);
  EXPECT(lq_gemm(W, 8192, (int64_t{1} << 22) + 8, 1 << 17, F, P, LQ_F16, 512, O, nullptr),
         LQ_ERR_SHAPE);
  EXPECT(lq_gemm_decoded_workspace_size(8192, 8192, &n), LQ_OK);
  EXPECT(lq_gemm_decoded(W, 8192, 8192, 640, F, 16, 40, F, P, LQ_BF16, 512, O, P, n, nullptr),
         LQ_ERR_DTYPE);
  EXPECT(lq_encode_workspace_size(16, 40, &n), LQ_ERR_SHAPE);
  EXPECT(lq_softmin_workspace_size(4096, 8, 16, &n), LQ_OK);
  EXPECT(lq_adam_update(O, F, O, O, 16, 0, 0.01f, 0.9f, 0.999f, 1e-8f, nullptr), LQ_ERR_SHAPE);
  EXPECT(lq_pack_signs(static_cast<const int8_t*>(P), 4, 64, 32, static_cast<uint32_t*>(P), 2,
                       nullptr),
         LQ_ERR_SHAPE);
  EXPECT(lq_stream_read(P, 100, static_cast<uint32_t*>(P), nullptr), LQ_ERR_SHAPE);
  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("abi sanitize: all checks passed\n");
  return 0;
}
