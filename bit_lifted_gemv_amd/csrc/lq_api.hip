// C ABI of liblq: host-side validation and dispatch (declarations in include/lq.h).
// Every entry point checks its arguments before launching anything, returns a
// status code and records a thread-local message on failure.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "lq_internal.h"

namespace {

thread_local char g_err[512] = "";

lq_status fail(lq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

lq_status ok() {
  g_err[0] = '\0';
  return LQ_OK;
}

lq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

bool valid_dtype(lq_dtype dt) { return dt == LQ_F32 || dt == LQ_F16 || dt == LQ_BF16; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

size_t dtype_size(lq_dtype dt) { return dt == LQ_F32 ? 4 : 2; }

// lq_gemm addresses a 128-row or 128-token block with 32-bit buffer offsets
constexpr int64_t kGemmMaxK = int64_t{1} << 22;

// lq_gemv kernels: one to five tokens in one launch on the float4-sign /
// float8-part matrix cores when a workgroup's LDS holds its sums (no
// workspace), otherwise on the slice-major float8-part kernel and its slice
// reduction; six to sixteen on the float8-part kernel with the parts as
// column blocks (preparation, product over splits of K, reduction).  (The
// float16 activation-sum table kernel serves lq_layer_b1.)
enum class GemvPath { kRows, kF4, kF4m };
GemvPath gemv_path(int64_t m, int64_t K, int64_t B) {
  if (lq::gemv_f4r_applies(m, K, B)) return GemvPath::kRows;
  return B <= 5 ? GemvPath::kF4 : GemvPath::kF4m;
}
size_t gemv_workspace(int64_t m, int64_t K, int64_t B) {
  switch (gemv_path(m, K, B)) {
    case GemvPath::kRows: return 0;
    case GemvPath::kF4: return lq::gemv_f4_workspace_bytes(m, K, B);
    default: return lq::gemv_f4m_workspace_bytes(m, K, B);
  }
}

// Shape, pointer and alignment checks shared by lq_gemv and lq_gemv_noalloc.
lq_status gemv_check(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw, const float* s,
                     const float* a_lift, int64_t B, float* out) {
  if (!w_packed || !s || !a_lift || !out) return fail(LQ_ERR_NULL, "null pointer");
  if (m < 1 || K < 1) return fail(LQ_ERR_SHAPE, "m=%lld K=%lld", (long long)m, (long long)K);
  if (B < 1 || B > 16) return fail(LQ_ERR_SHAPE, "B=%lld outside 1..16", (long long)B);
  if (ldw < (K + 31) / 32) return fail(LQ_ERR_SHAPE, "ldw=%lld < ceil(K/32)", (long long)ldw);
  if (ldw % 4) return fail(LQ_ERR_ALIGN, "ldw=%lld must be a multiple of 4", (long long)ldw);
  if (K % 4) return fail(LQ_ERR_SHAPE, "K=%lld must be a multiple of 4", (long long)K);
  // the kernels address weights and activations with 32-bit buffer offsets
  if (m * ldw * 4 > ((int64_t)1 << 30))
    return fail(LQ_ERR_SHAPE, "weights of %lld bytes exceed the 1 GiB per-call limit",
                (long long)(m * ldw * 4));
  if (K > ((int64_t)1 << 24))
    return fail(LQ_ERR_SHAPE, "K=%lld exceeds the per-call limit of 2^24", (long long)K);
  if (!aligned(w_packed, 16)) return fail(LQ_ERR_ALIGN, "w_packed must be 16-byte aligned");
  if (!aligned(a_lift, 16)) return fail(LQ_ERR_ALIGN, "a_lift must be 16-byte aligned");
  if (!aligned(s, 4) || !aligned(out, 4)) return fail(LQ_ERR_ALIGN, "misaligned s or out");
  return LQ_OK;
}

lq_status gemv_launch(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw, const float* s,
                      const float* a_lift, int64_t B, float* out, void* ws, hipStream_t st) {
  switch (gemv_path(m, K, B)) {
    case GemvPath::kRows:
      return hip_status(lq::launch_gemv_f4r(w_packed, m, K, ldw, s, a_lift, B, out, st),
                        "lq_gemv launch");
    case GemvPath::kF4:
      return hip_status(lq::launch_gemv_f4(w_packed, m, K, ldw, s, a_lift, B, out, ws, st),
                        "lq_gemv launch");
    default:
      return hip_status(lq::launch_gemv_f4m(w_packed, m, K, ldw, s, a_lift, B, out, ws, st),
                        "lq_gemv launch");
  }
}

// Scratch of lq_gemv_noalloc: one array per GPU, in the code object, held
// until the process ends.  Host code never uses the array's name as an
// address: its device address is looked up once per device (with that
// device current) and kept.  Every lq_gemv_noalloc call on a GPU shares it.
constexpr size_t kScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_pointer(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* lq_status_string(lq_status st) {
  switch (st) {
    case LQ_OK: return "LQ_OK";
    case LQ_ERR_NULL: return "LQ_ERR_NULL";
    case LQ_ERR_SHAPE: return "LQ_ERR_SHAPE";
    case LQ_ERR_DTYPE: return "LQ_ERR_DTYPE";
    case LQ_ERR_ALIGN: return "LQ_ERR_ALIGN";
    case LQ_ERR_UNSUPPORTED: return "LQ_ERR_UNSUPPORTED";
    case LQ_ERR_HIP: return "LQ_ERR_HIP";
    case LQ_ERR_WORKSPACE: return "LQ_ERR_WORKSPACE";
    default: return "LQ_ERR_UNKNOWN";
  }
}

const char* lq_last_error(void) { return g_err; }

const char* lq_version(void) { return "liblq 0.1 gfx950"; }

lq_status lq_pack_signs(const int8_t* signs, int64_t rows, int64_t K, int64_t lds,
                        uint32_t* packed, int64_t ldw, void* stream) {
  if (rows < 0 || K < 0 || ldw < 0 || lds < 0)
    return fail(LQ_ERR_SHAPE, "negative size (rows=%lld K=%lld lds=%lld ldw=%lld)",
                (long long)rows, (long long)K, (long long)lds, (long long)ldw);
  if (ldw < (K + 31) / 32) return fail(LQ_ERR_SHAPE, "ldw=%lld < ceil(K/32)", (long long)ldw);
  if (lds < K) return fail(LQ_ERR_SHAPE, "lds=%lld < K=%lld", (long long)lds, (long long)K);
  if (rows == 0 || ldw == 0) return ok();
  if (!packed || (K > 0 && !signs)) return fail(LQ_ERR_NULL, "null pointer");
  if (!aligned(packed, 4)) return fail(LQ_ERR_ALIGN, "packed must be 4-byte aligned");
  return hip_status(lq::launch_pack_signs(signs, rows, K, lds, packed, ldw, as_stream(stream)),
                    "lq_pack_signs launch");
}

lq_status lq_unpack_signs(const uint32_t* packed, int64_t rows, int64_t K, int64_t ldw,
                          int8_t* signs, int64_t lds, void* stream) {
  if (rows < 0 || K < 0 || ldw < 0 || lds < 0) return fail(LQ_ERR_SHAPE, "negative size");
  if (ldw < (K + 31) / 32) return fail(LQ_ERR_SHAPE, "ldw=%lld < ceil(K/32)", (long long)ldw);
  if (lds < K) return fail(LQ_ERR_SHAPE, "lds=%lld < K=%lld", (long long)lds, (long long)K);
  if (rows == 0 || K == 0) return ok();
  if (!packed || !signs) return fail(LQ_ERR_NULL, "null pointer");
  if (!aligned(packed, 4)) return fail(LQ_ERR_ALIGN, "packed must be 4-byte aligned");
  return hip_status(lq::launch_unpack_signs(packed, rows, K, ldw, signs, lds, as_stream(stream)),
                    "lq_unpack_signs launch");
}

lq_status lq_lift_activations(const void* a, lq_dtype a_dtype, int64_t B, int64_t n,
                              const void* t_inv, lq_dtype t_dtype, int32_t t_block,
                              const float* M, int32_t d, int32_t D, void* a_lift,
                              lq_dtype lift_dtype, void* stream) {
  if (!a || !t_inv || !M || !a_lift) return fail(LQ_ERR_NULL, "null pointer");
  if (!valid_dtype(a_dtype) || !valid_dtype(t_dtype) || !valid_dtype(lift_dtype))
    return fail(LQ_ERR_DTYPE, "unknown dtype");
  if (t_block != 128)
    return fail(LQ_ERR_UNSUPPORTED, "t_block=%d (only 128 is implemented)", (int)t_block);
  if (B < 1 || n < 1) return fail(LQ_ERR_SHAPE, "B=%lld n=%lld", (long long)B, (long long)n);
  if (d < 1 || d > 64 || D < 1 || D > 256 || d * D > 8192)
    return fail(LQ_ERR_SHAPE, "d=%d D=%d out of range (1..64, 1..256, d*D <= 8192)", (int)d,
                (int)D);
  if (n % 128) return fail(LQ_ERR_SHAPE, "n=%lld not a multiple of t_block", (long long)n);
  if (n % d) return fail(LQ_ERR_SHAPE, "n=%lld not a multiple of d=%d", (long long)n, (int)d);
  if ((int64_t)n / d * D > INT32_MAX || n > INT32_MAX || B > INT32_MAX / 2)
    return fail(LQ_ERR_SHAPE, "sizes exceed 32-bit indexing");
  if (!aligned(t_inv, 16) || !aligned(a, 16))
    return fail(LQ_ERR_ALIGN, "t_inv and a must be 16-byte aligned");
  if (!aligned(a_lift, dtype_size(lift_dtype)) || !aligned(M, 4))
    return fail(LQ_ERR_ALIGN, "misaligned pointer");
  return hip_status(lq::launch_lift(a, a_dtype, B, n, t_inv, t_dtype, M, d, D, a_lift, lift_dtype,
                                    as_stream(stream)),
                    "lq_lift_activations launch");
}

lq_status lq_lift_kron_workspace_size(int64_t B, int64_t n, size_t* bytes) {
  if (!bytes) return fail(LQ_ERR_NULL, "bytes is null");
  if (B < 1 || n < 1) return fail(LQ_ERR_SHAPE, "B=%lld n=%lld", (long long)B, (long long)n);
  *bytes = lq::lift_kron_workspace_bytes(B, n);
  return ok();
}

lq_status lq_lift_kron(const void* a, lq_dtype a_dtype, int64_t B, int64_t n, int32_t n1,
                       const float* s1, const float* p1_inv, const float* p2_inv,
                       const float* s2, const float* M, int32_t d, int32_t D, void* a_lift,
                       lq_dtype lift_dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!a || !s1 || !p1_inv || !p2_inv || !s2 || !M || !a_lift || !workspace)
    return fail(LQ_ERR_NULL, "null pointer");
  if (!valid_dtype(a_dtype) || !valid_dtype(lift_dtype)) return fail(LQ_ERR_DTYPE, "unknown dtype");
  if (B < 1 || n < 1) return fail(LQ_ERR_SHAPE, "B=%lld n=%lld", (long long)B, (long long)n);
  if (d < 1 || d > 64 || D < 1 || D > 256 || d * D > 8192)
    return fail(LQ_ERR_SHAPE, "d=%d D=%d out of range (1..64, 1..256, d*D <= 8192)", (int)d,
                (int)D);
  if (n > INT32_MAX || B > 65535 || (int64_t)n / d * D > INT32_MAX)
    return fail(LQ_ERR_SHAPE, "B=%lld (<= 65535) or n exceed the launch limits", (long long)B);
  if (n1 < 1 || n % n1 || n % d)
    return fail(LQ_ERR_SHAPE, "n=%lld must be a multiple of n1=%d and d=%d", (long long)n, (int)n1,
                (int)d);
  if (!lq::lift_kron_shape_ok(n, n1, d, D))
    return fail(LQ_ERR_UNSUPPORTED,
                "n1=%d n2=%lld d=%d D=%d: needs n1 <= 256, n2 <= 128, n2 %% d == 0 and the "
                "column tile in LDS", (int)n1, (long long)(n / n1), (int)d, (int)D);
  if (workspace_bytes < lq::lift_kron_workspace_bytes(B, n))
    return fail(LQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes,
                lq::lift_kron_workspace_bytes(B, n));
  if (!aligned(workspace, 256)) return fail(LQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(a, dtype_size(a_dtype)) || !aligned(a_lift, dtype_size(lift_dtype)) ||
      !aligned(s1, 4) || !aligned(p1_inv, 4) || !aligned(p2_inv, 4) || !aligned(s2, 4) ||
      !aligned(M, 4))
    return fail(LQ_ERR_ALIGN, "misaligned pointer");
  return hip_status(lq::launch_lift_kron(a, a_dtype, B, n, n1, s1, p1_inv, p2_inv, s2, M, d, D,
                                         a_lift, lift_dtype, workspace, as_stream(stream)),
                    "lq_lift_kron launch");
}

lq_status lq_gemm_decoded_workspace_size(int64_t m, int64_t n, size_t* bytes) {
  if (!bytes) return fail(LQ_ERR_NULL, "bytes is null");
  if (m < 1 || n < 1) return fail(LQ_ERR_SHAPE, "m=%lld n=%lld", (long long)m, (long long)n);
  *bytes = lq::gemm_decoded_workspace_bytes(m, n);
  return ok();
}

lq_status lq_gemm_decoded(const uint32_t* w_packed, int64_t m, int64_t n, int64_t ldw,
                          const float* M, int32_t d, int32_t D, const float* s, const void* u,
                          lq_dtype u_dtype, int64_t B, float* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!w_packed || !M || !s || !u || !out) return fail(LQ_ERR_NULL, "null pointer");
  if (u_dtype != LQ_F16) return fail(LQ_ERR_DTYPE, "u must be LQ_F16");
  if (m < 1 || n < 1 || B < 1 || m > INT32_MAX || n > INT32_MAX || B > INT32_MAX)
    return fail(LQ_ERR_SHAPE, "m=%lld n=%lld B=%lld", (long long)m, (long long)n, (long long)B);
  // a workgroup addresses 128 tokens of u and 128 rows of signs with 32-bit
  // buffer offsets
  if (n > (int64_t{1} << 22))
    return fail(LQ_ERR_SHAPE, "n=%lld exceeds the per-call limit of 2^22", (long long)n);
  if (d < 1 || d > 64 || D < 1 || D > 256 || n % d)
    return fail(LQ_ERR_SHAPE, "d=%d D=%d n=%lld (1 <= d <= 64, 1 <= D <= 256, n %% d == 0)",
                (int)d, (int)D, (long long)n);
  const int64_t K = n / d * D;
  if (ldw < (K + 31) / 32) return fail(LQ_ERR_SHAPE, "ldw=%lld < ceil(K/32)", (long long)ldw);
  if (ldw > (int64_t{1} << 22))
    return fail(LQ_ERR_SHAPE, "ldw=%lld exceeds the per-call limit of 2^22", (long long)ldw);
  if (!lq::gemm_decoded_shape_ok(d, D))
    return fail(LQ_ERR_UNSUPPORTED, "d=%d D=%d beyond the decode tiles", (int)d, (int)D);
  if (workspace_bytes < lq::gemm_decoded_workspace_bytes(m, n))
    return fail(LQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes,
                lq::gemm_decoded_workspace_bytes(m, n));
  if (!aligned(w_packed, 4) || !aligned(M, 4) || !aligned(s, 4) || !aligned(u, 2) ||
      !aligned(out, 4))
    return fail(LQ_ERR_ALIGN, "misaligned pointer");
  const hipError_t e = lq::launch_gemm_decoded(w_packed, m, n, ldw, M, d, D, s, u, B, out,
                                               workspace, as_stream(stream), nullptr);
  return hip_status(e, "lq_gemm_decoded launch");
}

lq_status lq_softmin_workspace_size(int64_t N, int32_t d, int32_t D, size_t* bytes) {
  if (!bytes) return fail(LQ_ERR_NULL, "bytes is null");
  if (N < 1 || N > INT32_MAX || d < 1 || D < d || D > 24)
    return fail(LQ_ERR_SHAPE, "N=%lld d=%d D=%d", (long long)N, (int)d, (int)D);
  *bytes = lq::softmin_workspace_bytes(N, d, D);
  return ok();
}

lq_status lq_softmin_grad(const float* w, int64_t N, const float* M, int32_t d, int32_t D,
                          float T, float* loss, float* grad, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!w || !M || !loss || !grad || !workspace) return fail(LQ_ERR_NULL, "null pointer");
  if (N < 1 || N > INT32_MAX) return fail(LQ_ERR_SHAPE, "N=%lld", (long long)N);
  if (d < 1 || D < d || D > 32)
    return fail(LQ_ERR_SHAPE, "d=%d D=%d outside 1 <= d <= D <= 32", (int)d, (int)D);
  if (D > 24)
    return fail(LQ_ERR_UNSUPPORTED, "D=%d: the soft-argmin runs over all 2^D codes (D <= 24)",
                (int)D);
  if (!(T >= 0.f) || !(T < 1e30f)) return fail(LQ_ERR_SHAPE, "T=%g must be finite and >= 0", T);
  if (workspace_bytes < lq::softmin_workspace_bytes(N, d, D))
    return fail(LQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes,
                lq::softmin_workspace_bytes(N, d, D));
  if (!aligned(workspace, 256)) return fail(LQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(w, 4) || !aligned(M, 4) || !aligned(loss, 4) || !aligned(grad, 4))
    return fail(LQ_ERR_ALIGN, "misaligned pointer");
  return hip_status(lq::launch_softmin_grad(w, N, M, d, D, T, loss, grad, workspace,
                                            as_stream(stream)),
                    "lq_softmin_grad launch");
}

lq_status lq_adam_update(float* M, const float* grad, float* m1, float* m2, int64_t count,
                         int32_t step, float lr, float beta1, float beta2, float eps,
                         void* stream) {
  if (count < 0) return fail(LQ_ERR_SHAPE, "count=%lld", (long long)count);
  if (count == 0) return ok();
  if (!M || !grad || !m1 || !m2) return fail(LQ_ERR_NULL, "null pointer");
  if (step < 1 || !(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) ||
      !(eps >= 0.f))
    return fail(LQ_ERR_SHAPE, "step=%d beta1=%g beta2=%g eps=%g", (int)step, beta1, beta2, eps);
  if (!aligned(M, 4) || !aligned(grad, 4) || !aligned(m1, 4) || !aligned(m2, 4))
    return fail(LQ_ERR_ALIGN, "misaligned pointer");
  return hip_status(lq::launch_adam(M, grad, m1, m2, count, step, lr, beta1, beta2, eps,
                                    as_stream(stream)),
                    "lq_adam_update launch");
}

lq_status lq_encode_workspace_size(int32_t d, int32_t D, size_t* bytes) {
  if (!bytes) return fail(LQ_ERR_NULL, "bytes is null");
  if (d < 1 || D < d || D > 32) return fail(LQ_ERR_SHAPE, "d=%d D=%d", (int)d, (int)D);
  *bytes = lq::encode_workspace_bytes(D);
  return ok();
}

lq_status lq_encode(const float* w, int64_t groups, const float* M, const float* A, int32_t d,
                    int32_t D, int8_t* codes, float* err, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (groups < 0) return fail(LQ_ERR_SHAPE, "groups=%lld", (long long)groups);
  if (d < 1 || D < d || D > 32)
    return fail(LQ_ERR_SHAPE, "d=%d D=%d outside 1 <= d <= D <= 32", (int)d, (int)D);
  if (A ? D - d > 24 : D > 24)
    return fail(LQ_ERR_UNSUPPORTED, "%s over 2^%d candidates (at most 2^24)",
                A ? "search" : "exhaustive search", A ? (int)(D - d) : (int)D);
  if (groups > (int64_t)INT32_MAX * 4)
    return fail(LQ_ERR_SHAPE, "groups=%lld exceeds the launch limits", (long long)groups);
  if (groups == 0) return ok();
  if (!w || !M || !codes) return fail(LQ_ERR_NULL, "null pointer");
  if (A) {
    if (!workspace) return fail(LQ_ERR_NULL, "workspace is null");
    if (workspace_bytes < lq::encode_workspace_bytes(D))
      return fail(LQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes,
                  lq::encode_workspace_bytes(D));
    if (!aligned(workspace, 256)) return fail(LQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  if (!aligned(w, 4) || !aligned(M, 4) || (A && !aligned(A, 4)) || (err && !aligned(err, 4)))
    return fail(LQ_ERR_ALIGN, "misaligned pointer");
  return hip_status(lq::launch_encode(w, groups, M, A, d, D, codes, err, workspace,
                                      as_stream(stream)),
                    "lq_encode launch");
}

lq_status lq_gemv_workspace_size(int64_t m, int64_t K, int64_t B, size_t* bytes) {
  if (!bytes) return fail(LQ_ERR_NULL, "bytes is null");
  if (m < 1 || K < 1 || B < 1 || B > 16)
    return fail(LQ_ERR_SHAPE, "m=%lld K=%lld B=%lld", (long long)m, (long long)K, (long long)B);
  *bytes = gemv_workspace(m, K, B);
  return ok();
}

lq_status lq_workspace_clear(void* workspace, size_t bytes, void* stream) {
  if (bytes == 0) return ok();
  if (!workspace) return fail(LQ_ERR_NULL, "workspace is null");
  if (!aligned(workspace, 16)) return fail(LQ_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(lq::launch_fill_zero(workspace, bytes, as_stream(stream)),
                    "lq_workspace_clear launch");
}

lq_status lq_gemv(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw, const float* s,
                  const float* a_lift, int64_t B, float* out, void* workspace,
                  size_t workspace_bytes, void* stream) {
  const lq_status st = gemv_check(w_packed, m, K, ldw, s, a_lift, B, out);
  if (st != LQ_OK) return st;
  const size_t need = gemv_workspace(m, K, B);
  if (need > 0) {
    if (!workspace) return fail(LQ_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (workspace_bytes < need)
      return fail(LQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(LQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  return gemv_launch(w_packed, m, K, ldw, s, a_lift, B, out, workspace, as_stream(stream));
}

lq_status lq_lift_parts_size(int64_t K, size_t* bytes) {
  if (!bytes) return fail(LQ_ERR_NULL, "bytes is null");
  if (K < 1 || K > ((int64_t)1 << 24))
    return fail(LQ_ERR_SHAPE, "K=%lld outside 1..2^24", (long long)K);
  *bytes = lq::lift_parts_bytes(K);
  return ok();
}

lq_status lq_lift_parts(const void* a, lq_dtype a_dtype, int64_t B, int64_t n,
                        const void* t_inv, lq_dtype t_dtype, int32_t t_block,
                        const float* M, int32_t d, int32_t D, void* parts,
                        size_t parts_bytes, void* stream) {
  if (!a || !t_inv || !M || !parts) return fail(LQ_ERR_NULL, "null pointer");
  if (!valid_dtype(a_dtype) || !valid_dtype(t_dtype)) return fail(LQ_ERR_DTYPE, "unknown dtype");
  if (a_dtype != t_dtype || a_dtype == LQ_F32)
    return fail(LQ_ERR_DTYPE, "a and t_inv must share one 16-bit type");
  if (t_block != 128)
    return fail(LQ_ERR_UNSUPPORTED, "t_block=%d (only 128 is implemented)", (int)t_block);
  if (B < 1 || B > 16 || n < 1)
    return fail(LQ_ERR_SHAPE, "B=%lld (1..16) n=%lld", (long long)B, (long long)n);
  if (n % 128) return fail(LQ_ERR_SHAPE, "n=%lld not a multiple of t_block", (long long)n);
  if (d < 1 || n % d) return fail(LQ_ERR_SHAPE, "n=%lld not a multiple of d=%d", (long long)n, (int)d);
  if (n > INT32_MAX || (int64_t)n / d * D > ((int64_t)1 << 24))
    return fail(LQ_ERR_SHAPE, "n=%lld or K exceed the per-call limits", (long long)n);
  if (!lq::lift_parts_applies(a_dtype, t_dtype, B, n, d, D))
    return fail(LQ_ERR_UNSUPPORTED, "d=%d D=%d: needs d in {4, 8, 16, 32} and d <= D <= 256",
                (int)d, (int)D);
  const size_t need = lq::lift_parts_bytes((int64_t)n / d * D);
  if (parts_bytes < need)
    return fail(LQ_ERR_WORKSPACE, "parts buffer %zu bytes < %zu required", parts_bytes, need);
  if (!aligned(t_inv, 16) || !aligned(a, 16) || !aligned(parts, 16))
    return fail(LQ_ERR_ALIGN, "a, t_inv and parts must be 16-byte aligned");
  if (!aligned(M, 4)) return fail(LQ_ERR_ALIGN, "misaligned M");
  return hip_status(lq::launch_lift_parts(a, a_dtype, B, n, t_inv, M, d, D, parts,
                                          as_stream(stream)),
                    "lq_lift_parts launch");
}

lq_status lq_gemv_parts_workspace_size(int64_t m, int64_t K, int64_t B, size_t* bytes) {
  if (!bytes) return fail(LQ_ERR_NULL, "bytes is null");
  if (m < 1 || K < 1 || B < 1 || B > 16)
    return fail(LQ_ERR_SHAPE, "m=%lld K=%lld B=%lld", (long long)m, (long long)K, (long long)B);
  *bytes = lq::gemv_f4m_parts_workspace_bytes(m, K, B);
  return ok();
}

lq_status lq_gemv_parts(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw,
                        const float* s, const void* parts, size_t parts_bytes, int64_t B,
                        float* out, void* workspace, size_t workspace_bytes, void* stream) {
  const lq_status st = gemv_check(w_packed, m, K, ldw, s, static_cast<const float*>(parts), B, out);
  if (st != LQ_OK) return st;
  if (parts_bytes < lq::lift_parts_bytes(K))
    return fail(LQ_ERR_WORKSPACE, "parts buffer %zu bytes < %zu required", parts_bytes,
                lq::lift_parts_bytes(K));
  const size_t need = lq::gemv_f4m_parts_workspace_bytes(m, K, B);
  if (!workspace) return fail(LQ_ERR_NULL, "workspace of %zu bytes required", need);
  if (workspace_bytes < need)
    return fail(LQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(LQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  return hip_status(lq::launch_gemv_f4m_parts(w_packed, m, K, ldw, s, parts, B, out, workspace,
                                              as_stream(stream)),
                    "lq_gemv_parts launch");
}

lq_status lq_stream_read(const void* buffer, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return ok();
  if (!buffer || !sink) return fail(LQ_ERR_NULL, "null pointer");
  if (bytes % 16) return fail(LQ_ERR_SHAPE, "bytes=%zu must be a multiple of 16", bytes);
  if (!aligned(buffer, 16) || !aligned(sink, 4)) return fail(LQ_ERR_ALIGN, "misaligned pointer");
  return hip_status(lq::launch_stream_read(buffer, bytes, sink, 4 * lq::num_cus(),
                                           as_stream(stream)),
                    "lq_stream_read launch");
}

lq_status lq_gemv_noalloc(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw,
                          const float* s, const float* a_lift, int64_t B, float* out,
                          void* stream) {
  const lq_status st = gemv_check(w_packed, m, K, ldw, s, a_lift, B, out);
  if (st != LQ_OK) return st;
  const size_t need = gemv_workspace(m, K, B);
  if (need > kScratchBytes)
    return fail(LQ_ERR_WORKSPACE,
                "this shape needs %zu bytes of scratch, more than the %zu bytes the library "
                "holds per GPU for lq_gemv_noalloc: use lq_gemv with a workspace",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_pointer(&ws);
    if (e != hipSuccess) return hip_status(e, "lq_gemv_noalloc scratch address");
  }
  return gemv_launch(w_packed, m, K, ldw, s, a_lift, B, out, ws, as_stream(stream));
}

lq_status lq_layer_b1_workspace_size(int64_t m, int64_t n, int32_t d, int32_t D,
                                     size_t* bytes) {
  if (!bytes) return fail(LQ_ERR_NULL, "bytes is null");
  if (m < 1 || n < 1 || d < 1 || D < 1 || n % d)
    return fail(LQ_ERR_SHAPE, "m=%lld n=%lld d=%d D=%d", (long long)m, (long long)n, (int)d,
                (int)D);
  *bytes = lq::gemv1_workspace_bytes(m, n / d * D);
  return ok();
}

lq_status lq_layer_b1(const void* a, lq_dtype a_dtype, int64_t n, const void* t_inv,
                      lq_dtype t_dtype, int32_t t_block, const float* M, int32_t d, int32_t D,
                      const uint32_t* w_packed, int64_t m, int64_t ldw, const float* s,
                      float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!a || !t_inv || !M || !w_packed || !s || !out) return fail(LQ_ERR_NULL, "null pointer");
  if (!valid_dtype(a_dtype) || a_dtype != t_dtype)
    return fail(LQ_ERR_DTYPE, "a and t_inv must share one of LQ_F16, LQ_BF16, LQ_F32");
  if (t_block != 128)
    return fail(LQ_ERR_UNSUPPORTED, "t_block=%d (only 128 is implemented)", (int)t_block);
  if (m < 1 || n < 1 || n % 128 || d < 1 || d > 64 || D > 256 || d * D > 8192 || n % d)
    return fail(LQ_ERR_SHAPE, "m=%lld n=%lld d=%d D=%d (n %% 128 == 0, n %% d == 0, 1 <= d <= "
                "64, D <= 256, d*D <= 8192)", (long long)m, (long long)n, (int)d, (int)D);
  if (D < d)
    return fail(LQ_ERR_UNSUPPORTED, "D=%d < d=%d (below one bit per weight) is not fused",
                (int)D, (int)d);
  const int64_t K = n / d * D;
  if (ldw < (K + 31) / 32) return fail(LQ_ERR_SHAPE, "ldw=%lld < ceil(K/32)", (long long)ldw);
  if (ldw % 4) return fail(LQ_ERR_ALIGN, "ldw=%lld must be a multiple of 4", (long long)ldw);
  if (K % 4) return fail(LQ_ERR_SHAPE, "K=%lld must be a multiple of 4", (long long)K);
  if (m * ldw * 4 > ((int64_t)1 << 30))
    return fail(LQ_ERR_SHAPE, "weights of %lld bytes exceed the 1 GiB per-call limit",
                (long long)(m * ldw * 4));
  if (K > ((int64_t)1 << 24))
    return fail(LQ_ERR_SHAPE, "K=%lld exceeds the per-call limit of 2^24", (long long)K);
  if (!aligned(w_packed, 16) || !aligned(a, 16) || !aligned(t_inv, 16))
    return fail(LQ_ERR_ALIGN, "w_packed, a and t_inv must be 16-byte aligned");
  if (!aligned(M, 4) || !aligned(s, 4) || !aligned(out, 4))
    return fail(LQ_ERR_ALIGN, "misaligned M, s or out");
  const size_t need = lq::gemv1_workspace_bytes(m, K);
  if (need > 0) {
    if (!workspace) return fail(LQ_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (workspace_bytes < need)
      return fail(LQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(LQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  return hip_status(lq::launch_layer_b1(a, a_dtype, t_inv, M, d, D, w_packed, m, K, ldw, s, out,
                                        workspace, as_stream(stream)),
                    "lq_layer_b1 launch");
}

lq_status lq_gemm(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw, const float* s,
                  const void* a_lift, lq_dtype lift_dtype, int64_t B, float* out, void* stream) {
  if (!w_packed || !s || !a_lift || !out) return fail(LQ_ERR_NULL, "null pointer");
  if (lift_dtype != LQ_F16 && lift_dtype != LQ_BF16)
    return fail(LQ_ERR_DTYPE, "lq_gemm takes LQ_F16 or LQ_BF16 lifted activations");
  if (m < 1 || K < 1 || B < 1)
    return fail(LQ_ERR_SHAPE, "m=%lld K=%lld B=%lld", (long long)m, (long long)K, (long long)B);
  if (ldw < (K + 31) / 32) return fail(LQ_ERR_SHAPE, "ldw=%lld < ceil(K/32)", (long long)ldw);
  if (K % 8) return fail(LQ_ERR_SHAPE, "K=%lld must be a multiple of 8", (long long)K);
  if (m > INT32_MAX || B > INT32_MAX || K > kGemmMaxK || ldw > kGemmMaxK)
    return fail(LQ_ERR_SHAPE, "m=%lld B=%lld must be < 2^31, K=%lld and ldw=%lld <= 2^22",
                (long long)m, (long long)B, (long long)K, (long long)ldw);
  if (!aligned(w_packed, 4)) return fail(LQ_ERR_ALIGN, "w_packed must be 4-byte aligned");
  if (!aligned(a_lift, 16)) return fail(LQ_ERR_ALIGN, "a_lift must be 16-byte aligned");
  if (!aligned(s, 4) || !aligned(out, 4)) return fail(LQ_ERR_ALIGN, "misaligned s or out");
  return hip_status(lq::launch_gemm(w_packed, m, K, ldw, s, a_lift, lift_dtype, B, out,
                                    as_stream(stream)),
                    "lq_gemm launch");
}

}  // extern "C"
