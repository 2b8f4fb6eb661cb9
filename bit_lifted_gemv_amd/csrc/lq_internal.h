// Internal declarations shared by the HIP translation units of liblq.
// Kernel launchers return hipError_t from the launch; argument validation
// happens in lq_api.hip before any of them is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lq.h"

namespace lq {

// ---------------------------------------------------------------- dtype helpers
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float f16_bits_to_float(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

__device__ __forceinline__ uint16_t float_to_f16_bits_rne(float f) {
  _Float16 h = static_cast<_Float16>(f);   // v_cvt_f16_f32: round to nearest even
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// Load element i of a typed 16/32-bit array as float.
template <int DT>
__device__ __forceinline__ float load_as_float(const void* p, int64_t i);

template <>
__device__ __forceinline__ float load_as_float<LQ_F32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_as_float<LQ_F16>(const void* p, int64_t i) {
  return f16_bits_to_float(static_cast<const uint16_t*>(p)[i]);
}
template <>
__device__ __forceinline__ float load_as_float<LQ_BF16>(const void* p, int64_t i) {
  return bf16_bits_to_float(static_cast<const uint16_t*>(p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_from_float(void* p, int64_t i, float v);

template <>
__device__ __forceinline__ void store_from_float<LQ_F32>(void* p, int64_t i, float v) {
  static_cast<float*>(p)[i] = v;
}
template <>
__device__ __forceinline__ void store_from_float<LQ_F16>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = float_to_f16_bits_rne(v);
}
template <>
__device__ __forceinline__ void store_from_float<LQ_BF16>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = float_to_bf16_bits_rne(v);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_pack_signs(const int8_t* signs, int64_t rows, int64_t K, int64_t lds,
                             uint32_t* packed, int64_t ldw, hipStream_t st);
hipError_t launch_unpack_signs(const uint32_t* packed, int64_t rows, int64_t K, int64_t ldw,
                               int8_t* signs, int64_t lds, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

hipError_t launch_lift(const void* a, lq_dtype a_dt, int64_t B, int64_t n, const void* t_inv,
                       lq_dtype t_dt, const float* M, int d, int D, void* out, lq_dtype out_dt,
                       hipStream_t st);

// The matrix-core lift (k_lift_mfma.hip) takes over from 8 tokens (from 4
// when n >= 12288, where T^-1 is large enough for its wider reads to pay)
// when a and T^-1 share a 16-bit type and d divides 128 (d = 4, 8, 16, 32).
bool lift_mfma_applies(lq_dtype a_dt, lq_dtype t_dt, int64_t B, int64_t n, int d, int D);
hipError_t launch_lift_mfma(const void* a, lq_dtype dt, int64_t B, int64_t n, const void* t_inv,
                            const float* M, int d, int D, void* out, lq_dtype out_dt,
                            hipStream_t st);

// Lift with the Kronecker-factored whitening (k_lift_kron.hip).
bool lift_kron_shape_ok(int64_t n, int n1, int d, int D);
// Decode-weights product, one kernel (k_gemm_dec.hip); no workspace.
bool gemm_decoded_shape_ok(int d, int D);
size_t gemm_decoded_workspace_bytes(int64_t m, int64_t n);
hipError_t launch_gemm_decoded(const uint32_t* w, int64_t m, int64_t n, int64_t ldw,
                               const float* M, int d, int D, const float* s, const void* u,
                               int64_t B, float* out, void* ws, hipStream_t st,
                               const char** why);

size_t softmin_workspace_bytes(int64_t N, int d, int D);
hipError_t launch_softmin_grad(const float* W, int64_t N, const float* M, int d, int D, float T,
                               float* loss, float* grad, void* ws, hipStream_t st);
hipError_t launch_adam(float* M, const float* g, float* m1, float* m2, int64_t count, int step,
                       float lr, float b1, float b2, float eps, hipStream_t st);

size_t encode_workspace_bytes(int D);
hipError_t launch_encode(const float* w, int64_t groups, const float* M, const float* A, int d,
                         int D, int8_t* codes, float* err, void* ws, hipStream_t st);

size_t lift_kron_workspace_bytes(int64_t B, int64_t n);
hipError_t launch_lift_kron(const void* a, lq_dtype a_dt, int64_t B, int64_t n, int n1,
                            const float* s1, const float* p1_inv, const float* p2_inv,
                            const float* s2, const float* M, int d, int D, void* out,
                            lq_dtype out_dt, void* ws, hipStream_t st);

// Plain streaming read (k_stream.hip): `groups` workgroups of 1024 threads.
hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, int groups,
                              hipStream_t st);

// Compute units of the current device (cached per device).
int num_cus();

// One-token GEMV on float16 activation-sum tables (k_gemv1.hip).
size_t gemv1_workspace_bytes(int64_t m, int64_t K);
// One-token layer with the lift in the GEMV's table prologue (k_gemv1.hip).
hipError_t launch_layer_b1(const void* a, lq_dtype dt, const void* t_inv, const float* M, int d,
                           int D, const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                           const float* s, float* out, void* ws, hipStream_t st);

// GEMV for 6 <= B <= 16 on float4 sign / float8 activation-part matrix
// cores, the three parts as column blocks (k_gemv_f4m.hip).
size_t gemv_f4m_workspace_bytes(int64_t m, int64_t K, int64_t B);
hipError_t launch_gemv_f4m(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                           const float* a_lift, int64_t B, float* out, void* ws, hipStream_t st);

// The same product on an operand image written by the parts lift (no
// preparation launch; the workspace holds only the split partial sums).
size_t gemv_f4m_parts_workspace_bytes(int64_t m, int64_t K, int64_t B);
hipError_t launch_gemv_f4m_parts(const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                                 const float* s, const void* parts, int64_t B, float* out,
                                 void* ws, hipStream_t st);

// The lift into that image (k_lift_parts.hip): bytes for K lifted
// positions, and whether the kernel takes the shape.
size_t lift_parts_bytes(int64_t K);
bool lift_parts_applies(lq_dtype a_dt, lq_dtype t_dt, int64_t B, int64_t n, int d, int D);
hipError_t launch_lift_parts(const void* a, lq_dtype dt, int64_t B, int64_t n, const void* t_inv,
                             const float* M, int d, int D, void* image, hipStream_t st);

// Few-token GEMV on float4 sign / float8 activation-part matrix cores
// (k_gemv_f4.hip), 1 <= B <= 5.
size_t gemv_f4_workspace_bytes(int64_t m, int64_t K, int64_t B);
hipError_t launch_gemv_f4(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                          const float* a_lift, int64_t B, float* out, void* ws, hipStream_t st);

// One-launch GEMV for 1 <= B <= 5 (k_gemv_f4r.hip): each workgroup owns
// whole rows; no workspace.  Applies when its LDS holds the sums.
bool gemv_f4r_applies(int64_t m, int64_t K, int64_t B);
hipError_t launch_gemv_f4r(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                           const float* a_lift, int64_t B, float* out, hipStream_t st);

hipError_t launch_gemm(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                       const void* a_lift, lq_dtype dt, int64_t B, float* out, hipStream_t st);

}  // namespace lq
