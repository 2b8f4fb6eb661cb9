// Tables of signed activation sums for the batch-1 GEMV (see k_gemv.hip).
//
// For each token t and 1024-position slice s of the lifted dimension, and
// every weight-byte value v, the entry of byte position p is
//   E_p(v) = sum_{i<8} (2*bit_i(v) - 1) * a_hat[t][1024 s + 8 p + i]
// so that a row's contribution from byte p is E_p(row byte).  The 128
// positions of a slice are stored under a slot permutation chosen for
// conflict-free LDS reads (lut_slot), 2-byte float16 entries, rounded to
// nearest even:
//   table (t, s): 64 KB, entry (v, slot) at byte 256 v + 2 slot.
// Positions at or past K count as zero activations.
#include "lq_internal.h"

namespace lq {

namespace {

constexpr int kLutThreads = 256;

// Entry of slot `sl` in each half of the table: one thread per (slot, half).
__global__ void __launch_bounds__(kLutThreads) build_lut_kernel(const float* __restrict__ ah,
                                                                int64_t K, int S,
                                                                uint16_t* __restrict__ lut) {
  const int s = blockIdx.x;
  const int t = blockIdx.y;
  const int sl = threadIdx.x & 127;
  const int half = threadIdx.x >> 7;            // v in [128 half, 128 half + 128)
  const int p = lut_pos(sl);
  const int64_t k0 = (int64_t)s * 1024 + 8 * p;
  const float* a = ah + (int64_t)t * K;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (k0 + i < K) ? a[k0 + i] : 0.f;
  // low nibble sums L[lo] = sum_{i<4} +-x_i, high nibble sums H[hi] = sum_{i<4} +-x_{4+i}
  float L[16], H[8];
#pragma unroll
  for (int lo = 0; lo < 16; ++lo) {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) v += ((lo >> i) & 1) ? x[i] : -x[i];
    L[lo] = v;
  }
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const int hi = 8 * half + h;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) v += ((hi >> i) & 1) ? x[4 + i] : -x[4 + i];
    H[h] = v;
  }
  uint16_t* out = lut + ((int64_t)t * S + s) * (256 * 128) + sl;
#pragma unroll
  for (int h = 0; h < 8; ++h)
#pragma unroll
    for (int lo = 0; lo < 16; ++lo) {
      const int v = 16 * (8 * half + h) + lo;
      out[v * 128] = float_to_f16_bits_rne(L[lo] + H[h]);
    }
}

}  // namespace

hipError_t launch_build_lut(const float* a_lift, int64_t B, int64_t K, void* lut,
                            hipStream_t st) {
  const int S = static_cast<int>((K + 1023) / 1024);
  hipLaunchKernelGGL(build_lut_kernel, dim3(S, static_cast<unsigned>(B)), dim3(kLutThreads), 0,
                     st, a_lift, K, S, static_cast<uint16_t*>(lut));
  return hipGetLastError();
}

}  // namespace lq
