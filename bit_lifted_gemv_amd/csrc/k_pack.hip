// Sign packing (set-up step, outside the timed layer): int8 signs <-> W_q words.
// Storage: lifted position k of a row is bit (k & 31) of word (k >> 5); the bit
// is 1 iff the sign is positive (LiftQuant notes, 关键设计 1: one bit per sign).
#include "lq_internal.h"

namespace lq {
namespace {

// One thread per output word; 32 sign bytes are folded into one word.
__global__ void __launch_bounds__(256) pack_signs_kernel(const int8_t* __restrict__ signs,
                                                         int64_t rows, int64_t K, int64_t lds,
                                                         uint32_t* __restrict__ packed,
                                                         int64_t ldw) {
  const int64_t total = rows * ldw;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / ldw;
    const int64_t w = idx - row * ldw;
    const int64_t k0 = w * 32;
    uint32_t word = 0;
    if (k0 < K) {
      const int8_t* src = signs + row * lds + k0;
      const int nb = (K - k0) < 32 ? static_cast<int>(K - k0) : 32;
      for (int b = 0; b < nb; ++b) word |= (src[b] > 0 ? 1u : 0u) << b;
    }
    packed[idx] = word;
  }
}

// One thread per sign.
__global__ void __launch_bounds__(256) unpack_signs_kernel(const uint32_t* __restrict__ packed,
                                                           int64_t rows, int64_t K, int64_t ldw,
                                                           int8_t* __restrict__ signs,
                                                           int64_t lds) {
  const int64_t total = rows * K;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / K;
    const int64_t k = idx - row * K;
    const uint32_t word = packed[row * ldw + (k >> 5)];
    signs[row * lds + k] = ((word >> (k & 31)) & 1u) ? int8_t(1) : int8_t(-1);
  }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(uint8_t* __restrict__ p, size_t bytes) {
  const size_t n16 = bytes / 16;
  uint4* p16 = reinterpret_cast<uint4*>(p);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += stride)
    p16[i] = make_uint4(0, 0, 0, 0);
  for (size_t i = n16 * 16 + blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < bytes; i += stride)
    p[i] = 0;
}

int grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return static_cast<int>(g);
}

}  // namespace

hipError_t launch_pack_signs(const int8_t* signs, int64_t rows, int64_t K, int64_t lds,
                             uint32_t* packed, int64_t ldw, hipStream_t st) {
  const int64_t total = rows * ldw;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_signs_kernel, dim3(grid_for(total)), dim3(256), 0, st, signs, rows, K,
                     lds, packed, ldw);
  return hipGetLastError();
}

hipError_t launch_unpack_signs(const uint32_t* packed, int64_t rows, int64_t K, int64_t ldw,
                               int8_t* signs, int64_t lds, hipStream_t st) {
  const int64_t total = rows * K;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(unpack_signs_kernel, dim3(grid_for(total)), dim3(256), 0, st, packed, rows,
                     K, ldw, signs, lds);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  // p is 16-byte aligned (checked by the caller).
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(static_cast<int64_t>(bytes / 16 + 1))),
                     dim3(256), 0, st, static_cast<uint8_t*>(p), bytes);
  return hipGetLastError();
}

}  // namespace lq
