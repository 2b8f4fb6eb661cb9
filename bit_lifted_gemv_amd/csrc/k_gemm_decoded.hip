// Decode-weights product for large batches: instead of contracting the 1-bit
// signs with the lifted activations over K = n D / d (关键设计 4's lifted
// GEMM), reconstruct the weights W_hat[i][g d + r] = sum_j M[r][j] y_ij
// (关键设计 1: w = M y) and contract over n with the whitened activations
// u = T^-1 a:  out[b][i] = s_i sum_{k<n} W_hat[i][k] u[b][k].  The two are
// the same linear map (y . (M^T x) = (M y) . x); this one costs 2 m n B
// flops for the product plus 2 m n D for the reconstruction, against
// 2 m K B lifted, fewer once B > D d / (D - d).
//
// decode kernel: a workgroup takes 16 rows.  It first builds, in LDS, one
// table per 8-sign chunk position p of a group: tab[p][c][r] = sum over the
// chunk's signs j of M[r][8p + j] (bit j of c set: +1, else -1), 256 entries
// of d floats (the last chunk covers D % 8 signs).  Then each thread takes
// groups (row i, group g): the D sign bits start at bit g D of the row, each
// 8-bit chunk selects a table entry, the d partial vectors add up to the
// group's d weights, scaled by s_i and stored as float16 (s folded into the
// decoded weights).
// product: a plain float16 x float16 -> float32 GEMM (rocBLAS), rows taken
// in chunks that bound the decoded buffer.
#include <rocblas/rocblas.h>

#include <unordered_map>

#include "lq_internal.h"

namespace lq {
namespace {

constexpr int kT = 256;
constexpr int kRows = 16;                   // rows per decode workgroup
constexpr int64_t kChunkElems = int64_t{1} << 27;   // decoded weights per product chunk

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int chunks_of(int D) { return (D + 7) / 8; }

// DM >= d, a multiple of 4: register width of a group's accumulated weights.
template <int DM>
__global__ void __launch_bounds__(kT) decode_kernel(const uint32_t* __restrict__ w, int64_t m,
                                                    int64_t ldw, int64_t groups_per_row,
                                                    const float* __restrict__ M, int d, int D,
                                                    const float* __restrict__ s,
                                                    uint16_t* __restrict__ out, int64_t n) {
  extern __shared__ f32x4 lds[];
  float* tab = reinterpret_cast<float*>(lds);       // [P][256][DM]
  const int P = chunks_of(D);
  // tables
  for (int e = threadIdx.x; e < P * 256; e += kT) {
    const int p = e >> 8;
    const int c = e & 255;
    const int nb = min(8, D - 8 * p);
    float acc[DM];
#pragma unroll
    for (int r = 0; r < DM; ++r) acc[r] = 0.f;
    for (int b = 0; b < nb; ++b) {
      const float sg = (c >> b) & 1 ? 1.f : -1.f;
      const int j = 8 * p + b;
#pragma unroll
      for (int r = 0; r < DM; ++r)
        if (r < d) acc[r] = fmaf(sg, M[r * D + j], acc[r]);
    }
#pragma unroll
    for (int r4 = 0; r4 < DM / 4; ++r4)
      *reinterpret_cast<f32x4*>(tab + (static_cast<size_t>(e) * DM + 4 * r4)) =
          f32x4{acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
  }
  __syncthreads();
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int rows = static_cast<int>(min<int64_t>(kRows, m - row0));
  const int64_t total = rows * groups_per_row;
  const uint32_t last_mask = (D % 8) ? (1u << (D % 8)) - 1u : 0xffu;
  for (int64_t e = threadIdx.x; e < total; e += kT) {
    const int64_t ri = e / groups_per_row;
    const int64_t g = e - ri * groups_per_row;
    const int64_t i = row0 + ri;
    const uint32_t* wr = w + i * ldw;
    float acc[DM];
#pragma unroll
    for (int r = 0; r < DM; ++r) acc[r] = 0.f;
    const int64_t bit0 = g * D;
    for (int p = 0; p < P; ++p) {
      const int64_t o = bit0 + 8 * p;
      const int64_t wi = o >> 5;
      const uint32_t sh = static_cast<uint32_t>(o & 31);
      // the chunk's nb real bits may straddle two words; the second word is
      // read only when some of them lie in it (so never past the row's last
      // data word)
      const int nb = p == P - 1 ? D - 8 * p : 8;
      uint32_t v = wr[wi] >> sh;
      if (static_cast<int>(sh) + nb > 32) v |= wr[wi + 1] << (32 - sh);
      uint32_t c = v & 0xffu;
      if (p == P - 1) c &= last_mask;
      const float* t = tab + (static_cast<size_t>(p) * 256 + c) * DM;
#pragma unroll
      for (int r4 = 0; r4 < DM / 4; ++r4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(t + 4 * r4);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[4 * r4 + q] += x[q];
      }
    }
    const float si = s[i];
    uint16_t* dst = out + i * n + g * d;          // row i of the chunk's buffer
    for (int r = 0; r < d; ++r) dst[r] = float_to_f16_bits_rne(si * acc[r]);
  }
}

// One rocBLAS handle per device and host thread (a handle carries a stream,
// so threads do not share one); created on first use, kept to the end of the
// process.
rocblas_handle handle_for_device(int dev) {
  thread_local std::unordered_map<int, rocblas_handle> mine;
  auto it = mine.find(dev);
  if (it != mine.end()) return it->second;
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
  mine.emplace(dev, h);
  return h;
}

template <int DM>
hipError_t launch_decode(const uint32_t* w, int64_t rows, int64_t ldw, int64_t gpr,
                         const float* M, int d, int D, const float* s, uint16_t* out, int64_t n,
                         hipStream_t st) {
  const size_t lds = static_cast<size_t>(chunks_of(D)) * 256 * DM * sizeof(float);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_kernel<DM>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_kernel<DM>, dim3(static_cast<unsigned>((rows + kRows - 1) / kRows)),
                     dim3(kT), lds, st, w, rows, ldw, gpr, M, d, D, s, out, n);
  return hipGetLastError();
}

int dm_for(int d) { return d <= 4 ? 4 : d <= 8 ? 8 : d <= 16 ? 16 : d <= 32 ? 32 : 64; }

}  // namespace

bool gemm_decoded_shape_ok(int d, int D) {
  return d <= 64 && static_cast<size_t>(chunks_of(D)) * 256 * dm_for(d) * sizeof(float) <=
                        128 * 1024;
}

int64_t gemm_decoded_chunk_rows(int64_t m, int64_t n) {
  const int64_t r = std::max<int64_t>(kRows, kChunkElems / n / kRows * kRows);
  return std::min(m, r);
}

size_t gemm_decoded_workspace_bytes(int64_t m, int64_t n) {
  return (static_cast<size_t>(gemm_decoded_chunk_rows(m, n)) * n * 2 + 255) / 256 * 256;
}

hipError_t launch_gemm_decoded(const uint32_t* w, int64_t m, int64_t n, int64_t ldw,
                               const float* M, int d, int D, const float* s, const void* u,
                               int64_t B, float* out, void* ws, hipStream_t st,
                               const char** why) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  rocblas_handle h = handle_for_device(dev);
  if (!h) {
    *why = "rocblas_create_handle failed";
    return hipErrorUnknown;
  }
  if (rocblas_set_stream(h, st) != rocblas_status_success) {
    *why = "rocblas_set_stream failed";
    return hipErrorUnknown;
  }
  const int64_t gpr = n / d;
  const int64_t chunk = gemm_decoded_chunk_rows(m, n);
  uint16_t* wh = static_cast<uint16_t*>(ws);
  const float alpha = 1.f, beta = 0.f;
  for (int64_t r0 = 0; r0 < m; r0 += chunk) {
    const int64_t rows = std::min(chunk, m - r0);
    const uint32_t* wc = w + r0 * ldw;
    switch (dm_for(d)) {
      case 4: e = launch_decode<4>(wc, rows, ldw, gpr, M, d, D, s + r0, wh, n, st); break;
      case 8: e = launch_decode<8>(wc, rows, ldw, gpr, M, d, D, s + r0, wh, n, st); break;
      case 16: e = launch_decode<16>(wc, rows, ldw, gpr, M, d, D, s + r0, wh, n, st); break;
      case 32: e = launch_decode<32>(wc, rows, ldw, gpr, M, d, D, s + r0, wh, n, st); break;
      default: e = launch_decode<64>(wc, rows, ldw, gpr, M, d, D, s + r0, wh, n, st); break;
    }
    if (e != hipSuccess) return e;
    // out (column-major rows x B, leading dimension m) = W_hat^T-stored (n x rows,
    // leading dimension n) transposed, times u (n x B, leading dimension n)
    const rocblas_status rs = rocblas_gemm_ex(
        h, rocblas_operation_transpose, rocblas_operation_none, static_cast<rocblas_int>(rows),
        static_cast<rocblas_int>(B), static_cast<rocblas_int>(n), &alpha, wh, rocblas_datatype_f16_r,
        static_cast<rocblas_int>(n), u, rocblas_datatype_f16_r, static_cast<rocblas_int>(n), &beta,
        out + r0, rocblas_datatype_f32_r, static_cast<rocblas_int>(m), out + r0,
        rocblas_datatype_f32_r, static_cast<rocblas_int>(m), rocblas_datatype_f32_r,
        rocblas_gemm_algo_standard, 0, 0);
    if (rs != rocblas_status_success) {
      *why = rocblas_status_to_string(rs);
      return hipErrorUnknown;
    }
  }
  return hipSuccess;
}

}  // namespace lq
