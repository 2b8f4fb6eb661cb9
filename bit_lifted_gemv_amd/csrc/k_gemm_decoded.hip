// Decode-weights product for large batches: instead of contracting the 1-bit
// signs with the lifted activations over K = n D / d (关键设计 4's lifted
// GEMM), reconstruct the weights W_hat[i][g d + r] = sum_j M[r][j] y_ij
// (关键设计 1: w = M y) and contract over n with the whitened activations
// u = T^-1 a:  out[b][i] = s_i sum_{k<n} W_hat[i][k] u[b][k].  The two are
// the same linear map (y . (M^T x) = (M y) . x); this one costs 2 m n B
// flops for the product plus 2 m n D for the reconstruction, against
// 2 m K B lifted, fewer once B > D d / (D - d).
//
// decode kernel: on the matrix cores.  For a group g the decoded weights of
// 16 rows are W_hat[rows][g d + c] = sum_j y[rows][g D + j] M[c][j], a
// 16 x d x D product with exact +-1 signs: a wave takes 16 rows and a slice
// of groups; each 8-sign byte expands to eight float16 +-1 through an LDS
// table, M's float16 fragments sit in LDS, and the float32 results are
// scaled by s_i and stored as float16 (s folded into the decoded weights; M
// and the product are rounded to float16 once each).
// product: a plain float16 x float16 -> float32 GEMM (rocBLAS), rows taken
// in chunks that bound the decoded buffer.
#include <rocblas/rocblas.h>

#include <unordered_map>

#include "lq_internal.h"

namespace lq {
namespace {

constexpr int kRows = 16;                   // rows per decode wave
constexpr int64_t kChunkElems = int64_t{1} << 27;   // decoded weights per product chunk

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));

using f16x8 = _Float16 __attribute__((ext_vector_type(8)));
constexpr int kWaves = 4;
constexpr int kMaxKB = 8;                   // D <= 256: k blocks of 32 signs
constexpr int kMaxNT = 4;                   // d <= 64: output tiles of 16 weights
constexpr int kSpan = 256;                  // staged float16 per row and wave (d <= 64 fits)

// A wave decodes 16 rows x a slice of groups on the matrix cores: for group
// g, W_hat[rows][g d + c] = sum_j y[rows][g D + j] M[c][j] is a 16 x 16 x 32
// f16 product per (k block of 32 signs, tile of 16 weights).  Lane (l % 16,
// q = l / 16) holds signs 32 kb + 8 q .. + 7 of row l % 16 (one byte of the
// sign string, expanded to eight exact +-1 halves through a 256-entry LDS
// table) and M[16 nt + l % 16][32 kb + 8 q .. + 7] (fragments prepared in
// LDS, zero past d and D, so padded signs add nothing).  The result lane
// holds rows 4 q + e of weight 16 nt + l % 16.
// The slice is taken in sub-slices of at most sub_groups groups: their sign
// words (16 rows x a contiguous run each) are first copied to LDS with
// coalesced loads, so the group loop reads only LDS; the decoded float16 of
// a sub-slice is staged in LDS and written back as contiguous row runs.
// Dynamic LDS: expand [256] u32x4 | mfrag [KB NT 64] u32x4 |
// per wave: sign words [16][words] u32, staged output [16][span] u16.
__global__ void __launch_bounds__(64 * kWaves) decode_mfma_kernel(
    const uint32_t* __restrict__ w, int64_t m, int64_t ldw, int64_t groups_per_row,
    int64_t groups_per_wave, int sub_groups, int words, const float* __restrict__ M, int d,
    int D, const float* __restrict__ s, uint16_t* __restrict__ out, int64_t n) {
  extern __shared__ u32x4 lds4[];
  const int KB = (D + 31) / 32;
  const int NT = (d + 15) / 16;
  const int span_max = sub_groups * d;
  const int span_pad = (span_max + 7) & ~7;
  u32x4* expand = lds4;
  u32x4* mfrag = expand + 256;
  uint32_t* sbits_all = reinterpret_cast<uint32_t*>(mfrag + KB * NT * 64);
  uint16_t* stage_all = reinterpret_cast<uint16_t*>(sbits_all + kWaves * 16 * words);
  for (int c = threadIdx.x; c < 256; c += 64 * kWaves) {
    u32x4 v;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t lo = (c >> (2 * h)) & 1 ? 0x3C00u : 0xBC00u;
      const uint32_t hi = (c >> (2 * h + 1)) & 1 ? 0x3C00u : 0xBC00u;
      v[h] = lo | (hi << 16);
    }
    expand[c] = v;
  }
  for (int e = threadIdx.x; e < KB * NT * 64; e += 64 * kWaves) {
    const int l = e & 63;
    const int f = e >> 6;                           // kb * NT + nt
    const int kb = f / NT;
    const int nt = f - kb * NT;
    const int r = 16 * nt + (l & 15);
    u32x4 v;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t pair = 0;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        // unconditional loads (clamped index) so that they overlap
        const int j = 32 * kb + 8 * (l >> 4) + 2 * h + b;
        const bool in = r < d && j < D;
        const float x = M[in ? r * D + j : 0];
        pair |= static_cast<uint32_t>(float_to_f16_bits_rne(in ? x : 0.f)) << (16 * b);
      }
      v[h] = pair;
    }
    mfrag[e] = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  uint32_t* sbits = sbits_all + wave * 16 * words;       // [16][words]
  uint16_t* stage = stage_all + wave * 16 * span_pad;     // [16][span_pad]
  const int q = lane >> 4;
  const int rl = lane & 15;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t g0 = (static_cast<int64_t>(blockIdx.y) * kWaves + wave) * groups_per_wave;
  const int64_t g1 = min(groups_per_row, g0 + groups_per_wave);
  float sr[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t r = row0 + 4 * q + e;
    const float x = s[r < m ? r : 0];
    sr[e] = r < m ? x : 0.f;
  }
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  for (int64_t gs = g0; gs < g1; gs += sub_groups) {
    const int cnt = static_cast<int>(min<int64_t>(sub_groups, g1 - gs));
    // sign words of rows row0 .. row0 + 15 covering bits gs D .. (gs + cnt) D
    const int64_t w0 = (gs * D) >> 5;
    const int64_t wlast = ((gs + cnt) * D - 1) >> 5;
    const int wc = static_cast<int>(wlast - w0 + 1);        // <= words
    // all loads first (a word per lane and row, two passes when the run is
    // longer than the wave), then the LDS writes: one memory latency
    for (int k0 = 0; k0 < wc; k0 += 64) {
      const int k = k0 + lane;
      uint32_t v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool in = k < wc && row0 + r < m;
        v[r] = w[in ? (row0 + r) * ldw + w0 + k : 0];
      }
      if (k < wc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sbits[r * words + k] = v[r];
      }
    }
    wave_sync();
    for (int gl = 0; gl < cnt; ++gl) {
      const int64_t g = gs + gl;
      f32x4 acc[kMaxNT];
#pragma unroll
      for (int nt = 0; nt < kMaxNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kb = 0; kb < KB; ++kb) {
        // byte 4 kb + q of the group's sign string (bits past D are
        // don't-care: their M entries are zero)
        const int j0 = 32 * kb + 8 * q;
        uint32_t byte = 0;
        if (j0 < D) {
          const int64_t o = g * D + j0 - w0 * 32;           // bit offset in the staged run
          const int wi = static_cast<int>(o >> 5);
          const uint32_t sh = static_cast<uint32_t>(o & 31);
          const int nb = min(8, D - j0);
          uint32_t v = sbits[rl * words + wi] >> sh;
          if (static_cast<int>(sh) + nb > 32) v |= sbits[rl * words + wi + 1] << (32 - sh);
          byte = v & 0xffu;
        }
        const f16x8 a = __builtin_bit_cast(f16x8, expand[byte]);
#pragma unroll
        for (int nt = 0; nt < kMaxNT; ++nt)
          if (nt < NT)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a, __builtin_bit_cast(f16x8, mfrag[(kb * NT + nt) * 64 + lane]), acc[nt], 0, 0,
                0);
      }
#pragma unroll
      for (int nt = 0; nt < kMaxNT; ++nt) {
        const int c = 16 * nt + rl;
        if (nt < NT && c < d) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            stage[(4 * q + e) * span_pad + gl * d + c] = float_to_f16_bits_rne(sr[e] * acc[nt][e]);
        }
      }
    }
    wave_sync();
    // rows row0 .. row0 + 15, columns gs d .. (gs + cnt) d as contiguous runs
    const int span = cnt * d;
    const int64_t col0 = gs * d;
    const bool vec = (col0 % 8) == 0 && (span % 8) == 0 && (n % 8) == 0;
    for (int r = 0; r < 16; ++r) {
      if (row0 + r >= m) break;
      uint16_t* dst = out + (row0 + r) * n + col0;
      const uint16_t* sp = stage + r * span_pad;
      if (vec) {
        for (int e = 8 * lane; e < span; e += 8 * 64)
          *reinterpret_cast<u32x4*>(dst + e) = *reinterpret_cast<const u32x4*>(sp + e);
      } else {
        for (int e = lane; e < span; e += 64) dst[e] = sp[e];
      }
    }
    wave_sync();
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

// Sub-slices: at most kSubWords sign words per row staged, at most kSpan
// decoded float16 per row staged.
constexpr int kSubWords = 96;

size_t decode_lds_bytes(int d, int D, int sub_groups, int words) {
  const int KB = (D + 31) / 32;
  const int NT = (d + 15) / 16;
  const int span_pad = (sub_groups * d + 7) & ~7;
  return 16 * (256 + static_cast<size_t>(KB) * NT * 64) +
         4 * static_cast<size_t>(kWaves) * 16 * words +
         2 * static_cast<size_t>(kWaves) * 16 * span_pad;
}

void decode_sub(int d, int D, int* sub_groups, int* words) {
  int sg = std::max(1, std::min(kSpan / d, ((kSubWords - 2) * 32) / D));
  *sub_groups = sg;
  *words = (sg * D + 31) / 32 + 2;
}

hipError_t launch_decode(const uint32_t* w, int64_t rows, int64_t ldw, int64_t gpr,
                         const float* M, int d, int D, const float* s, uint16_t* out, int64_t n,
                         hipStream_t st) {
  int sub_groups, words;
  decode_sub(d, D, &sub_groups, &words);
  const size_t lds = decode_lds_bytes(d, D, sub_groups, words);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_mfma_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  // slices of groups: about 16 waves per compute unit over the chunk
  const int64_t blocks = (rows + 15) / 16;
  const int64_t want = std::max<int64_t>(1, 16 * num_cus() / blocks);
  const int64_t per_wave = std::max<int64_t>(1, (gpr + want - 1) / want);
  const int64_t slices = (gpr + per_wave - 1) / per_wave;
  const int64_t by = (slices + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3(static_cast<unsigned>(blocks),
                                              static_cast<unsigned>(by)),
                     dim3(64 * kWaves), lds, st, w, rows, ldw, gpr, per_wave, sub_groups, words,
                     M, d, D, s, out, n);
  return hipGetLastError();
}

}  // namespace

bool gemm_decoded_shape_ok(int d, int D) { return d <= 16 * kMaxNT && D <= 32 * kMaxKB; }

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
    e = launch_decode(wc, rows, ldw, gpr, M, d, D, s + r0, wh, n, st);
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
