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
using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
using f32x4 = float __attribute__((ext_vector_type(4)));

using f16x8 = _Float16 __attribute__((ext_vector_type(8)));
constexpr int kWaves = 4;
constexpr int kMaxKB = 8;                   // D <= 256: k blocks of 32 signs
constexpr int kMaxNT = 4;                   // d <= 64: output tiles of 16 weights
constexpr int kSpan = 256;                  // decoded weights per row and sub-slice
constexpr int kGB = 4;                      // groups per step of the fixed-shape decode

// Byte `byte` (low 8 bits) -> 8 float16 values -sigma (bit 1: -1, bit 0: +1):
// one byte permute, then per pair a packed 16-bit shift that puts the bits at
// the sign positions and a bit select against +1.0 (mask and +1.0 are held
// where the compiler cannot fold them, so it emits v_and_or_b32 itself).
using us2 = unsigned short __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ u32x4 expand_signs(uint32_t byte, uint32_t sgn, uint32_t one) {
  const uint32_t rep = __builtin_amdgcn_perm(0u, byte, 0x0C000C00u);   // [x, 0, x, 0]
  us2 r;
  __builtin_memcpy(&r, &rep, 4);
  u32x4 d;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const us2 sh = {static_cast<unsigned short>(15 - 2 * p),
                    static_cast<unsigned short>(14 - 2 * p)};
    const us2 h = r << sh;
    uint32_t hv;
    __builtin_memcpy(&hv, &h, 4);
    d[p] = (hv & sgn) | (one & ~sgn);
  }
  return d;
}

// A wave decodes 16 rows x a slice of groups on the matrix cores: for group
// g the transposed weights W_hat^T[c][rows] = sum_j M[c][j] y[rows][g D + j]
// are one 16 x 16 x 32 float16 product per (tile of 16 weights c, k block of
// 32 signs), A = -M (fragments prepared in LDS, zero past d and D, so padded
// signs add nothing), B = the signs as -sigma (lane (l % 16, q = l / 16):
// row l % 16, signs 32 kb + 8 q .. + 7, one byte of the sign string).  The
// result lane holds weights 16 nt + 4 q + e (e < 4) of row l % 16: four
// consecutive float16 of one row, scaled by s and stored with one 8-byte
// store.  The slice is taken in sub-slices whose sign words (16 rows x a
// contiguous run each) are loaded into registers one sub-slice ahead and
// copied to LDS, so the group loop reads only LDS.
// Dynamic LDS: mfrag [KB NT 64] u32x4 | per wave: sign words [16][words] u32.
// KBT, NTT > 0: compile-time k blocks and tiles (the common shapes); a wave
// then decodes kGB groups per step as independent chains and keeps the M
// fragments in registers.  KBT = NTT = 0: any shape, one group per step.
template <int KBT, int NTT>
__global__ void __launch_bounds__(64 * kWaves) decode_mfma_kernel(
    const uint32_t* __restrict__ w, int64_t m, int64_t ldw, int64_t groups_per_row,
    int64_t groups_per_wave, int sub_groups, int words, const float* __restrict__ M, int d,
    int D, const float* __restrict__ s, uint16_t* __restrict__ out, int64_t n) {
  extern __shared__ u32x4 lds4[];
  constexpr bool kFixed = KBT > 0;
  const int KB = kFixed ? KBT : (D + 31) / 32;
  const int NT = kFixed ? NTT : (d + 15) / 16;
  u32x4* mfrag = lds4;
  uint32_t* sbits_all = reinterpret_cast<uint32_t*>(mfrag + KB * NT * 64);
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
        pair |= static_cast<uint32_t>(float_to_f16_bits_rne(in ? -x : 0.f)) << (16 * b);
      }
      v[h] = pair;
    }
    mfrag[e] = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  uint32_t* sbits = sbits_all + wave * 16 * words;       // [16][words]
  const int q = lane >> 4;
  const int rl = lane & 15;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t my_row = row0 + rl;
  const bool row_ok = my_row < m;
  const float srow = s[row_ok ? my_row : 0];
  uint16_t* orow = out + (row_ok ? my_row : 0) * n;
  const int64_t g0 = (static_cast<int64_t>(blockIdx.y) * kWaves + wave) * groups_per_wave;
  const int64_t g1 = min(groups_per_row, g0 + groups_per_wave);
  const uint32_t sgn = opaque(0x80008000u);
  const uint32_t one = opaque_v(0x3C003C00u);
  const bool vec_out = (d % 4) == 0 && (n % 4) == 0;
  // weights 16 nt + 4 q .. + 3 of group gl of the sub-slice at ob, row
  // my_row, from the result tile
  auto store4 = [&](uint16_t* ob, int gl, int nt, f32x4 acc) {
    const int c0 = 16 * nt + 4 * q;
    if (!row_ok || c0 >= d) return;
    uint16_t* dst = ob + gl * d + c0;
    if (vec_out) {                                  // c0 + 3 < d, 8-byte aligned
      u32x2 v;
      v[0] = float_to_f16_bits_rne(srow * acc[0]) | (float_to_f16_bits_rne(srow * acc[1]) << 16);
      v[1] = float_to_f16_bits_rne(srow * acc[2]) | (float_to_f16_bits_rne(srow * acc[3]) << 16);
      *reinterpret_cast<u32x2*>(dst) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c0 + e < d) dst[e] = float_to_f16_bits_rne(srow * acc[e]);
    }
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // sign words of rows row0 .. row0 + 15 covering the groups [gs, gs + cnt):
  // a word per lane and row, two passes when the run is longer than the wave
  uint32_t pre[2][16];
  auto prefetch = [&](int64_t gs_) {
    const int cnt_ = static_cast<int>(min<int64_t>(sub_groups, g1 - gs_));
    const int64_t w0_ = (gs_ * D) >> 5;
    const int wc_ = static_cast<int>((((gs_ + cnt_) * D - 1) >> 5) - w0_ + 1);   // <= words
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 64 * h + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool in = k < wc_ && row0 + r < m;
        pre[h][r] = w[in ? (row0 + r) * ldw + w0_ + k : 0];
      }
    }
  };
  if (g0 < g1) prefetch(g0);
  for (int64_t gs = g0; gs < g1; gs += sub_groups) {
    const int cnt = static_cast<int>(min<int64_t>(sub_groups, g1 - gs));
    const int64_t w0 = (gs * D) >> 5;
    const int wc = static_cast<int>((((gs + cnt) * D - 1) >> 5) - w0 + 1);
    wave_sync();                                    // the last sub-slice's reads are done
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 64 * h + lane;
      if (k < wc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sbits[r * words + k] = pre[h][r];
      }
    }
    wave_sync();
    if (gs + sub_groups < g1) prefetch(gs + sub_groups);
    // byte 4 kb + q of group g's sign string (bits past D are don't-care:
    // their M entries are zero)
    // (offsets relative to the sub-slice, in 32-bit arithmetic)
    const int bit_base = static_cast<int>(gs * D - w0 * 32);   // < 32
    uint16_t* obase = orow + gs * d;
    auto sign_byte = [&](int gl, int kb) -> uint32_t {
      const int j0 = 32 * kb + 8 * q;
      if (j0 >= D) return 0u;
      const int o = gl * D + j0 + bit_base;             // bit offset in the staged run
      const int wi = o >> 5;
      const uint32_t sh = static_cast<uint32_t>(o & 31);
      const int nb = min(8, D - j0);
      uint32_t v = sbits[rl * words + wi] >> sh;
      if (static_cast<int>(sh) + nb > 32) v |= sbits[rl * words + wi + 1] << (32 - sh);
      return v & 0xffu;
    };
    if constexpr (kFixed) {
      f16x8 afr[KBT][NTT];
#pragma unroll
      for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
        for (int nt = 0; nt < NTT; ++nt)
          afr[kb][nt] = __builtin_bit_cast(f16x8, mfrag[(kb * NTT + nt) * 64 + lane]);
      for (int gl0 = 0; gl0 < cnt; gl0 += kGB) {
        f16x8 y[kGB][KBT];
#pragma unroll
        for (int gi = 0; gi < kGB; ++gi)
#pragma unroll
          for (int kb = 0; kb < KBT; ++kb) {
            // past the sub-slice: any byte (the result is not stored)
            const int gl = min(gl0 + gi, cnt - 1);
            y[gi][kb] = __builtin_bit_cast(f16x8, expand_signs(sign_byte(gl, kb), sgn, one));
          }
#pragma unroll
        for (int gi = 0; gi < kGB; ++gi) {
#pragma unroll
          for (int nt = 0; nt < NTT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[kb][nt], y[gi][kb], acc, 0, 0, 0);
            if (gl0 + gi < cnt) store4(obase, gl0 + gi, nt, acc);
          }
        }
      }
    } else {
      for (int gl = 0; gl < cnt; ++gl) {
        f32x4 acc[kMaxNT];
#pragma unroll
        for (int nt = 0; nt < kMaxNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < KB; ++kb) {
          const f16x8 y = __builtin_bit_cast(f16x8, expand_signs(sign_byte(gl, kb), sgn, one));
#pragma unroll
          for (int nt = 0; nt < kMaxNT; ++nt)
            if (nt < NT)
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  __builtin_bit_cast(f16x8, mfrag[(kb * NT + nt) * 64 + lane]), y, acc[nt], 0, 0,
                  0);
        }
#pragma unroll
        for (int nt = 0; nt < kMaxNT; ++nt)
          if (nt < NT) store4(obase, gl, nt, acc[nt]);
      }
    }
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

// Sub-slices: at most kSubWords sign words per row staged and at most kSpan
// decoded weights per row (the groups of one sub-slice).
constexpr int kSubWords = 96;

size_t decode_lds_bytes(int d, int D, int sub_groups, int words) {
  (void)sub_groups;
  const int KB = (D + 31) / 32;
  const int NT = (d + 15) / 16;
  return 16 * static_cast<size_t>(KB) * NT * 64 + 4 * static_cast<size_t>(kWaves) * 16 * words;
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
  // slices of groups: about 16 waves per compute unit over the chunk
  const int64_t blocks = (rows + 15) / 16;
  const int64_t want = std::max<int64_t>(1, 16 * num_cus() / blocks);
  const int64_t per_wave = std::max<int64_t>(1, (gpr + want - 1) / want);
  const int64_t slices = (gpr + per_wave - 1) / per_wave;
  const int64_t by = (slices + kWaves - 1) / kWaves;
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(by));
  const int KB = (D + 31) / 32;
  const int NT = (d + 15) / 16;
  auto go = [&](auto kern) -> hipError_t {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(64 * kWaves), lds, st, w, rows, ldw, gpr, per_wave,
                       sub_groups, words, M, d, D, s, out, n);
    return hipGetLastError();
  };
  if (KB == 1 && NT == 1) return go(decode_mfma_kernel<1, 1>);
  if (KB == 1 && NT == 2) return go(decode_mfma_kernel<1, 2>);
  if (KB == 2 && NT == 1) return go(decode_mfma_kernel<2, 1>);
  if (KB == 2 && NT == 2) return go(decode_mfma_kernel<2, 2>);
  return go(decode_mfma_kernel<0, 0>);
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
