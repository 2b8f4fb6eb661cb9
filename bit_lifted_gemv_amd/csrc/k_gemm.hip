// Large-batch product on the matrix cores:
//   out[b][i] = s[i] * sum_k sigma_ik * a_hat[b][k]
// (LiftQuant notes, 关键设计 4: a product of 1-bit weights with floats; with a
// few hundred tokens it is a dense contraction, so it runs on MFMA).
//
// Signs are expanded in registers to exact 16-bit +-1 values (f16 or bf16,
// matching the lifted activations) and fed as the A operand of
// v_mfma_f32_32x32x16; the lifted activations are the B operand, staged
// through LDS.  Accumulation is float32.
//
// Expansion of one weight byte (8 lifted positions of one row, the A operand
// of one lane for one MFMA) into four dwords of two 16-bit values:
//   rep = byte | byte << 16                (v_perm_b32)
//   h   = rep << (15-2p, 14-2p) per half   (v_pk_lshlrev_b16: bit 2p -> bit 15,
//                                           bit 2p+1 -> bit 31)
//   dword_p = (h & 0x80008000) | ONE_ONE   (v_and_or_b32)
// A set bit sets the sign, so the tile holds -sigma; the epilogue multiplies
// by -s.
//
// Tiling: 128 rows x 128 tokens per workgroup, 4 waves in 2 x 2, each wave
// 64 x 64 (2 x 2 MFMA tiles of 32 x 32), k-step 32 per main-loop iteration,
// activations double-buffered in LDS.
#include "lq_internal.h"

namespace lq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 32;
constexpr int kThreads = 256;
constexpr int kLdsRow = kBK + 8;   // 16-bit elements per LDS row (80 B: conflict-free b128 reads)

template <int DT>
struct Mfma;

template <>
struct Mfma<LQ_F16> {
  static constexpr uint32_t kOneOne = 0x3C003C00u;
  __device__ static f32x16 run(const uint4& a, const uint4& b, const f32x16& c) {
    half8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
  }
};

template <>
struct Mfma<LQ_BF16> {
  static constexpr uint32_t kOneOne = 0x3F803F80u;
  __device__ static f32x16 run(const uint4& a, const uint4& b, const f32x16& c) {
    bf8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
  }
};

// Byte `byte_idx` of `word` -> 8 16-bit values -sigma (bit 1 -> -1, bit 0 -> +1).
template <int DT>
__device__ __forceinline__ uint4 expand_byte(uint32_t word, int byte_idx) {
  const uint32_t selr = static_cast<uint32_t>(byte_idx) | 0x0C000C00u |
                        (static_cast<uint32_t>(byte_idx) << 16);
  const uint32_t rep = __builtin_amdgcn_perm(0u, word, selr);   // [x, 0, x, 0]
  us2 r;
  __builtin_memcpy(&r, &rep, 4);
  uint32_t d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    us2 sh = {static_cast<unsigned short>(15 - 2 * p), static_cast<unsigned short>(14 - 2 * p)};
    const us2 h = r << sh;
    uint32_t hv;
    __builtin_memcpy(&hv, &h, 4);
    d[p] = (hv & 0x80008000u) | Mfma<DT>::kOneOne;
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

template <int DT>
__global__ void __launch_bounds__(kThreads) gemm_mfma_kernel(
    const uint32_t* __restrict__ w, int m, int K, int64_t ldw, const float* __restrict__ s,
    const uint16_t* __restrict__ ah, int B, float* __restrict__ out) {
  __shared__ uint16_t sB[2][kBN * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int row0 = blockIdx.x * kBM;
  const int tok0 = blockIdx.y * kBN;
  const int hi = lane >> 5;         // k-half of the MFMA operands
  const int l32 = lane & 31;

  // activation tile loader: thread -> (token, 16 k)
  const int ld_tok = tid >> 1;
  const int ld_k = (tid & 1) * 16;
  const bool tok_ok = (tok0 + ld_tok) < B;
  const uint16_t* ah_row = ah + (int64_t)(tok0 + ld_tok) * K;

  // weight rows of this lane (A operand rows of the two 32-row MFMA tiles)
  const int64_t arow0 = row0 + wm * 64 + l32;
  const int64_t arow1 = arow0 + 32;
  const bool ar0 = arow0 < m, ar1 = arow1 < m;
  const uint32_t* wr0 = w + arow0 * ldw;
  const uint32_t* wr1 = w + arow1 * ldw;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int ktiles = (K + kBK - 1) / kBK;

  auto load_b = [&](int kt, uint4& v0, uint4& v1) {
    const int k = kt * kBK + ld_k;
    v0 = make_uint4(0, 0, 0, 0);
    v1 = make_uint4(0, 0, 0, 0);
    if (tok_ok) {
      if (k + 8 <= K) v0 = *reinterpret_cast<const uint4*>(ah_row + k);
      if (k + 16 <= K) v1 = *reinterpret_cast<const uint4*>(ah_row + k + 8);
    }
  };
  auto store_b = [&](int buf, const uint4& v0, const uint4& v1) {
    uint4* dst = reinterpret_cast<uint4*>(&sB[buf][ld_tok * kLdsRow + ld_k]);
    dst[0] = v0;
    dst[1] = v1;
  };
  auto load_a = [&](int kt, uint32_t& a0, uint32_t& a1) {
    const int64_t wc = kt;            // one 32-bit word = 32 lifted positions = one k-tile
    a0 = (ar0 && wc < ldw) ? wr0[wc] : 0u;
    a1 = (ar1 && wc < ldw) ? wr1[wc] : 0u;
  };

  uint4 nb0, nb1;
  uint32_t na0, na1;
  load_b(0, nb0, nb1);
  load_a(0, na0, na1);
  store_b(0, nb0, nb1);
  __syncthreads();

  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    const uint32_t wa0 = na0, wa1 = na1;
    if (kt + 1 < ktiles) {
      load_b(kt + 1, nb0, nb1);
      load_a(kt + 1, na0, na1);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // B operands: token tok = wn*64 + ni*32 + l32, k = kk*16 + hi*8 .. +8
      uint4 bf[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int tok = wn * 64 + ni * 32 + l32;
        bf[ni] = *reinterpret_cast<const uint4*>(&sB[buf][tok * kLdsRow + kk * 16 + hi * 8]);
      }
      const int byte_idx = kk * 2 + hi;   // lifted positions kk*16 + hi*8 .. +8 of the word
      const uint4 af0 = expand_byte<DT>(wa0, byte_idx);
      const uint4 af1 = expand_byte<DT>(wa1, byte_idx);
      acc[0][0] = Mfma<DT>::run(af0, bf[0], acc[0][0]);
      acc[0][1] = Mfma<DT>::run(af0, bf[1], acc[0][1]);
      acc[1][0] = Mfma<DT>::run(af1, bf[0], acc[1][0]);
      acc[1][1] = Mfma<DT>::run(af1, bf[1], acc[1][1]);
    }
    if (kt + 1 < ktiles) {
      store_b(buf ^ 1, nb0, nb1);
      __syncthreads();
    }
  }

  // epilogue: D[i][j], i = row within the 32x32 tile, j = token; lane holds
  // j = l32 and rows 8*(e/4) + 4*hi + (e%4) for e = 0..15.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int tok = tok0 + wn * 64 + ni * 32 + l32;
      if (tok >= B) continue;
      float* orow = out + (int64_t)tok * m;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row0 + wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (row < m) orow[row] = -s[row] * acc[mi][ni][e];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                       const void* a_lift, lq_dtype dt, int64_t B, float* out, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((m + kBM - 1) / kBM),
                  static_cast<unsigned>((B + kBN - 1) / kBN));
  const uint16_t* ah = static_cast<const uint16_t*>(a_lift);
  if (dt == LQ_F16)
    hipLaunchKernelGGL(gemm_mfma_kernel<LQ_F16>, grid, dim3(kThreads), 0, st, w,
                       static_cast<int>(m), static_cast<int>(K), ldw, s, ah, static_cast<int>(B),
                       out);
  else
    hipLaunchKernelGGL(gemm_mfma_kernel<LQ_BF16>, grid, dim3(kThreads), 0, st, w,
                       static_cast<int>(m), static_cast<int>(K), ldw, s, ah, static_cast<int>(B),
                       out);
  return hipGetLastError();
}

}  // namespace lq
