// Lattice encoder of the LiftQuant notes (关键设计 2): for each d-wide
// weight group w, the code y in {+-1}^D whose projection M y is nearest to w
// (M is d x D, 关键设计 1).
//   exhaustive: every code, 2^D candidates; candidate t has y_j = +1 iff bit
//               j of t is set.
//   search:     the pseudo-inverse start plus an auxiliary vector: with the
//               completion A ((D-d) x D, an input) and B = [M; A]^-1,
//               candidate t is y = sign(B [w; v]) with v_k = +1 iff bit k of
//               t is set, 2^(D-d) candidates.  For [M; A] orthogonal,
//               B [w; v] = M^+ w + A^T v.
// The candidate with the smallest ||w - M y||^2 wins, ties to the smallest
// t; sign(0) = +1.  float32 arithmetic; B is formed in float64.
//
// One wave per group.  Each lane walks a contiguous range of candidate
// indices in Gray-code order, so consecutive candidates differ in one bit k:
// the search moves B [w; v] by +-2 B[:, d + k] and the exhaustive walk moves
// the residual w - M y by -+2 M[:, k].  In the search such a step flips only
// a few signs of B [w; v] (about 4 of 32 for the table's codes), so the
// residual moves by -+2 M[:, j] for each flipped sign j instead of being
// formed anew (D d multiply-adds).  All running sums are recomputed exactly
// every 32 steps to bound their drift.  The wave then reduces the lanes'
// best (error, index) pairs.
#include "lq_internal.h"

namespace lq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxDim = 32;
constexpr int kMaxBits = 24;
constexpr uint32_t kResync = 32;

using f32x4 = float __attribute__((ext_vector_type(4)));

// B = [M; A]^-1 by Gauss-Jordan elimination with partial pivoting in float64,
// one wave.  A zero pivot (singular completion) leaves that column's
// multiplier 0 and the result unspecified but finite.
__global__ void __launch_bounds__(64) encode_inverse_kernel(const float* __restrict__ M,
                                                            const float* __restrict__ A, int d,
                                                            int D, float* __restrict__ binv) {
  __shared__ double a[kMaxDim][2 * kMaxDim + 1];
  __shared__ double f[kMaxDim];
  __shared__ int piv;
  const int l = threadIdx.x;
  const int W2 = 2 * D;
  for (int e = l; e < D * W2; e += 64) {
    const int r = e / W2;
    const int c = e - r * W2;
    double v;
    if (c < D)
      v = r < d ? static_cast<double>(M[r * D + c]) : static_cast<double>(A[(r - d) * D + c]);
    else
      v = (c - D == r) ? 1.0 : 0.0;
    a[r][c] = v;
  }
  __syncthreads();
  for (int col = 0; col < D; ++col) {
    if (l == 0) {
      int best = col;
      double bv = fabs(a[col][col]);
      for (int r = col + 1; r < D; ++r)
        if (fabs(a[r][col]) > bv) {
          bv = fabs(a[r][col]);
          best = r;
        }
      piv = best;
    }
    __syncthreads();
    const int p = piv;
    if (p != col)
      for (int c = l; c < W2; c += 64) {
        const double t = a[p][c];
        a[p][c] = a[col][c];
        a[col][c] = t;
      }
    __syncthreads();
    const double pv = a[col][col];
    const double inv = pv != 0.0 ? 1.0 / pv : 0.0;
    __syncthreads();
    for (int c = l; c < W2; c += 64) a[col][c] *= inv;
    for (int r = l; r < D; r += 64) f[r] = r == col ? 0.0 : a[r][col];
    __syncthreads();
    for (int e = l; e < D * W2; e += 64) {
      const int r = e / W2;
      const int c = e - r * W2;
      if (r != col) a[r][c] -= f[r] * a[col][c];
    }
    __syncthreads();
  }
  for (int e = l; e < D * D; e += 64) {
    const int r = e / D;
    binv[e] = static_cast<float>(a[r][D + e - r * D]);
  }
}

// DM >= d and XM >= D bound the register arrays (entries past d or D are
// zero); the loops over them are unrolled with uniform guards.
template <int DM, int XM, bool SEARCH>
__global__ void __launch_bounds__(kThreads) encode_kernel(
    const float* __restrict__ w, int64_t groups, const float* __restrict__ M,
    const float* __restrict__ binv, int d, int D, int8_t* __restrict__ codes,
    float* __restrict__ err) {
  __shared__ __align__(16) float mt[XM][DM];                     // mt[j][r] = M[r][j]
  __shared__ __align__(16) float bv[SEARCH ? kMaxBits : 1][XM];  // bv[k][j] = B[j][d + k]
  __shared__ __align__(16) float bw[SEARCH ? DM : 1][XM];        // bw[r][j] = B[j][r]
  const int kbits = SEARCH ? D - d : D;
  for (int e = threadIdx.x; e < XM * DM; e += kThreads) {
    const int j = e / DM;
    const int r = e - j * DM;
    mt[j][r] = (r < d && j < D) ? M[r * D + j] : 0.f;
  }
  if constexpr (SEARCH) {
    for (int e = threadIdx.x; e < kbits * XM; e += kThreads) {
      const int k = e / XM;
      const int j = e - k * XM;
      bv[k][j] = j < D ? binv[j * D + d + k] : 0.f;
    }
    for (int e = threadIdx.x; e < DM * XM; e += kThreads) {
      const int r = e / XM;
      const int j = e - r * XM;
      bw[r][j] = (r < d && j < D) ? binv[j * D + r] : 0.f;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  if (g >= groups) return;                          // no barrier follows

  float wr[DM];
#pragma unroll
  for (int r = 0; r < DM; ++r) wr[r] = r < d ? w[g * d + r] : 0.f;

  const uint32_t nc = 1u << kbits;
  const uint32_t R = nc >= 64 ? nc >> 6 : 1u;
  const uint32_t t0 = nc >= 64 ? static_cast<uint32_t>(lane) * R : static_cast<uint32_t>(lane);
  const bool active = nc >= 64 || static_cast<uint32_t>(lane) < nc;

  // residual w - M y for the sign mask m (bit j set: y_j = +1)
  float res[DM];
  auto exact_res = [&](uint32_t m) {
#pragma unroll
    for (int r = 0; r < DM; ++r) res[r] = wr[r];
    // a runtime loop over the columns: M stays in LDS (unrolled, every read
    // of it would be hoisted out of the candidate loop into registers)
#pragma unroll 1
    for (int j = 0; j < D; ++j) {
      const float s = (m >> j) & 1u ? -1.f : 1.f;
#pragma unroll
      for (int r4 = 0; r4 < DM / 4; ++r4) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(&mt[j][4 * r4]);
#pragma unroll
        for (int q = 0; q < 4; ++q) res[4 * r4 + q] = fmaf(s, c[q], res[4 * r4 + q]);
      }
    }
  };
  // search: the start B [w; 0] and the point B [w; v(t)]
  float c0[SEARCH ? XM : 1];
  float x[SEARCH ? XM : 1];
  if constexpr (SEARCH) {
#pragma unroll
    for (int j = 0; j < XM; ++j) c0[j] = 0.f;
#pragma unroll
    for (int r = 0; r < DM; ++r)
#pragma unroll
      for (int j4 = 0; j4 < XM / 4; ++j4) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(&bw[r][4 * j4]);
#pragma unroll
        for (int q = 0; q < 4; ++q) c0[4 * j4 + q] = fmaf(b[q], wr[r], c0[4 * j4 + q]);
      }
  }
  auto exact_x = [&](uint32_t t) {
    if constexpr (SEARCH) {
#pragma unroll
      for (int j = 0; j < XM; ++j) x[j] = c0[j];
#pragma unroll 1
      for (int k = 0; k < kbits; ++k) {
        const float s = (t >> k) & 1u ? 1.f : -1.f;
#pragma unroll
        for (int j4 = 0; j4 < XM / 4; ++j4) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(&bv[k][4 * j4]);
#pragma unroll
          for (int q = 0; q < 4; ++q) x[4 * j4 + q] = fmaf(s, b[q], x[4 * j4 + q]);
        }
      }
    }
  };

  float best_e = __builtin_inff();
  uint32_t best_t = 0xffffffffu;
  uint32_t best_m = 0;
  uint32_t mprev = 0;                              // mask that res belongs to (search)
  uint32_t t = t0;
  for (uint32_t i = 0; i < R; ++i) {
    int k = 0;
    if (i) {
      k = __builtin_ctz(i);
      t ^= 1u << k;
    }
    const bool resync = (i % kResync) == 0;
    uint32_t m;
    if constexpr (SEARCH) {
      if (resync) {
        exact_x(t);
      } else {
        const float s = (t >> k) & 1u ? 2.f : -2.f;
#pragma unroll
        for (int j4 = 0; j4 < XM / 4; ++j4) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(&bv[k][4 * j4]);
#pragma unroll
          for (int q = 0; q < 4; ++q) x[4 * j4 + q] = fmaf(s, b[q], x[4 * j4 + q]);
        }
      }
      m = 0;
#pragma unroll
      for (int j = 0; j < XM; ++j)
        if (j < D) m |= (x[j] >= 0.f ? 1u : 0u) << j;
      if (resync) {
        exact_res(m);
      } else {
        // one step of v moves x along one column of B, which flips only a
        // few signs (about 4 of 32): update the residual column by column
        for (uint32_t diff = m ^ mprev; diff; diff &= diff - 1) {
          const int j = __builtin_ctz(diff);
          const float sj = (m >> j) & 1u ? -2.f : 2.f;
#pragma unroll
          for (int r4 = 0; r4 < DM / 4; ++r4) {
            const f32x4 c = *reinterpret_cast<const f32x4*>(&mt[j][4 * r4]);
#pragma unroll
            for (int q = 0; q < 4; ++q) res[4 * r4 + q] = fmaf(sj, c[q], res[4 * r4 + q]);
          }
        }
      }
      mprev = m;
    } else {
      m = t;
      if (resync) {
        exact_res(m);
      } else {
        const float s = (t >> k) & 1u ? -2.f : 2.f;
#pragma unroll
        for (int r4 = 0; r4 < DM / 4; ++r4) {
          const f32x4 c = *reinterpret_cast<const f32x4*>(&mt[k][4 * r4]);
#pragma unroll
          for (int q = 0; q < 4; ++q) res[4 * r4 + q] = fmaf(s, c[q], res[4 * r4 + q]);
        }
      }
    }
    float e = 0.f;
#pragma unroll
    for (int r = 0; r < DM; ++r) e = fmaf(res[r], res[r], e);
    if (active && (e < best_e || (e == best_e && t < best_t))) {
      best_e = e;
      best_t = t;
      best_m = m;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float oe = __shfl_xor(best_e, off, 64);
    const uint32_t ot = __shfl_xor(best_t, off, 64);
    const uint32_t om = __shfl_xor(best_m, off, 64);
    if (oe < best_e || (oe == best_e && ot < best_t)) {
      best_e = oe;
      best_t = ot;
      best_m = om;
    }
  }
  if (lane < D) codes[g * D + lane] = (best_m >> lane) & 1u ? int8_t{1} : int8_t{-1};
  if (lane == 0 && err) err[g] = best_e;
}

template <int DM, int XM>
hipError_t launch_dm_xm(const float* w, int64_t groups, const float* M, const float* binv,
                        int d, int D, int8_t* codes, float* err, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((groups + kWaves - 1) / kWaves));
  if (binv)
    hipLaunchKernelGGL((encode_kernel<DM, XM, true>), grid, dim3(kThreads), 0, st, w, groups, M,
                       binv, d, D, codes, err);
  else
    hipLaunchKernelGGL((encode_kernel<DM, XM, false>), grid, dim3(kThreads), 0, st, w, groups, M,
                       binv, d, D, codes, err);
  return hipGetLastError();
}

}  // namespace

size_t encode_workspace_bytes(int D) {
  return (static_cast<size_t>(D) * D * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_encode(const float* w, int64_t groups, const float* M, const float* A, int d,
                         int D, int8_t* codes, float* err, void* ws, hipStream_t st) {
  if (groups == 0) return hipSuccess;
  float* binv = nullptr;
  if (A) {
    binv = static_cast<float*>(ws);
    hipLaunchKernelGGL(encode_inverse_kernel, dim3(1), dim3(64), 0, st, M, A, d, D, binv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (D <= 16) {
    if (d <= 8) return launch_dm_xm<8, 16>(w, groups, M, binv, d, D, codes, err, st);
    return launch_dm_xm<16, 16>(w, groups, M, binv, d, D, codes, err, st);
  }
  if (d <= 8) return launch_dm_xm<8, 32>(w, groups, M, binv, d, D, codes, err, st);
  if (d <= 16) return launch_dm_xm<16, 32>(w, groups, M, binv, d, D, codes, err, st);
  return launch_dm_xm<32, 32>(w, groups, M, binv, d, D, codes, err, st);
}

}  // namespace lq
