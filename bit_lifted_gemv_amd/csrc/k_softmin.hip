// Learning the projection M of the LiftQuant notes (关键设计 2): the
// nearest-point objective E_w[min_y ||w - M y||] over Gaussian samples with
// the inner argmin replaced by a soft-argmin at temperature T (10 in the
// notes), differentiable in M.  For a batch W [N][d] and all 2^D codes y_t
// (y_tj = +1 iff bit j of t is set):
//   e_nt = ||w_n - C_t||^2 with C_t = M y_t,  p_nt = softmax_t(-T e_nt),
//   y_hat_n = sum_t p_nt y_t,  r_n = w_n - M y_hat_n,
//   loss = (1/N) sum_n ||r_n||^2,
//   grad = (1/N) [ -2 sum_n r_n y_hat_n^T
//                  + 2T sum_t (sum_n b_nt w_n - beta_t C_t) y_t^T ],
//   g_n = -2 M^T r_n, b_nt = p_nt (g_n . y_t - g_n . y_hat_n),
//   beta_t = sum_n b_nt.
// (The chain rule through y_hat = P Y and P = softmax(-T E).)
//
// Four kernels, float32, vector ALU (the per-pair work is a d-term distance,
// an exponential and D signed adds; no dense product large enough for the
// matrix cores):
//   fwd_partial: lane = sample, workgroup = 256 samples x one slice of the
//     codes, walked in Gray-code order so C_t moves by one column of M per
//     step (exact every 64 steps).  A running minimum e_min with rescaling
//     keeps every exponent <= 0; sums fold from 64-step chunks into totals.
//     Within a chunk the code bits >= 6 do not change, so their sums of p
//     are the chunk's sum of p: only the six low bits are summed per code.
//     Writes (e_min, Z, sum p [bit j]) per slice and sample.
//   fwd_merge: lane = sample; merges the slices, forms y_hat, r, g, g . y_hat
//     and the loss, keeps (e_min, 1/Z, g . y_hat, g) per sample, and sums the
//     workgroup's -2 r y_hat^T and loss.
//   bwd: lane = code t, workgroup = 256 codes x one slice of the samples
//     (staged in LDS, read as broadcasts); accumulates beta_t and
//     sum_n b_nt w_n, then sums 2T (sum b w - beta C_t) y_t^T over its codes.
//     The code bits >= 8 are those of the workgroup, so g_n . y_t over them
//     is formed once per staged sample; a pair adds only the 8 low bits.
//   reduce: the forward and backward partial rows are added column-wise by
//     a fixed tree (16 rows per node, consecutive rows, left to right),
//     then one small kernel forms the loss and the gradient.
// Everything is deterministic (fixed partition, fixed summation order).
#include <cmath>

#include "lq_internal.h"

namespace lq {
namespace {

constexpr int kT = 256;
constexpr int kLowBits = 6;
constexpr uint32_t kResync = 1u << kLowBits;   // Gray-code steps between exact recomputations
constexpr int kMaxBits = 24;

using f32x4 = float __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float expf_fast(float x) { return __expf(x); }

// mt[j][r] = M[r][j] (zero past d or D) into LDS; rows of DM floats.
template <int DM, int XM>
__device__ __forceinline__ void stage_m(const float* __restrict__ M, int d, int D,
                                        float (*mt)[DM]) {
  for (int e = threadIdx.x; e < XM * DM; e += kT) {
    const int j = e / DM;
    const int r = e - j * DM;
    mt[j][r] = (r < d && j < D) ? M[r * D + j] : 0.f;
  }
}

// acc[r] += s * mt[j][r] for r < DM
template <int DM>
__device__ __forceinline__ void axpy_col(float (&acc)[DM], float s, const float* col) {
#pragma unroll
  for (int r4 = 0; r4 < DM / 4; ++r4) {
    const f32x4 c = *reinterpret_cast<const f32x4*>(col + 4 * r4);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[4 * r4 + q] = fmaf(s, c[q], acc[4 * r4 + q]);
  }
}

template <int DM, int XM>
__global__ void __launch_bounds__(kT) softmin_fwd_partial_kernel(
    const float* __restrict__ W, int N, const float* __restrict__ M, int d, int D, float T,
    uint32_t slice_len, float* __restrict__ part) {
  __shared__ __align__(16) float mt[XM][DM];
  stage_m<DM, XM>(M, d, D, mt);
  __syncthreads();
  const int n = blockIdx.x * kT + threadIdx.x;
  const bool act = n < N;
  float w[DM];
#pragma unroll
  for (int r = 0; r < DM; ++r) w[r] = (act && r < d) ? W[static_cast<int64_t>(n) * d + r] : 0.f;

  float c[DM];
  auto exact_c = [&](uint32_t t) {
#pragma unroll
    for (int r = 0; r < DM; ++r) c[r] = 0.f;
#pragma unroll 1
    for (int j = 0; j < D; ++j) axpy_col<DM>(c, (t >> j) & 1u ? 1.f : -1.f, &mt[j][0]);
  };
  const float kInf = __builtin_inff();
  float emin = kInf, Z = 0.f, zl = 0.f;
  float num[XM], numl[kLowBits];
#pragma unroll
  for (int j = 0; j < XM; ++j) num[j] = 0.f;
#pragma unroll
  for (int j = 0; j < kLowBits; ++j) numl[j] = 0.f;
  // Close a chunk whose codes share their bits >= kLowBits with tp: those
  // bits' sums are the chunk's sum of p, the low bits' were kept per code.
  auto fold = [&](uint32_t tp) {
#pragma unroll
    for (int j = 0; j < XM; ++j) {
      if (j < kLowBits) {
        num[j] += numl[j];
        numl[j] = 0.f;
      } else if (j < D && ((tp >> j) & 1u)) {
        num[j] += zl;
      }
    }
    Z += zl;
    zl = 0.f;
  };
  uint32_t t = blockIdx.y * slice_len;
  for (uint32_t i = 0; i < slice_len; ++i) {
    int k = 0;
    if (i) {
      k = __builtin_ctz(i);
      t ^= 1u << k;
    }
    if (i % kResync == 0) {
      fold(t ^ (i ? 1u << k : 0u));                 // the last code of the chunk that ends here
      exact_c(t);
    } else {
      axpy_col<DM>(c, (t >> k) & 1u ? 2.f : -2.f, &mt[k][0]);
    }
    float e = 0.f;
#pragma unroll
    for (int r = 0; r < DM; ++r) {
      const float dr = w[r] - c[r];
      e = fmaf(dr, dr, e);
    }
    if (e < emin) {                                 // rescale what is summed to the new minimum
      const float sc = emin == kInf ? 0.f : expf_fast(-T * (emin - e));
      Z *= sc;
      zl *= sc;
#pragma unroll
      for (int j = 0; j < XM; ++j) num[j] *= sc;
#pragma unroll
      for (int j = 0; j < kLowBits; ++j) numl[j] *= sc;
      emin = e;
    }
    const float p = expf_fast(-T * (e - emin));
    zl += p;
#pragma unroll
    for (int j = 0; j < kLowBits; ++j)
      if (j < D) numl[j] = fmaf((t >> j) & 1u ? 1.f : 0.f, p, numl[j]);
  }
  fold(t);
  if (!act) return;
  float* o = part + (static_cast<int64_t>(blockIdx.y) * N + n) * (D + 2);
  o[0] = emin;
  o[1] = Z;
  for (int j = 0; j < D; ++j) o[2 + j] = num[j];
}

// Sum over the workgroup's 256 lanes of a[lane][r] * b[lane][j] (r < d,
// j < D) into out[r * D + j], staged through LDS (sa, sb hold 256 rows).
template <int DM, int XM>
__device__ __forceinline__ void block_outer_sum(const float (&a)[DM], const float (&b)[XM], int d,
                                                int D, float scale, float (*sa)[DM + 1],
                                                float (*sb)[XM + 1], float* __restrict__ out) {
#pragma unroll
  for (int r = 0; r < DM; ++r) sa[threadIdx.x][r] = a[r];
#pragma unroll
  for (int j = 0; j < XM; ++j) sb[threadIdx.x][j] = b[j];
  __syncthreads();
  for (int e = threadIdx.x; e < d * D; e += kT) {
    const int r = e / D;
    const int j = e - r * D;
    float s = 0.f;
    for (int l = 0; l < kT; ++l) s = fmaf(sa[l][r], sb[l][j], s);
    out[e] = scale * s;
  }
}

template <int DM, int XM>
__global__ void __launch_bounds__(kT) softmin_fwd_merge_kernel(
    const float* __restrict__ W, int N, const float* __restrict__ M, int d, int D, float T,
    int S, const float* __restrict__ part, float* __restrict__ samp,
    float* __restrict__ fpart) {
  __shared__ __align__(16) float mt[XM][DM];
  __shared__ float sa[kT][DM + 1];
  __shared__ float sb[kT][XM + 1];
  __shared__ float sl[kT];
  stage_m<DM, XM>(M, d, D, mt);
  __syncthreads();
  const int n = blockIdx.x * kT + threadIdx.x;
  const bool act = n < N;
  float r[DM], yh[XM];
#pragma unroll
  for (int q = 0; q < DM; ++q) r[q] = 0.f;
#pragma unroll
  for (int j = 0; j < XM; ++j) yh[j] = 0.f;
  float loss = 0.f;
  if (act) {
    float emin = __builtin_inff();
    for (int s = 0; s < S; ++s)
      emin = fminf(emin, part[(static_cast<int64_t>(s) * N + n) * (D + 2)]);
    float Z = 0.f;
    float num[XM];
#pragma unroll
    for (int j = 0; j < XM; ++j) num[j] = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* p = part + (static_cast<int64_t>(s) * N + n) * (D + 2);
      const float sc = p[0] == __builtin_inff() ? 0.f : expf_fast(-T * (p[0] - emin));
      Z = fmaf(sc, p[1], Z);
#pragma unroll
      for (int j = 0; j < XM; ++j)
        if (j < D) num[j] = fmaf(sc, p[2 + j], num[j]);
    }
    const float rz = 1.f / Z;
#pragma unroll
    for (int j = 0; j < XM; ++j) yh[j] = j < D ? fmaf(2.f * num[j], rz, -1.f) : 0.f;
#pragma unroll
    for (int q = 0; q < DM; ++q) r[q] = q < d ? W[static_cast<int64_t>(n) * d + q] : 0.f;
#pragma unroll 1
    for (int j = 0; j < D; ++j) axpy_col<DM>(r, -yh[j], &mt[j][0]);
    float gy = 0.f;
    float* o = samp + static_cast<int64_t>(n) * (D + 3);
    for (int j = 0; j < D; ++j) {
      float g = 0.f;
#pragma unroll
      for (int q = 0; q < DM; ++q) g = fmaf(mt[j][q], r[q], g);
      g *= -2.f;
      o[3 + j] = g;
      gy = fmaf(g, yh[j], gy);
    }
    o[0] = emin;
    o[1] = rz;
    o[2] = gy;
#pragma unroll
    for (int q = 0; q < DM; ++q) loss = fmaf(r[q], r[q], loss);
  }
  sl[threadIdx.x] = loss;
  float* out = fpart + static_cast<int64_t>(blockIdx.x) * (1 + d * D);
  block_outer_sum<DM, XM>(r, yh, d, D, -2.f, sa, sb, out + 1);
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int l = 0; l < kT; ++l) s += sl[l];
    out[0] = s;
  }
}

template <int DM, int XM>
__global__ void __launch_bounds__(kT) softmin_bwd_kernel(
    const float* __restrict__ W, int N, const float* __restrict__ M, int d, int D, float T,
    int n_slice, const float* __restrict__ samp, float* __restrict__ bpart) {
  __shared__ __align__(16) float mt[XM][DM];
  // one pool: the staged samples (sw, sg, se, srz, sgy, sgh) during the loop,
  // the outer-sum rows (sa, sb) after it
  __shared__ __align__(16) float pool[kT * (DM + XM + 4)];
  float(*sw)[DM] = reinterpret_cast<float(*)[DM]>(pool);
  float(*sg)[XM] = reinterpret_cast<float(*)[XM]>(pool + kT * DM);
  float* se = pool + kT * (DM + XM);
  float* srz = se + kT;
  float* sgy = srz + kT;
  // g_n . y_t over the code bits >= kLowJ, the same for the workgroup's 256
  // codes (bits >= 8 of t are those of blockIdx.x)
  float* sgh = sgy + kT;
  constexpr int kLowJ = XM < 8 ? XM : 8;
  const uint32_t tblk = blockIdx.x * kT;
  float(*sa)[DM + 1] = reinterpret_cast<float(*)[DM + 1]>(pool);
  float(*sb)[XM + 1] = reinterpret_cast<float(*)[XM + 1]>(pool + kT * (DM + 1));
  stage_m<DM, XM>(M, d, D, mt);
  __syncthreads();
  const uint32_t t = blockIdx.x * kT + threadIdx.x;
  const bool act = t < (1u << D);
  float ys[XM];
#pragma unroll
  for (int j = 0; j < XM; ++j) ys[j] = j < D ? ((t >> j) & 1u ? 1.f : -1.f) : 0.f;
  float c[DM];
#pragma unroll
  for (int r = 0; r < DM; ++r) c[r] = 0.f;
#pragma unroll 1
  for (int j = 0; j < D; ++j) axpy_col<DM>(c, ys[j], &mt[j][0]);

  const int n0 = blockIdx.y * n_slice;
  const int n1 = min(N, n0 + n_slice);
  float beta = 0.f;
  float q[DM];
#pragma unroll
  for (int r = 0; r < DM; ++r) q[r] = 0.f;
  for (int base = n0; base < n1; base += kT) {
    const int cnt = min(kT, n1 - base);
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < cnt) {
      const int64_t n = base + threadIdx.x;
      const float* o = samp + n * (D + 3);
#pragma unroll
      for (int r = 0; r < DM; ++r) sw[threadIdx.x][r] = r < d ? W[n * d + r] : 0.f;
#pragma unroll
      for (int j = 0; j < XM; ++j) sg[threadIdx.x][j] = j < D ? o[3 + j] : 0.f;
      se[threadIdx.x] = o[0];
      srz[threadIdx.x] = o[1];
      sgy[threadIdx.x] = o[2];
      float hi = 0.f;
#pragma unroll
      for (int j = kLowJ; j < XM; ++j)
        if (j < D) hi = fmaf((tblk >> j) & 1u ? 1.f : -1.f, o[3 + j], hi);
      sgh[threadIdx.x] = hi;
    }
    __syncthreads();
    float bl = 0.f;
    float ql[DM];
#pragma unroll
    for (int r = 0; r < DM; ++r) ql[r] = 0.f;
    for (int u = 0; u < cnt; ++u) {
      float wv[DM];
      float e = 0.f;
#pragma unroll
      for (int r4 = 0; r4 < DM / 4; ++r4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&sw[u][4 * r4]);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          wv[4 * r4 + qq] = x[qq];
          const float dr = x[qq] - c[4 * r4 + qq];
          e = fmaf(dr, dr, e);
        }
      }
      float a = sgh[u];
#pragma unroll
      for (int j4 = 0; j4 < kLowJ / 4; ++j4) {
        const f32x4 g = *reinterpret_cast<const f32x4*>(&sg[u][4 * j4]);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) a = fmaf(ys[4 * j4 + qq], g[qq], a);
      }
      const float p = expf_fast(-T * (e - se[u])) * srz[u];
      const float b = p * (a - sgy[u]);
      bl += b;
#pragma unroll
      for (int r = 0; r < DM; ++r) ql[r] = fmaf(b, wv[r], ql[r]);
    }
    beta += bl;
#pragma unroll
    for (int r = 0; r < DM; ++r) q[r] += ql[r];
  }
  float qd[DM];
#pragma unroll
  for (int r = 0; r < DM; ++r) qd[r] = act ? fmaf(-beta, c[r], q[r]) : 0.f;
  __syncthreads();
  block_outer_sum<DM, XM>(qd, ys, d, D, 2.f * T, sa, sb,
                          bpart + (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) *
                                      (d * D));
}

constexpr int kFan = 16;   // rows added per node of the reduction tree

// out[c][e] = in[kFan c][e] + ... + in[kFan c + kFan - 1][e] (rows past nrows
// count as absent), added left to right.  Row c of the output per blockIdx.x,
// columns in blocks of kT per blockIdx.y; all of a lane's loads are issued
// before the first add.
__global__ void __launch_bounds__(kT) softmin_sum_rows_kernel(const float* __restrict__ in,
                                                              int nrows, int ncols,
                                                              float* __restrict__ out) {
  const int e = blockIdx.y * kT + threadIdx.x;
  if (e >= ncols) return;
  const int r0 = blockIdx.x * kFan;
  float v[kFan];
#pragma unroll
  for (int u = 0; u < kFan; ++u)
    v[u] = r0 + u < nrows ? in[static_cast<int64_t>(r0 + u) * ncols + e] : 0.f;
  float sum = v[0];
#pragma unroll
  for (int u = 1; u < kFan; ++u) sum += v[u];
  out[static_cast<int64_t>(blockIdx.x) * ncols + e] = sum;
}

// f: the summed forward row (loss, then d D gradient terms); b: the summed
// backward row (d D terms).
__global__ void __launch_bounds__(kT) softmin_final_kernel(const float* __restrict__ f,
                                                           const float* __restrict__ b, int dD,
                                                           float inv_n, float* __restrict__ loss,
                                                           float* __restrict__ grad) {
  for (int e = threadIdx.x; e < dD; e += kT) grad[e] = (f[1 + e] + b[e]) * inv_n;
  if (threadIdx.x == 0) *loss = f[0] * inv_n;
}

__global__ void __launch_bounds__(kT) adam_kernel(float* __restrict__ M,
                                                  const float* __restrict__ g,
                                                  float* __restrict__ m1, float* __restrict__ m2,
                                                  int64_t count, float lr, float b1, float b2,
                                                  float c1, float c2, float eps) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kT + threadIdx.x;
  if (i >= count) return;
  const float gi = g[i];
  const float a = fmaf(b1, m1[i], (1.f - b1) * gi);
  const float v = fmaf(b2, m2[i], (1.f - b2) * gi * gi);
  m1[i] = a;
  m2[i] = v;
  M[i] -= lr * (a * c1) / (sqrtf(v * c2) + eps);
}

struct Plan {
  int S;            // code slices of the forward
  uint32_t slice;   // codes per slice (power of two)
  int nfw;          // forward workgroups (sample tiles)
  int nbx;          // backward code tiles
  int nby;          // backward sample slices
  int n_slice;      // samples per backward slice
};

Plan plan(int64_t N, int D) {
  Plan p;
  const int cus = num_cus();
  const uint32_t nc = 1u << D;
  p.nfw = static_cast<int>((N + kT - 1) / kT);
  p.S = 1;
  while (p.nfw * p.S < 8 * cus && (nc / (2 * p.S)) >= 64) p.S *= 2;
  p.slice = nc / p.S;
  p.nbx = static_cast<int>((nc + kT - 1) / kT);
  p.nby = 1;
  const int tiles = p.nfw;
  while (p.nbx * p.nby < 8 * cus && p.nby * 2 <= tiles) p.nby *= 2;
  p.n_slice = static_cast<int>(((N + p.nby - 1) / p.nby + kT - 1) / kT * kT);
  p.nby = static_cast<int>((N + p.n_slice - 1) / p.n_slice);
  return p;
}

struct Layout {
  size_t part, samp, fpart, bpart, ftree, btree, total;   // float offsets
};

// Floats of the two ping-pong buffers of a reduction of `rows` rows of
// `cols`: the first level's output and the second's.
size_t tree_floats(size_t rows, size_t cols) {
  const size_t l1 = (rows + kFan - 1) / kFan;
  const size_t l2 = (l1 + kFan - 1) / kFan;
  return (l1 + l2) * cols;
}

// Adds the rows of `in` column-wise, kFan rows per node, until one row
// remains; returns it (in `in` itself when rows == 1, else in `tree`).
const float* reduce_rows(const float* in, int rows, int cols, float* tree, hipStream_t st) {
  float* buf[2] = {tree, tree + static_cast<size_t>((rows + kFan - 1) / kFan) * cols};
  int k = 0;
  while (rows > 1) {
    const int out_rows = (rows + kFan - 1) / kFan;
    hipLaunchKernelGGL(softmin_sum_rows_kernel, dim3(out_rows, (cols + kT - 1) / kT), dim3(kT),
                       0, st, in, rows, cols, buf[k]);
    in = buf[k];
    k ^= 1;
    rows = out_rows;
  }
  return in;
}

Layout layout(int64_t N, int d, int D) {
  const Plan p = plan(N, D);
  Layout l;
  auto up = [](size_t x) { return (x + 63) / 64 * 64; };
  l.part = 0;
  l.samp = up(static_cast<size_t>(p.S) * N * (D + 2));
  l.fpart = l.samp + up(static_cast<size_t>(N) * (D + 3));
  l.bpart = l.fpart + up(static_cast<size_t>(p.nfw) * (1 + d * D));
  l.ftree = l.bpart + up(static_cast<size_t>(p.nbx) * p.nby * d * D);
  l.btree = l.ftree + up(tree_floats(p.nfw, 1 + d * D));
  l.total = l.btree + up(tree_floats(static_cast<size_t>(p.nbx) * p.nby, d * D));
  return l;
}

template <int DM, int XM>
hipError_t launch_dm(const float* W, int N, const float* M, int d, int D, float T, float* loss,
                     float* grad, float* ws, hipStream_t st) {
  const Plan p = plan(N, D);
  const Layout l = layout(N, d, D);
  hipLaunchKernelGGL((softmin_fwd_partial_kernel<DM, XM>), dim3(p.nfw, p.S), dim3(kT), 0, st, W,
                     N, M, d, D, T, p.slice, ws + l.part);
  hipLaunchKernelGGL((softmin_fwd_merge_kernel<DM, XM>), dim3(p.nfw), dim3(kT), 0, st, W, N, M,
                     d, D, T, p.S, ws + l.part, ws + l.samp, ws + l.fpart);
  hipLaunchKernelGGL((softmin_bwd_kernel<DM, XM>), dim3(p.nbx, p.nby), dim3(kT), 0, st, W, N, M,
                     d, D, T, p.n_slice, ws + l.samp, ws + l.bpart);
  const float* f = reduce_rows(ws + l.fpart, p.nfw, 1 + d * D, ws + l.ftree, st);
  const float* b = reduce_rows(ws + l.bpart, p.nbx * p.nby, d * D, ws + l.btree, st);
  hipLaunchKernelGGL(softmin_final_kernel, dim3(1), dim3(kT), 0, st, f, b, d * D,
                     1.f / static_cast<float>(N), loss, grad);
  return hipGetLastError();
}

}  // namespace

size_t softmin_workspace_bytes(int64_t N, int d, int D) {
  return (layout(N, d, D).total * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_softmin_grad(const float* W, int64_t N, const float* M, int d, int D, float T,
                               float* loss, float* grad, void* ws, hipStream_t st) {
  float* f = static_cast<float*>(ws);
  const int n = static_cast<int>(N);
  if (D <= 8) return launch_dm<8, 8>(W, n, M, d, D, T, loss, grad, f, st);
  if (D <= 16) {
    if (d <= 8) return launch_dm<8, 16>(W, n, M, d, D, T, loss, grad, f, st);
    return launch_dm<16, 16>(W, n, M, d, D, T, loss, grad, f, st);
  }
  if (d <= 8) return launch_dm<8, 24>(W, n, M, d, D, T, loss, grad, f, st);
  if (d <= 16) return launch_dm<16, 24>(W, n, M, d, D, T, loss, grad, f, st);
  return launch_dm<24, 24>(W, n, M, d, D, T, loss, grad, f, st);
}

hipError_t launch_adam(float* M, const float* g, float* m1, float* m2, int64_t count, int step,
                       float lr, float b1, float b2, float eps, hipStream_t st) {
  const double c1 = 1.0 / (1.0 - std::pow(static_cast<double>(b1), step));
  const double c2 = 1.0 / (1.0 - std::pow(static_cast<double>(b2), step));
  hipLaunchKernelGGL(adam_kernel, dim3(static_cast<unsigned>((count + kT - 1) / kT)), dim3(kT), 0,
                     st, M, g, m1, m2, count, lr, b1, b2, static_cast<float>(c1),
                     static_cast<float>(c2), eps);
  return hipGetLastError();
}

}  // namespace lq
