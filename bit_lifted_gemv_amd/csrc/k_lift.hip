// Activation lift: a_hat = (I (x) M^T) . blockdiag(T^-1) . a  (LiftQuant notes,
// 关键设计 4: the small transform of the activations done once per input;
// 关键设计 1 for the per-group M).  float32 accumulation throughout.
//
// One workgroup owns a run of whole groups (about 128 channels of u) and a
// chunk of tokens.  It stages the activation blocks its channels read in LDS,
// computes those u channels (each u channel is one 128-long dot product with a
// row of its T^-1 block, so groups that straddle two blocks need no special
// case), keeps u in LDS, and writes the lifted values of its groups.
#include "lq_internal.h"

namespace lq {
namespace {

constexpr int kTB = 128;      // transform block
constexpr int kThreads = 256;

template <int DT>
__device__ __forceinline__ void load8_as_float(const void* base, int64_t idx, float* v);

template <>
__device__ __forceinline__ void load8_as_float<LQ_BF16>(const void* base, int64_t idx, float* v) {
  const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8_as_float<LQ_F16>(const void* base, int64_t idx, float* v) {
  const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = f16_bits_to_float(static_cast<uint16_t>(w[i] & 0xFFFFu));
    v[2 * i + 1] = f16_bits_to_float(static_cast<uint16_t>(w[i] >> 16));
  }
}

template <>
__device__ __forceinline__ void load8_as_float<LQ_F32>(const void* base, int64_t idx, float* v) {
  const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
  const float4 x = p[0], y = p[1];
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}

// TBMAX: tokens handled per workgroup (compile-time bound of the register block).
template <int A_DT, int T_DT, int O_DT, int TBMAX>
__global__ void __launch_bounds__(kThreads) lift_kernel(const void* __restrict__ a,
                                                        const void* __restrict__ t_inv,
                                                        const float* __restrict__ M,
                                                        void* __restrict__ out, int B, int n,
                                                        int d, int D, int GW) {
  extern __shared__ float smem[];
  const int G = n / d;
  const int K = G * D;
  const int g0 = blockIdx.x * GW;
  const int gcount = min(GW, G - g0);
  const int c0 = g0 * d;
  const int cw = gcount * d;                     // channels of u owned here
  const int blk0 = c0 / kTB;
  const int nblk = (c0 + cw - 1) / kTB - blk0 + 1;
  const int b0 = blockIdx.y * TBMAX;
  const int bc = min(TBMAX, B - b0);

  float* sa = smem;                              // [TBMAX][nblk*128] activations
  float* su = sa + TBMAX * nblk * kTB;           // [TBMAX][cw] transformed
  float* sM = su + TBMAX * cw;                   // [d][D]

  const int tid = threadIdx.x;
  const int aw = nblk * kTB;
  for (int i = tid; i < bc * aw; i += kThreads) {
    const int b = i / aw;
    const int j = i - b * aw;
    sa[b * aw + j] = load_as_float<A_DT>(a, (int64_t)(b0 + b) * n + blk0 * kTB + j);
  }
  for (int i = tid; i < d * D; i += kThreads) sM[i] = M[i];
  __syncthreads();

  // u: thread (c, half) owns channel c0 + c and tokens b = half, half + H, ...
  constexpr int H = kThreads / kTB;              // 2 threads per channel
  const int c = tid % kTB;
  const int half = tid / kTB;
  if (c < cw) {
    const int ch = c0 + c;
    const int q = ch / kTB;
    const int r = ch - q * kTB;
    const int aoff = (q - blk0) * kTB;
    const int64_t trow = ((int64_t)q * kTB + r) * kTB;
    constexpr int NB = (TBMAX + H - 1) / H;
    float acc[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[i] = 0.f;
    for (int j = 0; j < kTB; j += 8) {
      float tv[8];
      load8_as_float<T_DT>(t_inv, trow + j, tv);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int b = half + H * i;
        if (b < bc) {
          const float* ab = sa + b * aw + aoff + j;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i] = fmaf(tv[e], ab[e], acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = half + H * i;
      if (b < bc) su[b * cw + c] = acc[i];
    }
  }
  __syncthreads();

  // a_hat for the groups of this workgroup: consecutive threads write
  // consecutive lifted positions of one token.
  const int ow = gcount * D;
  for (int i = tid; i < bc * ow; i += kThreads) {
    const int b = i / ow;
    const int rem = i - b * ow;
    const int g = rem / D;
    const int jj = rem - g * D;
    const float* ub = su + b * cw + g * d;
    float acc = 0.f;
    for (int rr = 0; rr < d; ++rr) acc = fmaf(sM[rr * D + jj], ub[rr], acc);
    store_from_float<O_DT>(out, (int64_t)(b0 + b) * K + (int64_t)g0 * D + rem, acc);
  }
}

template <int A_DT, int T_DT, int O_DT>
hipError_t launch_lift_t(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M,
                         int d, int D, void* out, hipStream_t st) {
  const int G = static_cast<int>(n / d);
  const int GW = kTB / d > 0 ? kTB / d : 1;           // about 128 channels per workgroup
  const int gx = (G + GW - 1) / GW;
  const int cwmax = GW * d;
  const int nblk = 2;                                 // cw <= 128 spans at most 2 blocks
  constexpr int TBMAX = 16;
  const int gy = static_cast<int>((B + TBMAX - 1) / TBMAX);
  const size_t lds = sizeof(float) * (TBMAX * nblk * kTB + TBMAX * cwmax + d * D);
  hipLaunchKernelGGL((lift_kernel<A_DT, T_DT, O_DT, TBMAX>), dim3(gx, gy), dim3(kThreads), lds,
                     st, a, t_inv, M, out, static_cast<int>(B), static_cast<int>(n), d, D, GW);
  return hipGetLastError();
}

template <int A_DT, int T_DT>
hipError_t dispatch_out(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M,
                        int d, int D, void* out, lq_dtype out_dt, hipStream_t st) {
  switch (out_dt) {
    case LQ_F32: return launch_lift_t<A_DT, T_DT, LQ_F32>(a, B, n, t_inv, M, d, D, out, st);
    case LQ_F16: return launch_lift_t<A_DT, T_DT, LQ_F16>(a, B, n, t_inv, M, d, D, out, st);
    default: return launch_lift_t<A_DT, T_DT, LQ_BF16>(a, B, n, t_inv, M, d, D, out, st);
  }
}

template <int A_DT>
hipError_t dispatch_t(const void* a, int64_t B, int64_t n, const void* t_inv, lq_dtype t_dt,
                      const float* M, int d, int D, void* out, lq_dtype out_dt, hipStream_t st) {
  switch (t_dt) {
    case LQ_F32: return dispatch_out<A_DT, LQ_F32>(a, B, n, t_inv, M, d, D, out, out_dt, st);
    case LQ_F16: return dispatch_out<A_DT, LQ_F16>(a, B, n, t_inv, M, d, D, out, out_dt, st);
    default: return dispatch_out<A_DT, LQ_BF16>(a, B, n, t_inv, M, d, D, out, out_dt, st);
  }
}

}  // namespace

hipError_t launch_lift(const void* a, lq_dtype a_dt, int64_t B, int64_t n, const void* t_inv,
                       lq_dtype t_dt, const float* M, int d, int D, void* out, lq_dtype out_dt,
                       hipStream_t st) {
  switch (a_dt) {
    case LQ_F32: return dispatch_t<LQ_F32>(a, B, n, t_inv, t_dt, M, d, D, out, out_dt, st);
    case LQ_F16: return dispatch_t<LQ_F16>(a, B, n, t_inv, t_dt, M, d, D, out, out_dt, st);
    default: return dispatch_t<LQ_BF16>(a, B, n, t_inv, t_dt, M, d, D, out, out_dt, st);
  }
}

}  // namespace lq
