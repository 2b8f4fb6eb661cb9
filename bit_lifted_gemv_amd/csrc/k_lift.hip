// Activation lift: a_hat = (I (x) M^T) . blockdiag(T^-1) . a  (LiftQuant notes,
// 关键设计 4: the small transform of the activations done once per input;
// 关键设计 1 for the per-group M).  float32 accumulation throughout.
//
// One workgroup owns a run of whole groups (about 32 channels of u, one
// group when d > 32) and a
// chunk of up to 16 tokens.  The T^-1 rows of its channels are contiguous in
// memory ([n/128][128][128], row r of block q is channel 128q + r), so it
// reads them with coalesced 16-byte loads, all issued before the first use:
// 16 lanes per row, 8 elements each.  Each lane dots its 8 elements with the
// matching activations (staged in LDS as float32), the 16 lanes of a row are
// combined by a shuffle tree, u goes to LDS, and the workgroup writes the
// lifted values of its groups (consecutive threads, consecutive positions).
// Groups may straddle two 128-blocks: each row reads the activations of its
// own block.
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

constexpr int kMaxRows = 64;                     // channels of u per workgroup (d <= 64)
constexpr int kPasses = kMaxRows / 16;           // 16 rows per pass of 256 threads

// TB: tokens per workgroup (1, 2, 4, 8 or 16).
template <int A_DT, int T_DT, int O_DT, int TB>
__global__ void __launch_bounds__(kThreads) lift_kernel(const void* __restrict__ a,
                                                        const void* __restrict__ t_inv,
                                                        const float* __restrict__ M,
                                                        void* __restrict__ out, int B, int n,
                                                        int d, int D, int GW) {
  extern __shared__ float smem[];
  float* sa = smem;                              // [TB][256] activations of <= 2 blocks
  float* su = sa + TB * 2 * kTB;                 // [TB][kMaxRows] transformed
  float* sM = su + TB * kMaxRows;                // [d][D]

  const int G = n / d;
  const int64_t K = (int64_t)G * D;
  const int g0 = blockIdx.x * GW;
  const int gcount = min(GW, G - g0);
  const int c0 = g0 * d;
  const int cw = gcount * d;                     // channels of u owned here (<= kMaxRows)
  const int blk0 = c0 / kTB;
  const int nblk = (c0 + cw - 1) / kTB - blk0 + 1;   // 1 or 2
  const int b0 = blockIdx.y * TB;
  const int bc = min(TB, B - b0);
  const int tid = threadIdx.x;

  // T^-1 rows c0 .. c0 + cw - 1: lane j of a row loads elements 8j .. 8j + 7
  const int j = tid & 15;
  float tv[kPasses][8];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = p * 16 + (tid >> 4);
    if (row < cw) {
      load8_as_float<T_DT>(t_inv, (int64_t)(c0 + row) * kTB + 8 * j, tv[p]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tv[p][e] = 0.f;
    }
  }
  // Activations of the (one or two) blocks for bc tokens, 8 elements per
  // 16-byte load, and M: every load is issued before the first LDS store.
  const int aw = nblk * kTB;
  const int avec = bc * (aw / 8);
  constexpr int kAPer = (TB * 2 * kTB / 8 + kThreads - 1) / kThreads;
  float av[kAPer][8];
#pragma unroll
  for (int k = 0; k < kAPer; ++k) {
    const int i = tid + k * kThreads;
    if (i < avec) {
      const int b = i / (aw / 8);
      const int col = (i - b * (aw / 8)) * 8;
      load8_as_float<A_DT>(a, (int64_t)(b0 + b) * n + blk0 * kTB + col, av[k]);
    }
  }
  for (int i0 = 0; i0 < d * D; i0 += 8 * kThreads) {
    float mv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kThreads + tid;
      mv[u] = i < d * D ? M[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kThreads + tid;
      if (i < d * D) sM[i] = mv[u];
    }
  }
#pragma unroll
  for (int k = 0; k < kAPer; ++k) {
    const int i = tid + k * kThreads;
    if (i < avec) {
      const int b = i / (aw / 8);
      const int col = (i - b * (aw / 8)) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) sa[b * 2 * kTB + col + e] = av[k][e];
    }
  }
  __syncthreads();

#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    if (p * 16 >= cw) break;                     // workgroup-uniform
    const int row = p * 16 + (tid >> 4);
    const int q = (c0 + row) / kTB - blk0;       // block of this row, relative
    float acc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const float* ab = sa + b * 2 * kTB + q * kTB + 8 * j;
      float s0 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s0 = fmaf(tv[p][e], ab[e], s0);
      acc[b] = s0;
    }
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      float v = acc[b];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      if (j == 0 && row < cw && b < bc) su[b * kMaxRows + row] = v;
    }
  }
  __syncthreads();

  // a_hat for the groups of this workgroup
  const int ow = gcount * D;
  for (int i = tid; i < bc * ow; i += kThreads) {
    const int b = i / ow;
    const int rem = i - b * ow;
    const int g = rem / D;
    const int jj = rem - g * D;
    const float* ub = su + b * kMaxRows + g * d;
    float acc = 0.f;
    for (int rr = 0; rr < d; ++rr) acc = fmaf(sM[rr * D + jj], ub[rr], acc);
    store_from_float<O_DT>(out, (int64_t)(b0 + b) * K + (int64_t)g0 * D + rem, acc);
  }
}

template <int A_DT, int T_DT, int O_DT, int TB>
hipError_t launch_lift_tb(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M,
                          int d, int D, void* out, hipStream_t st) {
  const int G = static_cast<int>(n / d);
  const int GW = 32 / d > 0 ? 32 / d : 1;        // whole groups: <= 32 channels, or one group
  const int gx = (G + GW - 1) / GW;
  const int gy = static_cast<int>((B + TB - 1) / TB);
  const size_t lds = sizeof(float) * (TB * 2 * kTB + TB * kMaxRows + d * D);
  hipLaunchKernelGGL((lift_kernel<A_DT, T_DT, O_DT, TB>), dim3(gx, gy), dim3(kThreads), lds, st,
                     a, t_inv, M, out, static_cast<int>(B), static_cast<int>(n), d, D, GW);
  return hipGetLastError();
}

template <int A_DT, int T_DT, int O_DT>
hipError_t launch_lift_t(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M,
                         int d, int D, void* out, hipStream_t st) {
  if (B <= 1) return launch_lift_tb<A_DT, T_DT, O_DT, 1>(a, B, n, t_inv, M, d, D, out, st);
  if (B <= 2) return launch_lift_tb<A_DT, T_DT, O_DT, 2>(a, B, n, t_inv, M, d, D, out, st);
  if (B <= 4) return launch_lift_tb<A_DT, T_DT, O_DT, 4>(a, B, n, t_inv, M, d, D, out, st);
  if (B <= 8) return launch_lift_tb<A_DT, T_DT, O_DT, 8>(a, B, n, t_inv, M, d, D, out, st);
  return launch_lift_tb<A_DT, T_DT, O_DT, 16>(a, B, n, t_inv, M, d, D, out, st);
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
  if (lift_mfma_applies(a_dt, t_dt, B, n, d, D))
    return launch_lift_mfma(a, a_dt, B, n, t_inv, M, d, D, out, out_dt, st);
  switch (a_dt) {
    case LQ_F32: return dispatch_t<LQ_F32>(a, B, n, t_inv, t_dt, M, d, D, out, out_dt, st);
    case LQ_F16: return dispatch_t<LQ_F16>(a, B, n, t_inv, t_dt, M, d, D, out, out_dt, st);
    default: return dispatch_t<LQ_BF16>(a, B, n, t_inv, t_dt, M, d, D, out, out_dt, st);
  }
}

}  // namespace lq
