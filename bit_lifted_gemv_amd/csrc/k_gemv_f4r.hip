// One-launch product of 1-bit weights with float lifted activations for one
// to five tokens:
//   out[b][i] = s[i] * sum_k sigma_ik * a_hat[b][k],  sigma = 2*bit - 1
// (LiftQuant notes, 关键设计 4: after the activation transform the layer is a
// product of 1-bit weights with floats, scaled per row by s).
//
// Matrix-core operands as in f4_parts.h: sign bits as float4 (A) masked in
// place, each activation as three float8 parts in B columns 3 b + p with a
// power-of-two hardware scale per 1024-position slice; a slice contributes
// 2 R - sum a, with R the sum of the activations whose bit is set.
//
// Work split.  Each workgroup owns a contiguous run of 16-row tiles and all
// of K, so no partial sum leaves it and the call is one launch.  It applies
// when the activation parts of every slice fit in LDS at once (3 bytes per
// position and token).  The start loads the activations first and waits for
// them before any weight load is issued (behind a flood of weight misses they
// would arrive late), then issues the weight ring, and each wave converts
// slices w, w + W, ... of the W waves (16 positions per lane, its own max
// over the slice);
// one barrier.  The workgroup's granules (row tile, slice) are taken in
// slice-major order and cut into contiguous runs, one per wave, so a
// wave's consecutive granules mostly share a slice and its B operands stay
// in registers until the slice changes.  Each granule leaves its 16 rows'
// sums for its slice in LDS; at the end the workgroup adds each row's slices
// in order, scales by s and writes the row.  Deterministic.
#include <type_traits>

#include "f4_parts.h"
#include "lq_internal.h"

namespace lq {
namespace {

// f(0), f(1), ..., f(N - 1) with compile-time arguments (register arrays
// indexed by them stay in registers).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

using f4::f32x4;
using f4::i32x8;
using f4::part_bytes;

constexpr int kSliceBits = 1024;
constexpr int kSliceBytes = kSliceBits / 8;     // 128 bytes of a row per slice
constexpr int kSteps = kSliceBits / 128;        // 8 MFMA steps per slice
constexpr uint32_t kNoLoad = 0x80000000u;       // past every buffer range: loads give 0
// Waves per workgroup: 16 at one token (twice the waves to load and convert
// the activations at the start: 70B up shape 19.3 -> 17.8 us), 8 for more
// tokens (16 measured slower there).  The weight ring holds 32 granules per
// workgroup either way (64 KB in flight per compute unit).
constexpr int waves_for(int nb) { return nb == 1 ? 16 : 8; }
constexpr int kRingPerWG = 32;
constexpr int kRows = 16;
constexpr int kXFloats = 80;                    // activation registers per lane
constexpr size_t kLdsBytes = 160 * 1024;

// A wave converts whole slices (16 positions per lane): at most this many.
constexpr int xs_per_wave(int nb) { return kXFloats / (16 * nb) > 0 ? kXFloats / (16 * nb) : 1; }

struct PlanR {
  int G;        // workgroups
  int RT;       // 16-row tiles per workgroup (the last may have fewer)
  int S;        // slices of K
  size_t lds;   // dynamic LDS bytes
};

// Dynamic LDS: parts [S][part_bytes] | column scale exponents [S][NB] int |
// activation sums [S][NB] float | partial sums [RT][S][NB][16] float.
template <int NB, int kWaves = waves_for(NB), int kThreads = 64 * kWaves,
          int kDepth = kRingPerWG / kWaves>
__global__ void __launch_bounds__(kThreads, 1) gemv_f4r_kernel(
    const uint32_t* __restrict__ w, int64_t m, int64_t K, int64_t ldw,
    const float* __restrict__ s, const float* __restrict__ ah, float* __restrict__ out,
    int NG, int RT, int S, uint32_t w_bytes, uint32_t a_bytes) {
  constexpr int NCOL = 3 * NB;
  constexpr int PB = part_bytes(NB);
  constexpr int XS = xs_per_wave(NB);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* parts = lds;
  int* esc = reinterpret_cast<int*>(lds + static_cast<size_t>(S) * PB);
  float* asum = reinterpret_cast<float*>(esc + S * NB);
  float* psum = reinterpret_cast<float*>(lds + static_cast<size_t>(S) * PB +
                                         ((static_cast<size_t>(S) * NB * 8 + 15) & ~size_t{15}));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt0 = blockIdx.x * RT;
  const int RTb = min(RT, NG - rt0);           // row tiles of this workgroup (>= 1)
  const int r = lane & 15;                      // A: row; B and D: column
  const int G = lane >> 4;
  const int col = r;
  const bool bcol = col < NCOL;
  const int cb = bcol ? col / 3 : 0;
  const int cp = bcol ? col - 3 * (col / 3) : 0;

  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w), (short)0, static_cast<int>(w_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ah), (short)0, static_cast<int>(a_bytes), 0x00020000);
  const uint32_t row_bytes = static_cast<uint32_t>(ldw * 4);
  const uint32_t lane_off0 = static_cast<uint32_t>(r) * row_bytes + 16 * G;
  const uint32_t lane_off1 = lane_off0 + 64;
  const uint32_t wg_off = static_cast<uint32_t>(rt0) * kRows * row_bytes;

  // 1. Activations of the slices this wave converts (w, w + kWaves, ...), lane l
  // holding positions 16 l .. 16 l + 15 of each.
  f32x4 xv[XS][NB][4];
#pragma unroll
  for (int i = 0; i < XS; ++i) {
    const int t = wave + kWaves * i;
    if (t < S) {
      const int64_t k0 = (int64_t)t * kSliceBits + 16 * lane;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t k = k0 + 4 * c;         // K % 4 == 0: all four or none
          const uint32_t off = k < K ? static_cast<uint32_t>(((int64_t)b * K + k) * 4) : kNoLoad;
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(ares, off, 0, 0);
          __builtin_memcpy(&xv[i][b][c], &v, 16);
        }
      }
    }
  }

  // 2. The largest |x| and the sum of each of those slices, over the wave.
  // Needs the activations, so they arrive before any weight load is issued.
  uint32_t mbs[XS][NB];
  float sums[XS][NB];
#pragma unroll
  for (int i = 0; i < XS; ++i) {
    if (wave + kWaves * i < S) f4::slice_stats<NB>(xv[i], mbs[i], sums[i]);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. The weight ring: the wave's run of granules [qa, qb) of the
  // workgroup's T = RTb * S, in slice-major order (granule q is slice
  // q / RTb, row tile q % RTb).
  const int T = RTb * S;
  const int qa = (wave * T) / kWaves, qb = ((wave + 1) * T) / kWaves;
  int qn = qa;                                  // next granule to issue
  uint4 wb[kDepth][2];
  int gq[kDepth];
  auto issue = [&](int e) __attribute__((always_inline)) {
    const int q = qn < qb ? qn : -1;
    uint32_t so = kNoLoad;
    if (q >= 0) {
      ++qn;
      const int sl = q / RTb;
      const int rtl = q - sl * RTb;
      so = wg_off + static_cast<uint32_t>(rtl) * kRows * row_bytes +
           static_cast<uint32_t>(sl) * kSliceBytes;
    }
    const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(wres, lane_off0, so, 0);
    const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(wres, lane_off1, so, 0);
    __builtin_memcpy(&wb[e][0], &v0, 16);
    __builtin_memcpy(&wb[e][1], &v1, 16);
    gq[e] = q;
  };
  static_for<kDepth>([&](auto ec) __attribute__((always_inline)) { issue(decltype(ec)::value); });

  // 4. Parts of the slices into LDS (f4::slice_parts).
#pragma unroll
  for (int i = 0; i < XS; ++i) {
    const int t = wave + kWaves * i;
    if (t < S) {
      int e[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        e[b] = f4::slice_exponent(mbs[i][b]);
        if (lane == 0) {
          esc[t * NB + b] = e[b];
          asum[t * NB + b] = sums[i][b];
        }
      }
      f4::slice_parts<NB>(xv[i], e, parts + t * PB, lane);
    }
  }
  __syncthreads();

  // 5. The granules.  Rounds of kDepth ring slots; each slot is refilled as
  // soon as its weights are in registers.
  const uint8_t* bsrc_col = parts + (static_cast<size_t>(bcol ? col : 0) * 4 + G) * 32;
  int cur = -1;                                 // slice whose B operands are in bv
  int scl = 127;
  float asl = 0.f;                              // sum of the slice's activations (token cb)
  i32x8 bv[kSteps];
  while (gq[0] >= 0) {
    static_for<kDepth>([&](auto ec) __attribute__((always_inline)) {
      constexpr int e = decltype(ec)::value;
      const int q = gq[e];
      if (q < 0) return;
      const int sl = q / RTb;
      const int rtl = q - sl * RTb;
      if (sl != cur) {
        cur = sl;
        const uint8_t* bs = bsrc_col + static_cast<size_t>(sl) * PB;
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
          bv[u] = i32x8{};
          if (bcol) {
            const uint4 y0 = *reinterpret_cast<const uint4*>(bs + u * NCOL * 128);
            const uint4 y1 = *reinterpret_cast<const uint4*>(bs + u * NCOL * 128 + 16);
            __builtin_memcpy(&bv[u], &y0, 16);
            __builtin_memcpy(reinterpret_cast<char*>(&bv[u]) + 16, &y1, 16);
          }
        }
        scl = 127 - esc[sl * NB + cb] - 4 * cp;
        asl = asum[sl * NB + cb];
      }
      const uint32_t wd[8] = {wb[e][0].x, wb[e][0].y, wb[e][0].z, wb[e][0].w,
                              wb[e][1].x, wb[e][1].y, wb[e][1].z, wb[e][1].w};
      issue(e);
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll
      for (int u = 0; u < kSteps; u += 2) {
        c0 = f4::mfma(f4::expand(wd[u]), bv[u], c0, scl);
        c1 = f4::mfma(f4::expand(wd[u + 1]), bv[u + 1], c1, scl);
      }
      const f32x4 c = c0 + c1;
      float4 v;
      v.x = f4::slice_sum(c[0], asl);
      v.y = f4::slice_sum(c[1], asl);
      v.z = f4::slice_sum(c[2], asl);
      v.w = f4::slice_sum(c[3], asl);
      if (bcol && cp == 0)
        *reinterpret_cast<float4*>(psum + ((static_cast<size_t>(rtl) * S + sl) * NB + cb) * kRows +
                                   4 * G) = v;
    });
  }
  __syncthreads();                              // every granule's sums are in LDS

  // 6. out[b][row] = s[row] * (sum over the slices, in order)
  for (int idx = tid; idx < RTb * kRows * NB; idx += kThreads) {
    const int b = idx / (RTb * kRows);
    const int rr = idx - b * RTb * kRows;       // row within the workgroup
    const int rtl = rr / kRows, ri = rr - rtl * kRows;
    const int64_t row = static_cast<int64_t>(rt0) * kRows + rr;
    const float* p = psum + (static_cast<size_t>(rtl) * S * NB + b) * kRows + ri;
    float acc = 0.f;
    for (int sl = 0; sl < S; ++sl) acc += p[static_cast<size_t>(sl) * NB * kRows];
    if (row < m) out[b * m + row] = s[row] * acc;
  }
}

PlanR plan_r(int64_t m, int64_t K, int64_t B) {
  PlanR p{};
  const int64_t NG = (m + kRows - 1) / kRows;
  p.S = static_cast<int>((K + kSliceBits - 1) / kSliceBits);
  const int64_t cus = num_cus();
  p.RT = static_cast<int>((NG + cus - 1) / cus);
  p.G = static_cast<int>((NG + p.RT - 1) / p.RT);
  p.lds = static_cast<size_t>(p.S) * part_bytes(static_cast<int>(B)) +
          ((static_cast<size_t>(p.S) * B * 8 + 15) & ~size_t{15}) +
          static_cast<size_t>(p.RT) * p.S * B * kRows * 4;
  return p;
}

template <int NB>
hipError_t launch_r(const PlanR& p, const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                    const float* s, const float* a_lift, float* out, hipStream_t st) {
  const int NG = static_cast<int>((m + kRows - 1) / kRows);
  const uint32_t w_bytes = static_cast<uint32_t>(m * ldw * 4);
  const uint32_t a_bytes = static_cast<uint32_t>(NB * K * 4);
  const void* fn = reinterpret_cast<const void*>(gemv_f4r_kernel<NB>);
  if (p.lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(p.lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gemv_f4r_kernel<NB>, dim3(p.G), dim3(64 * waves_for(NB)), p.lds, st, w, m, K,
                     ldw, s,
                     a_lift, out, NG, p.RT, p.S, w_bytes, a_bytes);
  return hipGetLastError();
}

}  // namespace

// The one-launch kernel applies when each wave converts at most as many
// slices as its registers hold and the parts of all slices, their scales
// and every (row tile, slice) sum fit in LDS together.
bool gemv_f4r_applies(int64_t m, int64_t K, int64_t B) {
  if (B < 1 || B > 5 || m < 1 || K < 1) return false;
  const PlanR p = plan_r(m, K, B);
  // Every workgroup loads and converts every slice: at one token the one
  // launch (16 waves) is taken up to 40 slices (160 KB of activations per
  // workgroup; 4096 x 28672, 28 slices: 10.2 us against 10.8 us for the
  // slice-major kernel and its reduction; with 8 waves it lost past 20).
  if (B == 1 && p.S > 40) return false;
  return p.S <= waves_for(static_cast<int>(B)) * xs_per_wave(static_cast<int>(B)) &&
         p.lds <= kLdsBytes;
}

hipError_t launch_gemv_f4r(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                           const float* a_lift, int64_t B, float* out, hipStream_t st) {
  const PlanR p = plan_r(m, K, B);
  switch (B) {
    case 1: return launch_r<1>(p, w, m, K, ldw, s, a_lift, out, st);
    case 2: return launch_r<2>(p, w, m, K, ldw, s, a_lift, out, st);
    case 3: return launch_r<3>(p, w, m, K, ldw, s, a_lift, out, st);
    case 4: return launch_r<4>(p, w, m, K, ldw, s, a_lift, out, st);
    default: return launch_r<5>(p, w, m, K, ldw, s, a_lift, out, st);
  }
}

}  // namespace lq
