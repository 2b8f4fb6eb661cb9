// Product of 1-bit weights with float lifted activations for a few tokens on
// the matrix cores:
//   out[b][i] = s[i] * sum_k sigma_ik * a_hat[b][k],  sigma = 2*bit - 1
// (LiftQuant notes, 关键设计 4: after the activation transform the layer is a
// product of 1-bit weights with floats, scaled per row by s).
//
// Matrix-core operands as in f4_parts.h: sign bits as float4 (A) masked in
// place, each activation as three float8 parts in B columns 3 b + p with a
// power-of-two hardware scale per 1024-position slice; a slice contributes
// 2 R - sum a, with R the sum of the activations whose bit is set.
//
// Work split (as the one-token table kernel): granule = 16 rows x one slice;
// granules ordered (slice, row) and cut into one range per workgroup (one
// workgroup of 8 waves per CU); each wave streams a contiguous run of
// granules per slice with a ring of DEPTH granules of loads in flight.  At
// the start of a slice the workgroup turns the slice's activations into the
// float8 parts (in LDS; one wave converts a slice, 16 positions per lane),
// and each wave keeps the B operands of the slice's 8 steps in registers
// while it streams the slice's granules.  Each granule
// leaves the 16 rows' sums of one slice per token in the workspace; a second
// kernel adds each row's S partial sums in slice order, scales by s and
// writes the row.  Deterministic.
#include <type_traits>

#include "f4_parts.h"
#include "lq_internal.h"

namespace lq {
namespace {

using f4::f32x4;
using f4::i32x8;

constexpr int kSliceBits = 1024;
constexpr int kSliceBytes = kSliceBits / 8;     // 128 bytes of a row per slice
constexpr int kSteps = kSliceBits / 128;        // 8 MFMA steps per slice
constexpr uint32_t kNoLoad = 0x80000000u;       // past every buffer range: loads give 0
constexpr int kWaves = 8;                       // two waves per SIMD: 256 registers each
constexpr int kDepth = 4;                       // granules of weights in flight per wave
constexpr int kEarly = 2;                       // of them issued before the parts exist
constexpr int kThreads = 64 * kWaves;
constexpr int kGranuleRows = 16;
constexpr int kMaxGroups = 256;
constexpr double kStraddleCost = 0.1;           // a second slice: parts and padded runs

struct Sched {
  int64_t NG;   // 16-row granules per slice
  int64_t T;    // granules in all: S * NG
  int S;        // slices
  int G;        // workgroups
  int64_t start[kMaxGroups + 1];
};

// NB: tokens (1..5); DEPTH: granules of weights in flight per wave.
template <int NB, int DEPTH, bool SPLIT>
__global__ void __launch_bounds__(kThreads, 1) gemv_f4_kernel(
    const uint32_t* __restrict__ w, int64_t m, int64_t K, int64_t ldw,
    const float* __restrict__ s, const float* __restrict__ ah, float* __restrict__ out,
    float* __restrict__ partials, Sched sc, uint32_t w_bytes, uint32_t a_bytes) {
  constexpr int NCOL = 3 * NB;
  constexpr int kPartBytes = f4::part_bytes(NB);               // per slice
  __shared__ __attribute__((aligned(16))) uint8_t parts[2][kPartBytes];
  __shared__ int esc[2][NB];
  __shared__ float asum[2][NB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t_begin = sc.start[blockIdx.x];
  const int64_t t_end = sc.start[blockIdx.x + 1];
  if (t_begin >= t_end) return;
  const int sl_first = static_cast<int>(t_begin / sc.NG);
  const int sl_last = static_cast<int>((t_end - 1) / sc.NG);

  const int r = lane & 15;           // A: row; B and D: column
  const int G = lane >> 4;           // lane group
  const int col = r;
  const int cb = col < NCOL ? col / 3 : 0;                 // token of the column
  const int cp = col < NCOL ? col - 3 * (col / 3) : 0;     // part of the column
  const int col_c = col < NCOL ? col : 0;                  // column read (unused ones: any)

  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w), (short)0, static_cast<int>(w_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ah), (short)0, static_cast<int>(a_bytes), 0x00020000);
  const uint32_t row_bytes = static_cast<uint32_t>(ldw * 4);
  const uint32_t granule_bytes = kGranuleRows * row_bytes;
  const uint32_t lane_off0 = static_cast<uint32_t>(r) * row_bytes + 16 * G;
  const uint32_t lane_off1 = lane_off0 + 64;

  auto lo_of = [&](int sl) -> int {
    const int64_t v = t_begin - (int64_t)sl * sc.NG;
    return v > 0 ? static_cast<int>(v) : 0;
  };
  auto hi_of = [&](int sl) -> int {
    const int64_t v = t_end - (int64_t)sl * sc.NG;
    return static_cast<int>(v < sc.NG ? v : sc.NG);
  };
  auto run_a = [&](int sl) -> int {
    const int lo = lo_of(sl);
    return lo + (wave * (hi_of(sl) - lo)) / kWaves;
  };
  auto run_b = [&](int sl) -> int {
    const int lo = lo_of(sl);
    return lo + ((wave + 1) * (hi_of(sl) - lo)) / kWaves;
  };

  // Load cursor (scalar): each slice's run is processed in rounds of DEPTH
  // ring slots, the last round padded with empty slots.
  int ld_sl = sl_first - 1, ld_k = 0, ld_n = 0, ld_slots = 0;
  uint32_t ld_off = 0;
  auto ld_next_slice = [&]() {
    do {
      ++ld_sl;
      ld_k = 0;
      if (ld_sl <= sl_last) {
        const int a = run_a(ld_sl);
        ld_n = run_b(ld_sl) - a;
        ld_slots = (ld_n + DEPTH - 1) / DEPTH * DEPTH;
        ld_off = static_cast<uint32_t>(a) * granule_bytes +
                 static_cast<uint32_t>(ld_sl) * kSliceBytes;
      } else {
        ld_n = 0;
        ld_slots = 1 << 30;
      }
    } while (ld_slots == 0);
  };
  uint4 wb[DEPTH][2];
  auto issue = [&](uint4 (&dst)[2]) {
    const uint32_t so = ld_k < ld_n ? ld_off : kNoLoad;
    const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(wres, lane_off0, so, 0);
    const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(wres, lane_off1, so, 0);
    ld_off += granule_bytes;
    ++ld_k;
    __builtin_memcpy(&dst[0], &v0, 16);
    __builtin_memcpy(&dst[1], &v1, 16);
  };

  // Activation parts of slices sp and sp + 1 (the second if the range
  // reaches it) into LDS slots 0 and 1, wave t converting slice sp + t.  The
  // activation loads are issued before any weight load of the workgroup (the
  // first barrier); with `first` each wave then issues two granules of
  // weights, which stream in while the parts are formed, and the rest of its
  // ring after.
  auto prepare = [&](int sp, bool first) __attribute__((always_inline)) {
    const int nt = sp + 1 <= sl_last ? 2 : 1;
    const bool conv = wave < nt;                // uniform
    f32x4 xv[NB][4];
    if (conv) {
      const int64_t k0 = (int64_t)(sp + wave) * kSliceBits + 16 * lane;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t k = k0 + 4 * c;         // K % 4 == 0: all four or none
          const uint32_t off = k < K ? static_cast<uint32_t>(((int64_t)b * K + k) * 4) : kNoLoad;
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(ares, off, 0, 0);
          __builtin_memcpy(&xv[b][c], &v, 16);
        }
      }
    }
    __syncthreads();                          // activations requested before any weight;
                                              // nobody reads the old parts any more
    if (first) {
      ld_next_slice();
#pragma unroll
      for (int e = 0; e < kEarly; ++e) issue(wb[e]);
    }
    if (conv) {
      uint32_t mb[NB];
      float sum[NB];
      f4::slice_stats<NB>(xv, mb, sum);
      int e[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        e[b] = f4::slice_exponent(mb[b]);
        if (lane == 0) {
          esc[wave][b] = e[b];
          asum[wave][b] = sum[b];
        }
      }
      f4::slice_parts<NB>(xv, e, parts[wave], lane);
    }
    __syncthreads();
    if (first) {
#pragma unroll
      for (int e = kEarly; e < DEPTH; ++e) issue(wb[e]);
    }
  };
  prepare(sl_first, true);

  int rnd = 0;
  auto process_run = [&](auto tsel, int sl) {
    constexpr int TI = decltype(tsel)::value;
    const int a = run_a(sl);
    const int n = run_b(sl) - a;
    // this slice's B operands and scales
    i32x8 bv[kSteps];
    const uint8_t* src = parts[TI] + (col_c * 4 + G) * 32;
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const uint4 y0 = *reinterpret_cast<const uint4*>(src + u * NCOL * 128);
      const uint4 y1 = *reinterpret_cast<const uint4*>(src + u * NCOL * 128 + 16);
      __builtin_memcpy(&bv[u], &y0, 16);
      __builtin_memcpy(reinterpret_cast<char*>(&bv[u]) + 16, &y1, 16);
    }
    const int scl = 127 - esc[TI][cb] - 4 * cp;
    const float asl = asum[TI][cb];
    const bool writer = col < NCOL && cp == 0;
    float* pout = SPLIT ? partials + (((int64_t)a * sc.S + sl) * NB + cb) * kGranuleRows + 4 * G
                        : out + (int64_t)cb * m + (int64_t)kGranuleRows * a + 4 * G;
    const float* ps = s + (int64_t)kGranuleRows * a + 4 * G;
    const int64_t pstep = SPLIT ? (int64_t)sc.S * NB * kGranuleRows : kGranuleRows;
    for (int k0 = 0; k0 < n; k0 += DEPTH, ++rnd) {
      if (ld_k >= ld_slots) ld_next_slice();
#pragma unroll
      for (int e = 0; e < DEPTH; ++e) {
        if (k0 + e < n) {
          const uint32_t wd[8] = {wb[e][0].x, wb[e][0].y, wb[e][0].z, wb[e][0].w,
                                  wb[e][1].x, wb[e][1].y, wb[e][1].z, wb[e][1].w};
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
          if constexpr (SPLIT) {
            if (writer) *reinterpret_cast<float4*>(pout) = v;
          } else {
            const int64_t row = (int64_t)kGranuleRows * (a + k0 + e) + 4 * G;
            if (writer) {
              if (row + 0 < m) pout[0] = ps[0] * v.x;
              if (row + 1 < m) pout[1] = ps[1] * v.y;
              if (row + 2 < m) pout[2] = ps[2] * v.z;
              if (row + 3 < m) pout[3] = ps[3] * v.w;
            }
            ps += pstep;
          }
          pout += pstep;
        }
        issue(wb[e]);
      }
    }
  };

  for (int sl = sl_first; sl <= sl_last; ++sl) {
    const int rel = sl - sl_first;
    if (rel >= 2 && (rel & 1) == 0) prepare(sl, false);
    if ((rel & 1) == 0)
      process_run(std::integral_constant<int, 0>{}, sl);
    else
      process_run(std::integral_constant<int, 1>{}, sl);
  }
}

// out[b][i] = s[i] * (sum over slices q of partials[i / 16][q][b][i % 16]):
// a wave per (16-row tile, token); lane (row l % 16, part l / 16) adds slices
// part, part + 4, ... in order (every load four whole 64-byte runs of the
// tile, all in flight), then the four parts are added in a fixed order.
// kChunk: slices of a lane in flight at once (the launch picks the smallest
// power of two that covers the lane's slices, at most 32).
template <int kChunk>
__global__ void __launch_bounds__(256) gemv_f4_reduce_kernel(const float* __restrict__ partials,
                                                             const float* __restrict__ s,
                                                             float* __restrict__ out, int64_t m,
                                                             int S, int NB, int64_t units) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;   // g * NB + b
  if (unit >= units) return;                    // whole waves
  const int64_t g = unit / NB;
  const int b = static_cast<int>(unit - g * NB);
  const int r = lane & 15, part = lane >> 4;
  // every load of a chunk is issued before the first add: slices past S read
  // the lane's last one again (an address known to be valid, no branch) and
  // are not added
  const float* p = partials + ((g * S + part) * NB + b) * kGranuleRows + r;
  const int64_t qstep = 4 * (int64_t)NB * kGranuleRows;
  const int qlast = part < S ? (S - 1 - part) / 4 : 0;   // this lane's last slice index
  float sum = 0.f;
  for (int i0 = 0; part + 4 * i0 < S; i0 += kChunk) {
    float v[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) v[i] = p[min(i0 + i, qlast) * qstep];
    // slices in increasing order, as many as this lane has
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      if (i0 + i <= qlast) sum += v[i];
  }
  sum += __shfl_xor(sum, 16);                   // parts 0 + 1, 2 + 3
  sum += __shfl_xor(sum, 32);                   // (0 + 1) + (2 + 3)
  const int64_t row = g * kGranuleRows + r;
  if (part == 0 && row < m) out[b * m + row] = s[row] * sum;
}

void reduce_slices(const float* partials, const float* s, float* out, int64_t m, int S, int NB,
                   hipStream_t st) {
  const int64_t units = (m + kGranuleRows - 1) / kGranuleRows * NB;
  const dim3 grid(static_cast<unsigned>((units + 3) / 4));
  const int per_lane = (S + 3) / 4;
  if (per_lane <= 4)
    hipLaunchKernelGGL(gemv_f4_reduce_kernel<4>, grid, dim3(256), 0, st, partials, s, out, m, S,
                       NB, units);
  else if (per_lane <= 8)
    hipLaunchKernelGGL(gemv_f4_reduce_kernel<8>, grid, dim3(256), 0, st, partials, s, out, m, S,
                       NB, units);
  else if (per_lane <= 16)
    hipLaunchKernelGGL(gemv_f4_reduce_kernel<16>, grid, dim3(256), 0, st, partials, s, out, m, S,
                       NB, units);
  else
    hipLaunchKernelGGL(gemv_f4_reduce_kernel<32>, grid, dim3(256), 0, st, partials, s, out, m, S,
                       NB, units);
}

Sched make_sched(int64_t m, int64_t K) {
  Sched sc{};
  sc.S = static_cast<int>((K + kSliceBits - 1) / kSliceBits);
  sc.NG = (m + kGranuleRows - 1) / kGranuleRows;
  sc.T = sc.NG * sc.S;
  const int64_t gmax = (sc.T + kWaves - 1) / kWaves;
  int cus = num_cus();
  if (cus > kMaxGroups) cus = kMaxGroups;
  sc.G = static_cast<int>(gmax < cus ? gmax : cus);
  const double share = (double)sc.T / sc.G;
  const double c = share < (double)sc.NG ? kStraddleCost * share : 0.0;
  const double span = (double)sc.NG + c;
  const double V = (double)sc.T + (sc.S - 1) * c;
  for (int w = 0; w < sc.G; ++w) {
    const double v = V * w / sc.G;
    int64_t sl = (int64_t)(v / span);
    if (sl >= sc.S) sl = sc.S - 1;
    double off = v - sl * span;
    if (off > (double)sc.NG) off = (double)sc.NG;
    int64_t t = sl * sc.NG + (int64_t)(off + 1e-9);
    if (t > sc.T) t = sc.T;
    if (w > 0 && t < sc.start[w - 1]) t = sc.start[w - 1];
    sc.start[w] = t;
  }
  sc.start[sc.G] = sc.T;
  return sc;
}

template <int NB>
hipError_t launch_nb(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                     const float* a_lift, float* out, void* ws, hipStream_t st) {
  constexpr int DEPTH = kDepth;
  const Sched sc = make_sched(m, K);
  const uint32_t w_bytes = static_cast<uint32_t>(m * ldw * 4);
  const uint32_t a_bytes = static_cast<uint32_t>(NB * K * 4);
  if (sc.S == 1) {
    hipLaunchKernelGGL((gemv_f4_kernel<NB, DEPTH, false>), dim3(sc.G), dim3(kThreads), 0, st, w,
                       m, K, ldw, s, a_lift, out, nullptr, sc, w_bytes, a_bytes);
    return hipGetLastError();
  }
  float* partials = static_cast<float*>(ws);
  hipLaunchKernelGGL((gemv_f4_kernel<NB, DEPTH, true>), dim3(sc.G), dim3(kThreads), 0, st, w, m,
                     K, ldw, s, a_lift, out, partials, sc, w_bytes, a_bytes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  reduce_slices(partials, s, out, m, sc.S, NB, st);
  return hipGetLastError();
}

}  // namespace

size_t gemv_f4_workspace_bytes(int64_t m, int64_t K, int64_t B) {
  const Sched sc = make_sched(m, K);
  if (sc.S == 1) return 0;
  return sizeof(float) * kGranuleRows * (size_t)sc.NG * sc.S * B;
}

hipError_t launch_gemv_f4(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                          const float* a_lift, int64_t B, float* out, void* ws, hipStream_t st) {
  switch (B) {
    case 1: return launch_nb<1>(w, m, K, ldw, s, a_lift, out, ws, st);
    case 2: return launch_nb<2>(w, m, K, ldw, s, a_lift, out, ws, st);
    case 3: return launch_nb<3>(w, m, K, ldw, s, a_lift, out, ws, st);
    case 4: return launch_nb<4>(w, m, K, ldw, s, a_lift, out, ws, st);
    default: return launch_nb<5>(w, m, K, ldw, s, a_lift, out, ws, st);
  }
}

}  // namespace lq
