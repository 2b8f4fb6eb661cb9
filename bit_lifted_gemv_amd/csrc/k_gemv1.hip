// One-token product of 1-bit weights with float lifted activations:
//   out[i] = s[i] * sum_k sigma_ik * a_hat[k],  sigma = 2*bit - 1
// (LiftQuant notes, 关键设计 4: after the activation transform the layer is a
// product of 1-bit weights with floats, scaled per row by s).
//
// The weights stream from HBM once; each weight byte costs one table read and
// one add, against tables of signed activation sums.  A table serves one
// 1024-bit slice of the lifted dimension,
//   E_p[v] = sum_{t<8} (2*bit_t(v) - 1) * a_hat[1024 sl + 8p + t]   (p < 128, v < 256),
// and costs about as much to build as a few thousand rows of lookups, so it
// has to serve many rows: the work is ordered slice-major.
//
// Tables are float16 (64 KB per slice), so that the two slices a workgroup's
// range can straddle both stay in LDS and no wave ever waits for another.
// Each table is built from the slice's activations scaled by a power of two
// that puts the largest possible entry (8 max|a|) just below 2^14, and the
// row sums are scaled back by the inverse power: the scaling is exact, and
// each entry carries one float16 rounding (relative 2^-11) whatever the range
// of the activations.  Lookups add the float16 entries in float32.
//
// Work split.  Granule = 16 rows x one slice (2 KB of weights).  The granules
// are ordered (slice, row) and cut into one equal range per workgroup (one
// workgroup per CU), so a workgroup covers a long run of rows of one or two
// slices.  In each slice the 16 waves split the workgroup's granules into 16
// contiguous runs; each wave streams its runs on its own with a ring of DEPTH
// granules of loads in flight (lane (r, c) loads 16 bytes of rows r and r + 8
// of the granule, 8 lanes per row).
//
// Reduction over slices.  Each granule leaves its 16 row sums of one slice in
// the workspace (plain stores); a second kernel adds each row's S partial
// sums in slice order (4 lanes per row, then a fixed tree), scales by s and
// writes the row, so the result does not depend on timing.  Split-K with an
// in-kernel last-arriver reduction would put the slowest wave's reductions on
// the critical path; the kernel boundary costs less than that.
#include <type_traits>

#include "lq_internal.h"

namespace lq {
namespace {

constexpr int kSliceBits = 1024;                // lifted positions per table
constexpr int kSliceBytes = kSliceBits / 8;     // 128
constexpr uint32_t kNoLoad = 0x80000000u;       // outside every buffer resource: loads give 0

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return v + __int_as_float(o);
}

// Sum over the 8 lanes of an aligned lane group; every lane gets the total.
__device__ __forceinline__ float sum8(float v) {
  v = dpp_add<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);   // row_half_mirror
  return v;
}

__host__ __device__ constexpr int gray(int i) { return i ^ (i >> 1); }
__host__ __device__ constexpr int ctz6(int i) {
  return (i & 1) ? 0 : (i & 2) ? 1 : (i & 4) ? 2 : (i & 8) ? 3 : (i & 16) ? 4 : 5;
}

// Activations of byte position p of slice sl for token t (zero past K).
__device__ __forceinline__ void load_x(__amdgpu_buffer_rsrc_t ares, int64_t K, int t, int sl,
                                       int p, float4& x0, float4& x1) {
  const int64_t k0 = (int64_t)sl * kSliceBits + 8 * p;
  const uint32_t base = static_cast<uint32_t>(((int64_t)t * K + k0) * 4);
  const uint32_t o0 = (k0 + 4 <= K) ? base : kNoLoad;
  const uint32_t o1 = (k0 + 8 <= K) ? base + 16 : kNoLoad;
  const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(ares, o0, 0, 0);
  const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(ares, o1, 0, 0);
  __builtin_memcpy(&x0, &v0, 16);
  __builtin_memcpy(&x1, &v1, 16);
}

#ifndef LQ_GEMV1_WAVES
#define LQ_GEMV1_WAVES 16
#endif
#ifndef LQ_GEMV1_DEPTH
#define LQ_GEMV1_DEPTH 3
#endif
constexpr int kWaves = LQ_GEMV1_WAVES;         // 16: four waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kDepth = LQ_GEMV1_DEPTH;         // granules in flight per wave
constexpr int kGranuleRows = 16;
constexpr int kMaxGroups = 256;                // workgroups of one launch (at most)
// A workgroup whose range crosses a slice boundary builds two tables and
// runs two padded runs per wave: it gets this fraction less work.
#ifndef LQ_GEMV1_STRADDLE
#define LQ_GEMV1_STRADDLE 0.2
#endif
constexpr double kStraddleCost = LQ_GEMV1_STRADDLE;
constexpr int kTableHalves = 32768;            // float16 entries per table

// Slot of byte position p = 16c + 4d + b of a slice (c: 16-byte chunk, d:
// dword, b: byte) in a float16 table, whose entry (slot, v) sits at byte
// 256 v + 2 slot:  slot bits [0] = d & 1, [2:1] = b, [5:3] = c, [6] = d >> 1.
// At lookup step i, lane (r, c) reads byte b = (i + r) & 3 of its dword d;
// the 32 lanes of a half-wave (r < 4) then hit banks (slot >> 1) % 32 =
// 4c + b: all different.  h_pos inverts h_slot.
__host__ __device__ constexpr int h_slot(int p) {
  return ((p >> 2) & 1) | ((p & 3) << 1) | (((p >> 4) & 7) << 3) | (((p >> 3) & 1) << 6);
}
__host__ __device__ constexpr int h_pos(int sl) {
  return 16 * ((sl >> 3) & 7) + 4 * ((sl & 1) | (((sl >> 6) & 1) << 1)) + ((sl >> 1) & 3);
}

struct Sched1 {
  int64_t NG;   // 16-row granules per slice
  int64_t T;    // granules in all: S * NG
  int S;        // 1024-bit slices
  int G;        // workgroups
  int64_t start[kMaxGroups + 1];   // workgroup w: granules [start[w], start[w + 1])
};

// v, available only once `dep` is: ties a later memory operation to the wait
// for the load that produced `dep`.
__device__ __forceinline__ uint32_t after(uint32_t v, uint32_t dep) {
  asm volatile("; after %1" : "+v"(v) : "v"(dep));
  return v;
}

// acc + the float16 in the low half of h, in float32 (one v_fma_mix_f32).
__device__ __forceinline__ float add_h(float acc, uint32_t h) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(acc));
  return r;
}

// Power of two 2^(11 - e) with max|x| = f * 2^e, f in [0.5, 1): entries of
// the scaled table stay below 8 * 2^e * 2^(11 - e) = 2^14.
// e_up = e - 11 is the exponent of the inverse.
__device__ __forceinline__ float table_scale(float xmax, int& e_up) {
  if (!(xmax > 0.f)) {
    e_up = 0;
    return 1.f;
  }
  int e;
  (void)frexpf(xmax, &e);
  e_up = e - 11;
  return ldexpf(1.f, 11 - e);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two float32 values as two float16 (round to nearest even) in one word.
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  const float2_t f = {lo, hi};
  const half2_t h = __builtin_convertvector(f, half2_t);   // v_cvt_pk_f16_f32
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// Inputs of the lift when it runs in the kernel's table prologue (the fused
// one-token layer): a [n] and the block-diagonal T^-1 [n/128][128][128] of
// one element type, M [d][D].
struct LiftIn {
  const void* a;
  const void* t;
  const float* M;
  int d;
  int D;
};

// 16 consecutive elements at index i (a multiple of 8), raw: two 16-byte
// vectors for 16-bit types (r[0..1]), four for float32 (r[0..3]).
template <int DT>
__device__ __forceinline__ void load16raw(const void* base, int64_t i, uint4 (&r)[4]) {
  if constexpr (DT == LQ_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = p[k];
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + i);
    r[0] = p[0];
    r[1] = p[1];
  }
}

// Element k (< 16) of a raw run.
template <int DT>
__device__ __forceinline__ float raw_elem(const uint4 (&r)[4], int k) {
  if constexpr (DT == LQ_F32) {
    const uint4 q = r[k >> 2];
    const uint32_t wv = (k & 3) == 0 ? q.x : (k & 3) == 1 ? q.y : (k & 3) == 2 ? q.z : q.w;
    return __uint_as_float(wv);
  } else {
    const uint4 q = r[k >> 3];
    const int h = (k & 7) >> 1;
    const uint32_t wv = h == 0 ? q.x : h == 1 ? q.y : h == 2 ? q.z : q.w;
    if constexpr (DT == LQ_BF16)
      return __uint_as_float((k & 1) ? (wv & 0xFFFF0000u) : (wv << 16));
    else
      return f16_bits_to_float(static_cast<uint16_t>((k & 1) ? (wv >> 16) : (wv & 0xFFFFu)));
  }
}

constexpr int kMaxLiftCh = kSliceBits + 2 * 64;   // channels behind one slice (D >= d, d <= 64)

// Float16 table of one slice, built by the WAVES waves.  Flipping every bit
// of a weight byte flips every sign, so E[255 - v] = -E[v]: wave w computes
// the entries of v in [VB w, VB w + VB), VB = 128 / WAVES (low bits of v in
// Gray-code order, one add per entry), and writes them and their negations
// (sign bits flipped: exact) for slots 2 lane and 2 lane + 1, one packed
// 32-bit LDS store per v.  x0, x1: the 8 scaled activations of the byte
// positions of the two slots.
template <int WAVES>
__device__ __forceinline__ void build_table16(uint16_t* __restrict__ tab, const float (&x0)[8],
                                              const float (&x1)[8], int wave, int lane) {
  constexpr int VB = 128 / WAVES;
  constexpr int LB = VB == 16 ? 4 : VB == 8 ? 3 : 2;     // Gray-coded low bits
  float v0 = -x0[7], v1 = -x1[7];                          // bit 7 of v is 0
#pragma unroll
  for (int t = 0; t < LB; ++t) {
    v0 -= x0[t];
    v1 -= x1[t];
  }
#pragma unroll
  for (int t = LB; t < 7; ++t) {
    const bool on = (wave >> (t - LB)) & 1;
    v0 += on ? x0[t] : -x0[t];
    v1 += on ? x1[t] : -x1[t];
  }
  uint32_t* lo = reinterpret_cast<uint32_t*>(tab) + (VB * wave) * 64 + lane;
  uint32_t* hi = reinterpret_cast<uint32_t*>(tab) + (255 - VB * wave) * 64 + lane;
  auto put = [&](int i) {
    const uint32_t h = pack_h2(v0, v1);
    lo[gray(i) * 64] = h;
    hi[-gray(i) * 64] = h ^ 0x80008000u;
  };
  put(0);
#pragma unroll
  for (int i = 1; i < VB; ++i) {
    const int t = ctz6(i);
    const bool up = (gray(i) >> t) & 1;
    v0 = up ? v0 + 2.f * x0[t] : v0 - 2.f * x0[t];
    v1 = up ? v1 + 2.f * x1[t] : v1 - 2.f * x1[t];
    put(i);
  }
}

// LDT < 0: the lifted activations a_hat come from memory.  LDT = the element
// type of a and T^-1: the table prologue computes the slice's a_hat itself
// (the fused layer): u = T^-1 a for the slice's channels, 8 lanes per
// channel with 16 of the 128 terms each (added across the 8 lanes), then
// a_hat[g D + j] = sum_r M[r][j] u[g d + r], one position per thread.
template <bool SPLIT, int LDT>
__global__ void __launch_bounds__(kThreads, 1) gemv1_kernel(
    const uint32_t* __restrict__ w, int64_t m, int64_t K, int64_t ldw,
    const float* __restrict__ s, const float* __restrict__ ah, float* __restrict__ out,
    float* __restrict__ partials, Sched1 sc, uint32_t w_bytes, uint32_t a_bytes, LiftIn li) {
  __shared__ __attribute__((aligned(16))) uint16_t tabs[2 * kTableHalves];   // 128 KB
  constexpr bool kFused = LDT >= 0;
  __shared__ __attribute__((aligned(16))) float ul[kFused ? kMaxLiftCh : 1];   // u of the slice
  __shared__ __attribute__((aligned(16))) float xs[kFused ? 2 * kSliceBits : 1];  // a_hat
  static_assert(kWaves >= 8 && (kWaves & (kWaves - 1)) == 0 && kWaves <= 32, "8..32 waves");
  constexpr int D = kDepth;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups are dispatched round-robin over the 8 XCDs.  With the lift in
  // the prologue, the ones on an XCD take consecutive ranges, so that the
  // workgroups sharing a slice (and its T^-1 rows) mostly share an L2.
  int wg = blockIdx.x;
  if (kFused && (sc.G & 7) == 0) wg = (blockIdx.x & 7) * (sc.G >> 3) + (blockIdx.x >> 3);
  const int64_t t_begin = sc.start[wg];
  const int64_t t_end = sc.start[wg + 1];
  if (t_begin >= t_end) return;
  const int sl_first = static_cast<int>(t_begin / sc.NG);
  const int sl_last = static_cast<int>((t_end - 1) / sc.NG);
  const int NG = static_cast<int>(sc.NG);       // < 2^22: m * ldw * 4 <= 2^30, ldw >= 4

  const int r = lane >> 3;                      // rows r and r + 8 of the granule
  const int c = lane & 7;                       // 16-byte chunk of the 128-byte slice row
  // Address of entry (slot, v) of table t for byte b of dword d of the
  // lane's chunk: 2 slot = (16c + 4b) + (2 (d & 1) + 128 (d >> 1)).  One
  // v_perm_b32 builds 65536 t + 256 v + 16c + 4b from the weight dword (byte
  // 1: the weight byte) and a lane constant (byte 0: 16c + 4b, byte 2: t);
  // the part that depends on d only goes in the LDS read's offset field.
  uint32_t lc[2][4], sel[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (i + (r & 3)) & 3;
    sel[i] = 0u | ((4u + b) << 8) | (0x02u << 16) | (0x0Cu << 24);
#pragma unroll
    for (int t = 0; t < 2; ++t) lc[t][i] = (16u * c + 4u * b) | (static_cast<uint32_t>(t) << 16);
  }
  constexpr int kDwordOff[4] = {0, 2, 128, 130};

  // Weight loads: per-lane offsets (rows r and r + 8, chunk c) plus a scalar
  // granule offset.  Lanes past the row's last weight byte read bytes that
  // pair with zero activations (their entries are 0); rows past m fall past
  // the end of `w` (w_bytes = m * row_bytes), where the buffer's range check
  // returns zeros, as it does for the scalar kNoLoad.  Offsets stay below
  // 2^31 + 2^25 (row_bytes <= 2^21), so nothing wraps.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w), (short)0, static_cast<int>(w_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ah), (short)0, static_cast<int>(a_bytes), 0x00020000);
  const uint32_t row_bytes = static_cast<uint32_t>(ldw * 4);
  const uint32_t granule_bytes = kGranuleRows * row_bytes;
  const uint32_t lane_off0 = static_cast<uint32_t>(r) * row_bytes + 16 * c;
  const uint32_t lane_off1 = lane_off0 + 8 * row_bytes;

  // This workgroup's granules of slice sl: [lo, hi) within the slice; this
  // wave's run of them: [run_a, run_b).
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

  // Load cursor (all scalar).  Each slice's run is processed in rounds of D
  // ring slots, the last round padded with empty slots, so every slice
  // starts at slot 0; the cursor runs one round ahead of the granules being
  // processed and so only changes slice between rounds.
  int ld_sl = sl_first - 1, ld_k = 0, ld_n = 0, ld_slots = 0;
  uint32_t ld_off = 0;                          // offset of the next granule of the run
  auto ld_next_slice = [&]() {
    do {
      ++ld_sl;
      ld_k = 0;
      if (ld_sl <= sl_last) {
        const int a = run_a(ld_sl);
        ld_n = run_b(ld_sl) - a;
        ld_slots = (ld_n + D - 1) / D * D;
        ld_off = static_cast<uint32_t>(a) * granule_bytes +
                 static_cast<uint32_t>(ld_sl) * kSliceBytes;
      } else {
        ld_n = 0;
        ld_slots = 1 << 30;
      }
    } while (ld_slots == 0);
  };
  auto issue = [&](uint4 (&dst)[2]) {
    const uint32_t so = ld_k < ld_n ? ld_off : kNoLoad;
    const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(wres, lane_off0, so, 0);
    const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(wres, lane_off1, so, 0);
    ld_off += granule_bytes;
    ++ld_k;
    __builtin_memcpy(&dst[0], &v0, 16);
    __builtin_memcpy(&dst[1], &v1, 16);
  };

  // Tables of slices sp and sp + 1 (the second only if the range reaches
  // it).  Every wave builds part of each table for all 128 slots (lane l:
  // slots 2l and 2l + 1), so it loads the activations of all the slice's byte
  // positions, and takes their largest magnitude (the table's scale) in the
  // wave.  These loads are issued before any weight load of the workgroup
  // (the first barrier), so the weights queue behind them; with `first` each
  // wave then issues two granules of weights, which stream in while the
  // tables are built, and the rest of its ring after (issuing all of it at
  // once would stall on the full memory queue).
  uint4 wb[D][2];
  float scale_up[2];
  // Fused layer: a_hat of slice sl into xs[t * 1024 ..] (zero past K).  The
  // T^-1 rows and activations of up to 3 passes of 128 channels are loaded
  // before any is used; `first` issues the workgroup's first two granules
  // of weights after the first loads, so they stream during the lift.
  auto lift_slice = [&](int sl, int t, bool first) {
    if constexpr (kFused) {
      const int64_t k0 = (int64_t)sl * kSliceBits;
      const int64_t kend = k0 + kSliceBits < K ? k0 + kSliceBits : K;
      const int64_t g_lo = k0 / li.D;
      const int64_t c_lo = g_lo * li.d;
      const int64_t c_hi = ((kend - 1) / li.D + 1) * li.d;
      const int nch = static_cast<int>(c_hi - c_lo);
      const int sub = tid & 7;                  // 16 of the row's 128 terms
      const int npass = (nch + 127) / 128;
      bool issued = !first;
      constexpr int kP = LDT == LQ_F32 ? 1 : 3;  // passes in flight
      for (int p0 = 0; p0 < npass; p0 += kP) {
        uint4 tv[kP][4], av[kP][4];
#pragma unroll
        for (int u = 0; u < kP; ++u) {
          const int ci = (p0 + u) * 128 + (tid >> 3);
          if (p0 + u < npass && ci < nch) {
            const int64_t c = c_lo + ci;
            const int64_t q = c >> 7;
            load16raw<LDT>(li.t, (q * 128 + (c & 127)) * 128 + 16 * sub, tv[u]);
            load16raw<LDT>(li.a, q * 128 + 16 * sub, av[u]);
          }
        }
        if (!issued) {
          ld_next_slice();
          issue(wb[0]);
          issue(wb[1]);
          issued = true;
        }
#pragma unroll
        for (int u = 0; u < kP; ++u) {
          const int ci = (p0 + u) * 128 + (tid >> 3);
          float acc = 0.f;
          if (p0 + u < npass && ci < nch) {
#pragma unroll
            for (int k = 0; k < 16; ++k)
              acc = fmaf(raw_elem<LDT>(tv[u], k), raw_elem<LDT>(av[u], k), acc);
          }
          acc = sum8(acc);
          if (p0 + u < npass && ci < nch && sub == 0) ul[ci] = acc;
        }
      }
      __syncthreads();                          // u complete; xs of the last tables read
      {
        const int64_t k = k0 + tid;
        float v = 0.f;
        if (k < kend) {
          const int64_t g = k / li.D;
          const int j = static_cast<int>(k - g * li.D);
          const float* ur = ul + (g * li.d - c_lo);
          for (int r2 = 0; r2 < li.d; ++r2) v = fmaf(li.M[r2 * li.D + j], ur[r2], v);
        }
        xs[t * kSliceBits + tid] = v;
      }
      __syncthreads();                          // xs complete; ul free again
    }
  };
  auto tables = [&](int sp, bool first) {
    const int nt = sp + 1 <= sl_last ? 2 : 1;
    float4 xa[2][4];
    if constexpr (kFused) {
      // every wave is past its lookups of the old tables once it reaches the
      // lift's first barrier
      lift_slice(sp, 0, first);
      if (nt == 2) lift_slice(sp + 1, 1, false);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (t < nt) {
          const float4* x4 = reinterpret_cast<const float4*>(xs + t * kSliceBits);
          xa[t][0] = x4[2 * h_pos(2 * lane)];
          xa[t][1] = x4[2 * h_pos(2 * lane) + 1];
          xa[t][2] = x4[2 * h_pos(2 * lane + 1)];
          xa[t][3] = x4[2 * h_pos(2 * lane + 1) + 1];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (t < nt) {
          load_x(ares, K, 0, sp + t, h_pos(2 * lane), xa[t][0], xa[t][1]);
          load_x(ares, K, 0, sp + t, h_pos(2 * lane + 1), xa[t][2], xa[t][3]);
        }
      }
      __syncthreads();                          // activations requested before any weight;
                                                // nobody reads the old tables any more
      if (first) {
        ld_next_slice();
        issue(wb[0]);
        issue(wb[1]);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t < nt) {
        float mx = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xa[t][k].x), fabsf(xa[t][k].y)),
                               fmaxf(fabsf(xa[t][k].z), fabsf(xa[t][k].w))));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        int e_up;
        const float sd = table_scale(mx, e_up);
        scale_up[t] = ldexpf(1.f, e_up);        // exact inverse of sd
        const float y0[8] = {xa[t][0].x * sd, xa[t][0].y * sd, xa[t][0].z * sd, xa[t][0].w * sd,
                             xa[t][1].x * sd, xa[t][1].y * sd, xa[t][1].z * sd, xa[t][1].w * sd};
        const float y1[8] = {xa[t][2].x * sd, xa[t][2].y * sd, xa[t][2].z * sd, xa[t][2].w * sd,
                             xa[t][3].x * sd, xa[t][3].y * sd, xa[t][3].z * sd, xa[t][3].w * sd};
        build_table16<kWaves>(tabs + t * kTableHalves, y0, y1, wave, lane);
      }
    }
    __syncthreads();
    if (first) {
#pragma unroll
      for (int e = 2; e < D; ++e) issue(wb[e]);
    }
  };
  tables(sl_first, true);

  const char* tb = reinterpret_cast<const char*>(tabs);
  // Sum of the table-TI entries of one row's 16 weight bytes held by a lane.
  auto lookup_row = [&]<int TI>(const uint32_t (&wd)[4]) -> float {
    float a[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      a[d] = add_h(0.f, *reinterpret_cast<const uint16_t*>(
                            tb + __builtin_amdgcn_perm(wd[d], lc[TI][0], sel[0]) + kDwordOff[d]));
#pragma unroll
    for (int i = 1; i < 4; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        a[d] = add_h(a[d], *reinterpret_cast<const uint16_t*>(
                               tb + __builtin_amdgcn_perm(wd[d], lc[TI][i], sel[i]) +
                               kDwordOff[d]));
    return (a[0] + a[1]) + (a[2] + a[3]);
  };
  int rnd = 0;                                  // rounds processed so far
  auto process_run = [&](auto tsel, int sl) {
    constexpr int TI = decltype(tsel)::value;
    const int a = run_a(sl);
    const int n = run_b(sl) - a;
    const float up = scale_up[TI];
    float* pout = SPLIT ? partials + ((int64_t)a * sc.S + sl) * kGranuleRows
                        : out + (int64_t)kGranuleRows * a;
    const float* ps = s + (int64_t)kGranuleRows * a;
    const int64_t pstep = SPLIT ? (int64_t)sc.S * kGranuleRows : kGranuleRows;
    for (int k0 = 0; k0 < n; k0 += D, ++rnd) {
      if (ld_k >= ld_slots) ld_next_slice();    // this round's loads go to the next slice
      uint32_t dep0 = 0;                        // a word of the round's first granule
#pragma unroll
      for (int e = 0; e < D; ++e) {
        if (k0 + e < n) {                       // always true for e = 0
          const uint32_t wd0[4] = {wb[e][0].x, wb[e][0].y, wb[e][0].z, wb[e][0].w};
          const uint32_t wd1[4] = {wb[e][1].x, wb[e][1].y, wb[e][1].z, wb[e][1].w};
          if (e == 0) dep0 = wd0[0];
          // one row's lookups at a time keeps the loaded entries of only 16
          // lookups live
          const float v0 = sum8(lookup_row.template operator()<TI>(wd0)) * up;
          __builtin_amdgcn_sched_barrier(0);
          const float v1 = sum8(lookup_row.template operator()<TI>(wd1)) * up;
          // lanes c = 0 and 1 write rows r and r + 8
          const int rr = r + 8 * c;
          const float v = c == 0 ? v0 : v1;
          if constexpr (SPLIT) {
            if (c < 2) pout[rr] = v;
          } else {
            const int64_t row = (int64_t)kGranuleRows * (a + k0 + e) + rr;
            if (c < 2 && row < m) pout[rr] = ps[rr] * v;
            ps += pstep;
          }
          pout += pstep;
        }
        issue(wb[e]);
      }
    }
  };

  for (int sl = sl_first; sl <= sl_last; ++sl) {   // the same slices in every wave
    const int rel = sl - sl_first;
    if (rel >= 2 && (rel & 1) == 0) tables(sl, false);   // only when the range spans > 2 slices
    if ((rel & 1) == 0)
      process_run(std::integral_constant<int, 0>{}, sl);
    else
      process_run(std::integral_constant<int, 1>{}, sl);
  }
}

// out[i] = s[i] * (sum over slices q of partials[i / 16][q][i % 16]), added in
// a fixed order: P lanes share a row (P a power of two with at most 8 slices
// per lane, so all of a lane's loads are in flight at once), lane part j adds
// slices j, j + P, ... in order, and the P parts combine by a fixed tree.  A
// wave covers 64 / P rows.
template <int P>
__global__ void __launch_bounds__(256) gemv1_reduce_kernel(const float* __restrict__ partials,
                                                           const float* __restrict__ s,
                                                           float* __restrict__ out, int64_t m,
                                                           int S) {
  constexpr int R = 64 / P;                     // rows per wave
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int part = lane % P;
  const int64_t row = wave * R + lane / P;
  float sum = 0.f;
  if (row < m) {
    const float* p = partials + ((row >> 4) * S) * kGranuleRows + (row & 15);
    for (int q0 = part; q0 < S; q0 += 8 * P) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u * P;
        v[u] = q < S ? p[(int64_t)q * kGranuleRows] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
  }
#pragma unroll
  for (int o = 1; o < P; o <<= 1) sum += __shfl_xor(sum, o);
  if (row < m && part == 0) out[row] = s[row] * sum;
}

template <int P>
static void launch_reduce(const float* partials, const float* s, float* out, int64_t m, int S,
                          hipStream_t st) {
  constexpr int rows_per_block = 4 * (64 / P);
  hipLaunchKernelGGL(gemv1_reduce_kernel<P>,
                     dim3(static_cast<unsigned>((m + rows_per_block - 1) / rows_per_block)),
                     dim3(256), 0, st, partials, s, out, m, S);
}

// Ranges of the workgroups over the (slice, granule) order.  A range that
// crosses a slice boundary pays for a second table and a second run per
// wave, about kStraddleCost of a share: the granules are laid on a line with
// a gap of c = kStraddleCost * share after each slice, the line is cut into
// G equal pieces, and each piece takes the granules it covers (a piece that
// contains a gap gets c fewer).  Cut points inside a gap go to the slice end.
Sched1 make_sched1(int64_t m, int64_t K) {
  Sched1 sc{};
  sc.S = static_cast<int>((K + kSliceBits - 1) / kSliceBits);
  sc.NG = (m + kGranuleRows - 1) / kGranuleRows;
  sc.T = sc.NG * sc.S;
  const int64_t gmax = (sc.T + kWaves - 1) / kWaves;
  int cus = num_cus();
  if (cus > kMaxGroups) cus = kMaxGroups;
  sc.G = static_cast<int>(gmax < cus ? gmax : cus);
  const double share = (double)sc.T / sc.G;
  const double c = share < (double)sc.NG ? kStraddleCost * share : 0.0;
  const double span = (double)sc.NG + c;                 // a slice and its gap
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

template <int P>
static void launch_reduce(const float* partials, const float* s, float* out, int64_t m, int S,
                          hipStream_t st);

void reduce_slices(const float* partials, const float* s, float* out, int64_t m, int S,
                   hipStream_t st) {
  const int need = (S + 7) / 8;                 // parts so that each adds <= 8 slices
  if (need <= 1)
    launch_reduce<1>(partials, s, out, m, S, st);
  else if (need <= 2)
    launch_reduce<2>(partials, s, out, m, S, st);
  else if (need <= 4)
    launch_reduce<4>(partials, s, out, m, S, st);
  else if (need <= 8)
    launch_reduce<8>(partials, s, out, m, S, st);
  else
    launch_reduce<16>(partials, s, out, m, S, st);
}

template <int LDT>
hipError_t launch_fused(const LiftIn& li, const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                        const float* s, float* out, void* ws, hipStream_t st) {
  const Sched1 sc = make_sched1(m, K);
  const uint32_t w_bytes = static_cast<uint32_t>(m * ldw * 4);
  const uint32_t a_bytes = static_cast<uint32_t>(K * 4);
  if (sc.S == 1) {
    hipLaunchKernelGGL((gemv1_kernel<false, LDT>), dim3(sc.G), dim3(kThreads), 0, st, w, m, K,
                       ldw, s, nullptr, out, nullptr, sc, w_bytes, a_bytes, li);
    return hipGetLastError();
  }
  float* partials = static_cast<float*>(ws);
  hipLaunchKernelGGL((gemv1_kernel<true, LDT>), dim3(sc.G), dim3(kThreads), 0, st, w, m, K, ldw,
                     s, nullptr, out, partials, sc, w_bytes, a_bytes, li);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  reduce_slices(partials, s, out, m, sc.S, st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layer_b1(const void* a, lq_dtype dt, const void* t_inv, const float* M, int d,
                           int D, const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                           const float* s, float* out, void* ws, hipStream_t st) {
  const LiftIn li{a, t_inv, M, d, D};
  switch (dt) {
    case LQ_F32: return launch_fused<LQ_F32>(li, w, m, K, ldw, s, out, ws, st);
    case LQ_F16: return launch_fused<LQ_F16>(li, w, m, K, ldw, s, out, ws, st);
    default: return launch_fused<LQ_BF16>(li, w, m, K, ldw, s, out, ws, st);
  }
}

size_t gemv1_workspace_bytes(int64_t m, int64_t K) {
  const Sched1 sc = make_sched1(m, K);
  if (sc.S == 1) return 0;
  // one partial sum per (granule row, slice); every one is written each call
  return sizeof(float) * kGranuleRows * (size_t)sc.NG * sc.S;
}

}  // namespace lq
