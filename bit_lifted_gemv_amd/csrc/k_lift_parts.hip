// Lift straight into the operand image of the several-token GEMV (LiftQuant
// notes, 关键设计 4: the small transform of the activations, done once per
// input, then the 1-bit product; 关键设计 1 for the per-group M):
//   u[b][128q + r]    = sum_c T_q[r][c] * a[b][128q + c]
//   a_hat[b][g D + j] = sum_{r<d} M[r][j] * u[b][g d + r]
// and then, instead of writing a_hat, the float8 parts and exponents of
// f4m_image.h, so that the GEMV needs no preparation launch.
//
// One workgroup of 4 waves per span (512 lifted positions) and group of 2,
// 4 or 8 (as the span count allows about one workgroup per compute unit) of the
// image's 16 token columns (every column is written, zero past B): the
// conversion is a chain of dependent steps per value, so the work is spread
// over more compute units than there are spans.  The workgroup
// computes u for its tokens and the channels of every lift group that
// overlaps the span (rounded out to 16-channel tiles, which never straddle a
// 128-block) on v_mfma_f32_16x16x32_{f16,bf16}: A = 16 token rows (2, 4 or 8 live)
// x 32 positions of a, B = 32 positions x 16 channels of T^-1 rows, both
// exact 16-bit values, float32 sums; the tiles are dealt to the waves round
// robin, all loads of a wave issued before its products.  u goes to LDS;
// then a thread per (token, group) multiplies its d values of u by M (staged
// in LDS, read at addresses common to most of the wave's lanes) and writes
// the group's positions that fall inside the span to an LDS row of a_hat
// (zero past K and past B); then a thread per (step, token, word, half)
// reads its word and writes its parts.  Padding spans past K come out zero.
#include "f4m_image.h"
#include "lq_internal.h"

namespace lq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTB = 128;                          // transform block
constexpr int kXP = f4m::kSpanPositions + 4;      // floats per token row of a_hat in LDS
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kNoLoad = 0x80000000u;         // past every range: the load gives zero

template <int DT>
__device__ __forceinline__ f32x4 mfma16x32(const uint4& a, const uint4& b, const f32x4& c);

template <>
__device__ __forceinline__ f32x4 mfma16x32<LQ_F16>(const uint4& a, const uint4& b, const f32x4& c) {
  half8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mfma16x32<LQ_BF16>(const uint4& a, const uint4& b, const f32x4& c) {
  bf16x8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

// Channels of u a span needs, rounded out to 16: at most this many.
__host__ __device__ constexpr int max_span_channels(int d, int D) {
  return ((f4m::kSpanPositions - 1) / D + 2) * d + 32;
}

// DT: type of a and T^-1; DD = d; kTok: token columns per workgroup (2, 4
// or 8).  cpad: floats per token row of u in LDS.
template <int DT, int DD, int kTok>
__global__ void __launch_bounds__(kThreads) lift_parts_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ t_inv,
    const float* __restrict__ M, int B, int n, int D, int cpad, uint8_t* __restrict__ image) {
  extern __shared__ float lds[];
  float* su = lds;                               // [kTok][cpad]
  float* sx = lds + kTok * cpad;                 // [kTok][kXP]
  float* sM = sx + kTok * kXP;                   // [d][D]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x;
  const int tok0 = blockIdx.y * kTok;            // first token column
  const int p0 = c * f4m::kSpanPositions;
  const int ngroups = n / DD;
  const int g_lo = min(p0 / D, ngroups);
  const int g_hi = min((p0 + f4m::kSpanPositions - 1) / D + 1, ngroups);   // exclusive
  const int ch0 = (g_lo * DD) & ~15;
  const int ch1 = min(n, (g_hi * DD + 15) & ~15);
  const int ntiles = ch1 > ch0 ? (ch1 - ch0) / 16 : 0;

  // M is staged in LDS: its first kThreads entries are loaded ahead of the
  // tile operands and stored after them (one round trip for both).
  const float m0 = tid < DD * D ? M[tid] : 0.f;

  // ---- u for channels ch0 .. ch1 - 1, one 16 x 16 tile (tokens x channels)
  // at a time.  Lane (i, kg): token tok0 + i of A (zero for i >= kTok and past
  // B), channel i of B, positions 32 ks + 8 kg .. + 7 of the block in both.
  const int li = lane & 15;
  const int kg = lane >> 4;
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a), (short)0,
      static_cast<int>(static_cast<uint32_t>(B) * static_cast<uint32_t>(n) * 2u), kRsrcWord3);
  auto load_tile = [&](int t, uint4 (&af)[4], uint4 (&bt)[4]) {
    const int tt = t < ntiles ? t : 0;            // a past-the-end tile reloads tile 0, unused
    const int cb = ch0 + 16 * tt;                 // first channel of the tile
    const int q = cb / kTB;
    const uint32_t a_off = li < kTok && tok0 + li < B
        ? (static_cast<uint32_t>(tok0 + li) * n + q * kTB + 8 * kg) * 2u : kNoLoad;
    const uint16_t* trow = t_inv + (static_cast<int64_t>(cb + li)) * kTB + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const auto r = __builtin_amdgcn_raw_buffer_load_b128(ares, a_off, 64 * ks, 0);
      __builtin_memcpy(&af[ks], &r, 16);
      bt[ks] = *reinterpret_cast<const uint4*>(trow + 32 * ks);
    }
  };
  auto mma_tile = [&](int t, const uint4 (&af)[4], const uint4 (&bt)[4]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma16x32<DT>(af[ks], bt[ks], acc);
    // D[token][channel]: lane (i, kg) holds channel i, tokens 4 kg .. 4 kg + 3
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * kg + e < kTok) su[(4 * kg + e) * cpad + 16 * t + li] = acc[e];
  };
  // kTW tiles per wave per round (one round at the workload shapes), every
  // load of a round issued before its MFMAs.
  constexpr int kW = kThreads / 64;
  constexpr int kTW = 5;
  for (int t0 = 0; t0 < ntiles; t0 += kTW * kW) {
    uint4 af[kTW][4], bt[kTW][4];
#pragma unroll
    for (int i = 0; i < kTW; ++i) load_tile(t0 + wave + i * kW, af[i], bt[i]);
    if (t0 == 0) {
      for (int i = tid; i < kTok * kXP; i += kThreads) sx[i] = 0.f;
      if (tid < DD * D) sM[tid] = m0;
      for (int i = tid + kThreads; i < DD * D; i += kThreads) sM[i] = M[i];
    }
#pragma unroll
    for (int i = 0; i < kTW; ++i)
      if (t0 + wave + i * kW < ntiles) mma_tile(t0 + wave + i * kW, af[i], bt[i]);
  }
  if (ntiles == 0) {
    for (int i = tid; i < kTok * kXP; i += kThreads) sx[i] = 0.f;
    if (tid < DD * D) sM[tid] = m0;
    for (int i = tid + kThreads; i < DD * D; i += kThreads) sM[i] = M[i];
  }
  __syncthreads();

  // ---- a_hat of the span: a thread per (token, group); the positions of a
  // group that straddles the span's ends are written by both spans.
  const int ng = g_hi - g_lo;
  for (int pr = tid; pr < kTok * ng; pr += kThreads) {
    const int tok = pr / ng;
    const int g = g_lo + (pr - tok * ng);
    float uv[DD];
#pragma unroll
    for (int r = 0; r < DD; ++r) uv[r] = su[tok * cpad + g * DD - ch0 + r];
    const int pg = g * D - p0;                   // the group's first position in the span
    const int j0 = max(0, -pg);
    const int j1 = min(D, f4m::kSpanPositions - pg);
    for (int j = j0; j < j1; ++j) {
      float o = 0.f;
#pragma unroll
      for (int r = 0; r < DD; ++r) o = fmaf(sM[r * D + j], uv[r], o);
      sx[tok * kXP + pg + j] = o;
    }
  }
  __syncthreads();

  // ---- parts: thread (u, n, g, h) takes token tok0 + n's word 4 g + u
  // (waves 0 and 1; the eight threads of a (step, token) are consecutive)
  if (tid >= 4 * kTok * 8) return;
  const int h = tid & 1;
  const int g = (tid >> 1) & 3;
  const int nt = (tid >> 3) & (kTok - 1);
  const int u = tid / (8 * kTok);
  float x[32];
  const float4* src = reinterpret_cast<const float4*>(sx + nt * kXP + 32 * (4 * g + u));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float4 v = src[j];
    x[4 * j] = v.x;
    x[4 * j + 1] = v.y;
    x[4 * j + 2] = v.z;
    x[4 * j + 3] = v.w;
  }
  f4m::write_span_parts(x, true, u, tok0 + nt, g, h,
                        image + static_cast<int64_t>(c) * f4m::kSpanBytes);
}

template <int DT, int DD, int kTok>
hipError_t launch_tok(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M,
                      int D, void* image, hipStream_t st) {
  const int64_t K = n / DD * D;
  const int cpad = (max_span_channels(DD, D) + 15) / 16 * 16 + 4;
  const size_t lds = (static_cast<size_t>(kTok) * (cpad + kXP) + DD * D) * 4;
  const void* fn = reinterpret_cast<const void*>(lift_parts_kernel<DT, DD, kTok>);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((lift_parts_kernel<DT, DD, kTok>),
                     dim3(static_cast<unsigned>(f4m::image_spans(K)), 16 / kTok),
                     dim3(kThreads), lds, st, static_cast<const uint16_t*>(a),
                     static_cast<const uint16_t*>(t_inv), M, static_cast<int>(B),
                     static_cast<int>(n), D, cpad, static_cast<uint8_t*>(image));
  return hipGetLastError();
}

// Two token columns per workgroup while that keeps the grid within about
// one workgroup per compute unit, else four, else eight.
template <int DT, int DD>
hipError_t launch_dd(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M,
                     int D, void* image, hipStream_t st) {
  const int64_t spans = f4m::image_spans(n / DD * D);
  if (spans * 8 <= num_cus()) return launch_tok<DT, DD, 2>(a, B, n, t_inv, M, D, image, st);
  if (spans * 4 <= num_cus()) return launch_tok<DT, DD, 4>(a, B, n, t_inv, M, D, image, st);
  return launch_tok<DT, DD, 8>(a, B, n, t_inv, M, D, image, st);
}

template <int DT>
hipError_t launch_t(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M, int d,
                    int D, void* image, hipStream_t st) {
  switch (d) {
    case 4: return launch_dd<DT, 4>(a, B, n, t_inv, M, D, image, st);
    case 8: return launch_dd<DT, 8>(a, B, n, t_inv, M, D, image, st);
    case 16: return launch_dd<DT, 16>(a, B, n, t_inv, M, D, image, st);
    default: return launch_dd<DT, 32>(a, B, n, t_inv, M, D, image, st);
  }
}

}  // namespace

size_t lift_parts_bytes(int64_t K) {
  return static_cast<size_t>(f4m::image_spans(K)) * f4m::kSpanBytes;
}

bool lift_parts_applies(lq_dtype a_dt, lq_dtype t_dt, int64_t B, int64_t n, int d, int D) {
  const int64_t lds =
      (int64_t{8} * ((max_span_channels(d, D) + 15) / 16 * 16 + 4 + kXP) + int64_t{d} * D) * 4;
  return a_dt == t_dt && (a_dt == LQ_F16 || a_dt == LQ_BF16) && B >= 1 && B <= 16 &&
         (d == 4 || d == 8 || d == 16 || d == 32) && D >= d && D <= 256 && lds <= 160 * 1024 &&
         int64_t{16} * n * 2 < (int64_t{1} << 31);
}

hipError_t launch_lift_parts(const void* a, lq_dtype dt, int64_t B, int64_t n, const void* t_inv,
                             const float* M, int d, int D, void* image, hipStream_t st) {
  if (dt == LQ_F16) return launch_t<LQ_F16>(a, B, n, t_inv, M, d, D, image, st);
  return launch_t<LQ_BF16>(a, B, n, t_inv, M, d, D, image, st);
}

}  // namespace lq
