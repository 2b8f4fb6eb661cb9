// Product of 1-bit weights with float lifted activations for 6 to 16 tokens
// on the matrix cores:
//   out[b][i] = s[i] * sum_k sigma_ik * a_hat[b][k],  sigma = 2*bit - 1
// (LiftQuant notes, 关键设计 4: after the activation transform the layer is a
// product of 1-bit weights with floats, scaled per row by s).
//
// Operands of v_mfma_scale_f32_16x16x128_f8f6f4 (16 rows x 128 positions of
// float4 A against 128 positions x 16 columns of float8 B, each B lane with
// its own power-of-two scale).
// - A: the signs as float4 (E2M1) +-1: a set bit gives -1 (nibble 0xA), a
//   clear one +1 (0x2), so the tile holds -sigma and the epilogue multiplies
//   by -s.  Dword q of a lane's operand takes bits q, q + 4, ..., q + 28 of a
//   word of 32 signs: bit 4 t + q moves to bit 3 of nibble t by one shift,
//   and one bitfield insert puts the 0x2 pattern around it.
// - B: the 16 columns are the 16 tokens (zero past B), and each activation
//   is three float8 (E4M3) parts, one per MFMA: per token and step (128
//   positions), with f the biased exponent of their largest |x| and
//   e = min(134 - f, 119), y = x 2^e lies below 256 in magnitude;
//   p0 = fp8(y), p1 = fp8(16 (y - p0)), p2 = fp8(16 (y - p0 - p1 / 16)) (the
//   remainders are exact in float32), and part p's hardware scale is
//   2^(-e - 4 p).  The three MFMAs of a step accumulate into the same tile,
//   so the parts add up inside the accumulator; the error is that of 12
//   significant bits per value, relative to its step's largest value.
//   Products are exact and accumulate in float32.
//
// Position order.  The weights come in spans of 16 words (512 positions);
// lane (i, g) of a 16-row tile loads words 4 g .. 4 g + 3 of the span of row
// i (one 16-byte load covers 64 contiguous bytes of each of the 16 rows).
// Step u of a span takes word 4 g + u from lane group g, whose bit 4 t + q
// is A slot k = 32 g + 8 q + t.  In the float8 B operand, lane group h holds
// k = 16 h .. 16 h + 15 in bytes 0 .. 15 and k = 64 + 16 h .. 64 + 16 h + 15
// in bytes 16 .. 31, so the word's slots 0 .. 15 go to lane group
// 2 (g % 2) and slots 16 .. 31 to lane group 2 (g % 2) + 1, in bytes
// 16 (g / 2) .. 16 (g / 2) + 15.
//
// Kernels.  A preparation kernel writes every word's parts and exponent
// once to the workspace, in the order the B operand is read (per span:
// [step][part][half][lane][16 bytes], so that each 16-byte LDS read of a
// wave covers 1 KB of consecutive banks, then [step][token] exponents).  The main
// kernel gives each wave RT tiles of 16 rows; the 8 waves of a workgroup
// share the parts of one span at a time in LDS (double-buffered, loaded into
// registers two spans ahead and written to LDS one span ahead) and stream
// their weights two spans ahead in registers.  The lifted dimension is split
// over S workgroups so that every compute unit holds one; each split writes
// float32 partial sums to the workspace and a reduction kernel adds them in
// split order and scales by s.  Deterministic.
#include "lq_internal.h"

#include <type_traits>

namespace lq {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kFar = 0x40000000u;     // past every weight range (<= 2^30 bytes)
constexpr int kSpanWords = 16;
constexpr int kPartBytes = 4 * 3 * 64 * 32;            // per span
constexpr int kSpanBytes = kPartBytes + 4 * 16 * 4;    // parts, then exponents
constexpr int kSpanVec = kSpanBytes / 16;
constexpr int kRT = 2;                                 // 16-row tiles per wave

// A per-lane value the compiler cannot fold (kept in a vector register).
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// (x & mask) | (c & ~mask), one v_bfi_b32.
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t x, uint32_t c) {
  return (x & mask) | (c & ~mask);
}

// The A operand of one step from a word of sign bits: -sigma as float4.
__device__ __forceinline__ i32x8 expand_pm(uint32_t w, uint32_t two) {
  const uint32_t m = 0x88888888u;
  i32x8 a;
  a[0] = static_cast<int>(bfi(m, w << 3, two));
  a[1] = static_cast<int>(bfi(m, w << 2, two));
  a[2] = static_cast<int>(bfi(m, w << 1, two));
  a[3] = static_cast<int>(bfi(m, w, two));
  a[4] = a[5] = a[6] = a[7] = 0;               // unused with a float4 A operand
  return a;
}

__device__ __forceinline__ f32x4 mfma(const i32x8& a, const i32x8& b, const f32x4& c, int sc) {
  // A: E2M1 (cbsz 4), scale 2^0; B: E4M3 (blgp 0), scale 2^(sc - 127)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, 127, 0, sc);
}

// Preparation: one thread per (span c, step u, token n, word g, half h):
// the slots 16 h .. 16 h + 15 (q = 2 h, 2 h + 1) of token n's word
// 16 c + 4 g + u.  The eight threads of (c, u, n) are consecutive lanes and
// share their exponent (a butterfly over them).  Positions >= K and tokens
// >= B are zero.
__global__ void __launch_bounds__(256) gemv_f4m_prep_kernel(const float* __restrict__ ah, int B,
                                                            int K, int nspans,
                                                            uint8_t* __restrict__ ws) {
  const int idx = blockIdx.x * 256 + threadIdx.x;   // every lane of a wave runs
  const int h = idx & 1;
  const int g = (idx >> 1) & 3;
  const int n = (idx >> 3) & 15;
  const int u = (idx >> 7) & 3;
  const int c = idx >> 9;
  const bool live = c < nspans;
  const int64_t k0 = (static_cast<int64_t>(c) * kSpanWords + 4 * g + u) * 32;
  // buffer loads: every load is issued at once, and the ones outside the
  // activations (token >= B, position >= K) read zero without a branch
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ah), (short)0, static_cast<int>(static_cast<uint32_t>(B) * K * 4u),
      kRsrcWord3);
  float x[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t k = k0 + 4 * j;               // K % 4 == 0: a 4-group is all in or out
    const uint32_t off = live && n < B && k < K
        ? static_cast<uint32_t>((static_cast<int64_t>(n) * K + k) * 4) : kFar;
    const auto r = __builtin_amdgcn_raw_buffer_load_b128(ares, off, 0, 0);
    float4 v;
    __builtin_memcpy(&v, &r, 16);
    x[4 * j] = v.x;
    x[4 * j + 1] = v.y;
    x[4 * j + 2] = v.z;
    x[4 * j + 3] = v.w;
  }
  uint32_t mb = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) mb = max(mb, __float_as_uint(x[j]) & 0x7FFFFFFFu);
  mb = max(mb, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mb), 1)));
  mb = max(mb, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mb), 2)));
  mb = max(mb, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mb), 4)));
  if (!live) return;
  const int e = mb == 0 ? 0 : min(134 - static_cast<int>(mb >> 23), 119);
  // dword (q', hh) of this half holds slots 8 q + 4 hh .. + 3 (q = 2 h + q'),
  // i.e. positions 4 t + q for t = 4 hh .. 4 hh + 3
  uint32_t d[3][4];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = ldexpf(x[4 * (4 * hh + j) + 2 * h + qq], e);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], v, true);
        d[p][2 * qq + hh] = static_cast<uint32_t>(v);
        if (p < 2) {
          y[0] = 16.f * (y[0] - __builtin_amdgcn_cvt_f32_fp8(v, 0));
          y[1] = 16.f * (y[1] - __builtin_amdgcn_cvt_f32_fp8(v, 1));
          y[2] = 16.f * (y[2] - __builtin_amdgcn_cvt_f32_fp8(v, 2));
          y[3] = 16.f * (y[3] - __builtin_amdgcn_cvt_f32_fp8(v, 3));
        }
      }
    }
  }
  uint8_t* span = ws + static_cast<int64_t>(c) * kSpanBytes;
  const int blane = 16 * (2 * (g & 1) + h) + n;  // B lane group 2 (g % 2) + h
  const int byte0 = 16 * (g >> 1);
#pragma unroll
  for (int p = 0; p < 3; ++p)
    *reinterpret_cast<uint4*>(span + (((u * 3 + p) * 2 + (byte0 >> 4)) * 64 + blane) * 16) =
        make_uint4(d[p][0], d[p][1], d[p][2], d[p][3]);
  if (g == 0 && h == 0) reinterpret_cast<int*>(span + kPartBytes)[u * 16 + n] = e;
}

// RT: 16-row tiles per wave; kW: waves per workgroup.  Grid: x = row groups,
// y = splits of the lifted dimension (whole span pairs each).
template <int RT, int kW>
__global__ void __launch_bounds__(64 * kW, 1) gemv_f4m_kernel(
    const uint32_t* __restrict__ w, int m, int ldw, int nw, const uint8_t* __restrict__ bws,
    int nspans, int B, float* __restrict__ partials) {
  constexpr int kThreads = 64 * kW;
  // parts: kPer vectors per thread; exponents: 16 vectors, threads 0 .. 15
  constexpr int kPer = kPartBytes / 16 / kThreads;
  static_assert(kPer * kThreads * 16 == kPartBytes, "whole vectors per thread");
  __shared__ u32x4 sb[2][kSpanVec];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i = lane & 15;
  const int g = lane >> 4;
  // this split's spans: a whole number of span pairs (nspans is even)
  const int S = gridDim.y;
  const int c0 = 2 * (blockIdx.y * (nspans / 2) / S);
  const int c1 = 2 * ((blockIdx.y + 1) * (nspans / 2) / S);

  // Weights of this workgroup's rows: rows past m read as zero and are
  // never stored; words past a row's last one, nw, are not fetched (they
  // read as zero) and meet zero activations.
  const int wg_row0 = blockIdx.x * kW * 16 * RT;
  const int wg_rows = min(kW * 16 * RT, m - wg_row0);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w + static_cast<int64_t>(wg_row0) * ldw), (short)0,
      static_cast<int>(static_cast<uint32_t>(wg_rows) * static_cast<uint32_t>(ldw) * 4u), kRsrcWord3);
  uint32_t w_off[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
    w_off[t] = static_cast<uint32_t>((wave * 16 * RT + t * 16 + i) * ldw + 4 * g) * 4u;
  auto load_w = [&](int c, int t) -> uint4 {
    const int word0 = c * kSpanWords + 4 * g;
    const uint32_t vo = word0 < nw ? w_off[t] : kFar;
    const int so = c < c1 ? c * kSpanWords * 4 : static_cast<int>(kFar);
    const auto r = __builtin_amdgcn_raw_buffer_load_b128(wres, vo, so, 0);
    uint4 v;
    __builtin_memcpy(&v, &r, 16);
    return v;
  };
  const u32x4* bsrc = reinterpret_cast<const u32x4*>(bws);
  const int xe = tid < 16 ? tid : 0;            // exponent vector of this thread
  auto load_b = [&](int c, u32x4 (&v)[kPer + 1]) {
    const u32x4* src = bsrc + static_cast<int64_t>(c) * kSpanVec;
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = src[tid + k * kThreads];
    v[kPer] = src[kPer * kThreads + xe];
  };
  auto store_b = [&](int buf, const u32x4 (&v)[kPer + 1]) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) sb[buf][tid + k * kThreads] = v[k];
    if (tid < 16) sb[buf][kPer * kThreads + tid] = v[kPer];
  };

  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t two = opaque_v(0x22222222u);

  uint4 wv[2][RT];
  u32x4 nbv[2][kPer + 1];
#pragma unroll
  for (int t = 0; t < RT; ++t) wv[0][t] = load_w(c0, t);
#pragma unroll
  for (int t = 0; t < RT; ++t) wv[1][t] = load_w(c0 + 1, t);
  load_b(c0, nbv[0]);
  load_b(c0 + 1, nbv[1]);
  store_b(0, nbv[0]);
  __syncthreads();

  // One span, c % 2 == P (counted from c0): wv[P] holds its weights, LDS
  // buffer P its parts, nbv[P ^ 1] the next span's parts.  The parts of span
  // c + 2 are loaded first (into nbv[P]); the weight registers are refilled
  // with span c + 2 after the last step; the next span's parts go to the
  // other buffer at the end.
  auto span = [&](auto P, int c) {
    constexpr int p = decltype(P)::value;
    load_b(c + 2, nbv[p]);
    const uint8_t* sp = reinterpret_cast<const uint8_t*>(&sb[p][0]);
    const int* se = reinterpret_cast<const int*>(sp + kPartBytes);
    // B operands of step u (three parts) and its exponent, read one step
    // ahead of their products
    auto read_step = [&](int u, i32x8 (&bf)[3], int& e) {
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const uint4 y0 = *reinterpret_cast<const uint4*>(sp + (((u * 3 + q) * 2) * 64 + lane) * 16);
        const uint4 y1 = *reinterpret_cast<const uint4*>(sp + (((u * 3 + q) * 2 + 1) * 64 + lane) * 16);
        __builtin_memcpy(&bf[q], &y0, 16);
        __builtin_memcpy(reinterpret_cast<char*>(&bf[q]) + 16, &y1, 16);
      }
      e = se[u * 16 + i];
    };
    i32x8 bf[2][3];
    int ex[2];
    read_step(0, bf[0], ex[0]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < 3) read_step(u + 1, bf[(u + 1) & 1], ex[(u + 1) & 1]);
      // keeps the reads of later steps from being hoisted into registers
      asm volatile("" ::: "memory");
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint32_t W = u == 0 ? wv[p][t].x : u == 1 ? wv[p][t].y : u == 2 ? wv[p][t].z : wv[p][t].w;
        const i32x8 a = expand_pm(W, two);
#pragma unroll
        for (int q = 0; q < 3; ++q) acc[t] = mfma(a, bf[u & 1][q], acc[t], 127 - ex[u & 1] - 4 * q);
      }
      // the step's products are issued here, not sunk past later steps
#pragma unroll
      for (int t = 0; t < RT; ++t) asm volatile("" : "+v"(acc[t]));
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) wv[p][t] = load_w(c + 2, t);
    store_b(p ^ 1, nbv[p ^ 1]);
    __syncthreads();
  };
  // Pairs of spans without branches inside the loop body, so the waits on
  // the loads are the same every turn.  The workspace holds two spans more
  // than the layer needs, for the part loads two spans ahead.
  for (int c = c0; c < c1; c += 2) {
    span(std::integral_constant<int, 0>{}, c);
    span(std::integral_constant<int, 1>{}, c + 1);
  }

  // Epilogue.  acc[t][r] = D[row 4 g + r][token i] of tile t (-sum sigma a).
  float* dst = partials + static_cast<int64_t>(blockIdx.y) * B * m;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row0 = wg_row0 + wave * 16 * RT + t * 16 + 4 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + r;
      if (row < m && i < B) dst[static_cast<int64_t>(i) * m + row] = acc[t][r];
    }
  }
}

// out[b][i] = -s[i] * sum over splits of partials[split][b][i], in split
// order, for b < B.
__global__ void __launch_bounds__(256) gemv_f4m_reduce_kernel(const float* __restrict__ partials,
                                                              const float* __restrict__ s,
                                                              float* __restrict__ out, int m,
                                                              int B, int S) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(B) * m;
  if (idx >= n) return;
  // eight loads in flight at a time, added in split order
  float v = 0.f;
  for (int y0 = 0; y0 < S; y0 += 8) {
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = y0 + j < S ? partials[(y0 + j) * n + idx] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (y0 + j < S) v += p[j];
  }
  out[idx] = -s[idx % m] * v;
}

struct Plan {
  int RT, W, S, nspans;
  size_t b_bytes, p_bytes;
};

Plan plan(int64_t m, int64_t K, int64_t B) {
  Plan p;
  p.RT = kRT;
  p.W = 8;                                   // waves per workgroup (2 per SIMD)
  // an even number of spans (a padding span of zero activations adds nothing)
  const int64_t nwords = (K + 31) / 32;
  p.nspans = static_cast<int>((nwords + 2 * kSpanWords - 1) / (2 * kSpanWords) * 2);
  // as many splits of the lifted dimension as keep one workgroup per CU
  const int64_t groups = (m + 16 * p.RT * p.W - 1) / (16 * p.RT * p.W);
  int64_t S = num_cus() / groups;
  S = S < 1 ? 1 : S;
  S = S > p.nspans / 2 ? p.nspans / 2 : S;
  p.S = static_cast<int>(S);
  // the layer's spans plus two read ahead of the last (never used)
  p.b_bytes = static_cast<size_t>(p.nspans + 2) * kSpanBytes;
  p.p_bytes = static_cast<size_t>(p.S) * B * m * 4;
  return p;
}

}  // namespace

size_t gemv_f4m_workspace_bytes(int64_t m, int64_t K, int64_t B) {
  const Plan p = plan(m, K, B);
  return p.b_bytes + p.p_bytes;
}

hipError_t launch_gemv_f4m(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                           const float* a_lift, int64_t B, float* out, void* ws, hipStream_t st) {
  const Plan p = plan(m, K, B);
  uint8_t* bws = static_cast<uint8_t*>(ws);
  float* partials = reinterpret_cast<float*>(bws + p.b_bytes);
  const int prep_threads = (p.nspans + 2) * 4 * 16 * 8;
  hipLaunchKernelGGL(gemv_f4m_prep_kernel, dim3((prep_threads + 255) / 256), dim3(256), 0, st,
                     a_lift, static_cast<int>(B), static_cast<int>(K), p.nspans + 2, bws);
  constexpr int RT = kRT, W = 8;
  const int rows_wg = W * 16 * RT;
  const dim3 grid(static_cast<unsigned>((m + rows_wg - 1) / rows_wg), static_cast<unsigned>(p.S));
  hipLaunchKernelGGL((gemv_f4m_kernel<RT, W>), grid, dim3(64 * W), 0, st, w, static_cast<int>(m),
                     static_cast<int>(ldw), static_cast<int>((K + 31) / 32), bws, p.nspans,
                     static_cast<int>(B), partials);
  const int64_t n = B * m;
  hipLaunchKernelGGL(gemv_f4m_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, st, partials, s, out, static_cast<int>(m), static_cast<int>(B),
                     p.S);
  return hipGetLastError();
}

}  // namespace lq
