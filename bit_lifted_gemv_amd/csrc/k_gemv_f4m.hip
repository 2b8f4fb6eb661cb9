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
// once to the workspace, in the order a lane holds its B operand (per span:
// [step][part][half][lane][16 bytes], then [step][token] exponents).  In the
// main kernel each wave keeps one span's B operands in registers for the
// whole kernel and streams its workgroup's row tiles through them; the
// eight waves of a workgroup hold eight consecutive spans, and their partial
// tiles are added in wave order through LDS.  The lifted dimension is split
// into runs of eight spans (the grid's y) and the rows into groups of row
// tiles (its x); each split writes float32 partial sums to the workspace and
// a reduction kernel adds them in split order and scales by s.
// Deterministic.
#include "f4m_image.h"
#include "lq_internal.h"

#include <type_traits>

namespace lq {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kFar = 0x40000000u;     // past every weight range (<= 2^30 bytes)
using f4m::kSpanWords;
using f4m::kPartBytes;
using f4m::kSpanBytes;

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
  f4m::write_span_parts(x, live, u, n, g, h, ws + static_cast<int64_t>(c) * f4m::kSpanBytes);
}

// Main kernel.  A workgroup of 8 waves owns TW tiles of 16 rows and eight
// consecutive spans (4096 positions); wave w keeps the B operands of span
// 8 y + w (four steps, three parts: 96 registers) for the whole kernel and
// streams the workgroup's tiles through them, T tiles per batch, with the
// weights of the next two batches in flight.  After each batch the eight
// waves' partial tiles go to LDS and are added in wave order (one barrier
// per batch, two LDS buffers) into an LDS stage of the workgroup's sums,
// which is written out once at the end: the loop issues no global stores,
// so its waits on the weight loads stay exact.  Grid: x = row groups of TW
// tiles, y = splits of eight spans.
template <int T>
__global__ void __launch_bounds__(512, 1) gemv_f4m_kernel(
    const uint32_t* __restrict__ w, int m, int ldw, int nw, const uint8_t* __restrict__ bws,
    int TW, int B, float* __restrict__ partials) {
  constexpr int kW = 8;
  static_assert(T == 4, "the sums of a batch: one thread per (tile, lane, row pair)");
  extern __shared__ f32x4 red[];                // [2][kW][T][64], then the stage [16][(TW + 2 T) 16]
  float* stage = reinterpret_cast<float*>(red + 2 * kW * T * 64);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15;
  const int g = lane >> 4;
  const int c = blockIdx.y * kW + wave;         // this wave's span

  // Weights of this workgroup's rows: rows past its last read as zero and
  // are never stored; words past a row's last one, nw, read as zero (they
  // meet zero activations).
  const int NT = (m + 15) / 16;
  const int tile0 = blockIdx.x * TW;
  const int nt = min(TW, NT - tile0);           // tiles of this workgroup (>= 1)
  const int wg_row0 = tile0 * 16;
  const int wg_rows = min(TW * 16, m - wg_row0);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w + static_cast<int64_t>(wg_row0) * ldw), (short)0,
      static_cast<int>(static_cast<uint32_t>(wg_rows) * static_cast<uint32_t>(ldw) * 4u), kRsrcWord3);
  const uint32_t w_lane = c * kSpanWords + 4 * g < nw
      ? static_cast<uint32_t>(i * ldw + c * kSpanWords + 4 * g) * 4u : kFar;
  const uint32_t tile_bytes = static_cast<uint32_t>(16 * ldw) * 4u;
  auto load_w = [&](int j) -> uint4 {           // tile j of the workgroup
    const int so = j < nt ? static_cast<int>(j * tile_bytes) : static_cast<int>(kFar);
    const auto r = __builtin_amdgcn_raw_buffer_load_b128(wres, w_lane, so, 0);
    uint4 v;
    __builtin_memcpy(&v, &r, 16);
    return v;
  };

  const uint32_t two = opaque_v(0x22222222u);
  const int nb = (nt + T - 1) / T;              // batches
  // the first batch's weights go out before the span's operands, so that
  // batch 0 can start on each step's operands as they arrive
  uint4 wv[2][T];
#pragma unroll
  for (int t = 0; t < T; ++t) wv[0][t] = load_w(t);
  __builtin_amdgcn_sched_barrier(0);

  // B operands of the span: [step][part] with both 16-byte halves, and the
  // exponent of column i at each step.
  i32x8 bq[4][3];
  int ex[4];
  {
    const uint8_t* sp = bws + static_cast<int64_t>(c) * kSpanBytes;
    // exponents first, then the operands step by step (the order they are
    // needed in)
#pragma unroll
    for (int u = 0; u < 4; ++u) ex[u] = reinterpret_cast<const int*>(sp + kPartBytes)[u * 16 + i];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const uint4 y0 = *reinterpret_cast<const uint4*>(sp + (((u * 3 + q) * 2) * 64 + lane) * 16);
        const uint4 y1 = *reinterpret_cast<const uint4*>(sp + (((u * 3 + q) * 2 + 1) * 64 + lane) * 16);
        __builtin_memcpy(&bq[u][q], &y0, 16);
        __builtin_memcpy(reinterpret_cast<char*>(&bq[u][q]) + 16, &y1, 16);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < T; ++t) wv[1][t] = load_w(T + t);
  const int st_t = (tid >> 6) & 3;              // tile of the batch
  const int st_h = tid >> 8;                    // rows 2 h, 2 h + 1 of the lane's four
  // The stage holds a batch of rows before the first (where the sums of
  // the batch before batch 0 land) and one after the last, so its writes
  // need no branch.
  const int TR = (TW + 2 * T) * 16;             // stage row stride (per token)

  // The sums of the batch whose partial tiles are in LDS buffer q, in wave
  // order, into the stage rows of batch bb (acc[r] of (tile t, lane) is
  // D[row 4 g + r][token i]).
  auto batch_sums = [&](int q, int bb) {
    const float2* rb2 = reinterpret_cast<const float2*>(red + q * kW * T * 64);
    float2 y[kW];
#pragma unroll
    for (int k = 0; k < kW; ++k) y[k] = rb2[((k * T + st_t) * 64 + lane) * 2 + st_h];
    float2 v = y[0];
#pragma unroll
    for (int k = 1; k < kW; ++k) {
      v.x += y[k].x;
      v.y += y[k].y;
    }
    const int r = ((bb + 1) * T + st_t) * 16 + 4 * g + 2 * st_h;
    *reinterpret_cast<float2*>(stage + i * TR + r) = v;
  };

  // Batch b (b % 2 == P): the sums of batch b - 1 (LDS buffer P ^ 1) are
  // formed while the batch's products run; then the weights are refilled
  // with batch b + 2, the partial tiles go to LDS buffer P, one barrier.
  auto batch = [&](auto P, int b) {
    constexpr int p = decltype(P)::value;
    // the batch's products stay after the previous batch's barrier (they
    // need no memory, so the scheduler would otherwise hoist them and wait
    // for both batches' weights at once)
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t W = u == 0 ? wv[p][t].x : u == 1 ? wv[p][t].y : u == 2 ? wv[p][t].z : wv[p][t].w;
        const i32x8 a = expand_pm(W, two);
#pragma unroll
        for (int q = 0; q < 3; ++q) acc[t] = mfma(a, bq[u][q], acc[t], 127 - ex[u] - 4 * q);
      }
      if (u == 0) batch_sums(p ^ 1, b - 1);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) asm volatile("" : "+v"(acc[t]));
#pragma unroll
    for (int t = 0; t < T; ++t) wv[p][t] = load_w((b + 2) * T + t);
    f32x4* rb = red + p * kW * T * 64;
#pragma unroll
    for (int t = 0; t < T; ++t) rb[(wave * T + t) * 64 + lane] = acc[t];
    __syncthreads();
  };
  // Batch 0 on its own: its products wait for the span's operands step by
  // step as they arrive.  Then the operands are marked as in registers, so
  // that the loops' waits count only weight loads.  With nb even, batch 1
  // is taken on its own too; the rest go in pairs (buffers alternate, so a
  // loop body holds one batch of each parity).
  batch(std::integral_constant<int, 0>{}, 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int q = 0; q < 3; ++q) asm volatile("" : "+v"(bq[u][q]));
    asm volatile("" : "+v"(ex[u]));
  }
  if (nb & 1) {
    int b = 1;
    while (b < nb) {
      batch(std::integral_constant<int, 1>{}, b);
      batch(std::integral_constant<int, 0>{}, b + 1);
      b += 2;
    }
    batch_sums(0, nb - 1);
  } else {
    batch(std::integral_constant<int, 1>{}, 1);
    int b = 2;
    while (b < nb) {
      batch(std::integral_constant<int, 0>{}, b);
      batch(std::integral_constant<int, 1>{}, b + 1);
      b += 2;
    }
    batch_sums(1, nb - 1);
  }
  __syncthreads();

  // this split's partials [B][m], row-contiguous per token: 32 threads a
  // token, four rows a thread (one 16-byte store when m % 4 == 0)
  float* dst = partials + static_cast<int64_t>(blockIdx.y) * B * m + wg_row0;
  const float* src = stage + T * 16;
  const int n = tid >> 5;
  if (n < B) {
    for (int r = (tid & 31) * 4; r < wg_rows; r += 128) {
      const float4 v = *reinterpret_cast<const float4*>(src + n * TR + r);
      float* d = dst + static_cast<int64_t>(n) * m + r;
      if ((m & 3) == 0 && r + 4 <= wg_rows) {
        *reinterpret_cast<float4*>(d) = v;
      } else {
        d[0] = v.x;
        if (r + 1 < wg_rows) d[1] = v.y;
        if (r + 2 < wg_rows) d[2] = v.z;
        if (r + 3 < wg_rows) d[3] = v.w;
      }
    }
  }
}

// out[b][i] = -s[i] * sum over splits of partials[split][b][i], in split
// order, for b < B.
// kChunk: splits in flight at once (the launch picks the smallest power of
// two that covers S, at most 32).
template <int kChunk>
__global__ void __launch_bounds__(256) gemv_f4m_reduce_kernel(const float* __restrict__ partials,
                                                              const float* __restrict__ s,
                                                              float* __restrict__ out, int m,
                                                              int B, int S) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(B) * m;
  if (idx >= n) return;
  // every load of a chunk is issued before the first add: splits past S
  // read the last one again (an address known to be valid, no branch) and
  // are not added
  float v = 0.f;
  for (int y0 = 0; y0 < S; y0 += kChunk) {
    float p[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) p[j] = partials[static_cast<int64_t>(min(y0 + j, S - 1)) * n + idx];
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      if (y0 + j < S) v += p[j];
  }
  out[idx] = -s[idx % m] * v;
}

constexpr int kT = 4;                                 // tiles per batch
constexpr int kSpansWG = 8;                           // spans per workgroup (one per wave)
constexpr int kMaxTW = 84;                            // tiles per workgroup: (84 + 8) KB of sums in LDS

struct Plan {
  int S, TW, groups, nspans;                 // splits, tiles per workgroup, row groups, spans written
  size_t b_bytes, p_bytes, lds;
};

Plan plan(int64_t m, int64_t K, int64_t B) {
  Plan p;
  const int64_t nwords = (K + 31) / 32;
  const int64_t nsp = (nwords + kSpanWords - 1) / kSpanWords;
  p.S = static_cast<int>((nsp + kSpansWG - 1) / kSpansWG);
  // row groups: about one workgroup per CU, whole batches each, and each
  // workgroup's sums within the LDS stage
  const int64_t NT = (m + 15) / 16;
  int64_t G = num_cus() / p.S;
  G = G < 1 ? 1 : G;
  int64_t TW = (NT + G - 1) / G;
  TW = (TW + kT - 1) / kT * kT;
  TW = TW > kMaxTW ? kMaxTW : TW;
  p.TW = static_cast<int>(TW);
  p.groups = static_cast<int>((NT + TW - 1) / TW);
  p.nspans = p.S * kSpansWG;                 // padding spans are zero
  p.b_bytes = static_cast<size_t>(p.nspans) * kSpanBytes;
  p.p_bytes = static_cast<size_t>(p.S) * B * m * 4;
  p.lds = static_cast<size_t>(2) * 8 * kT * 64 * 16 + static_cast<size_t>(16) * (TW + 2 * kT) * 16 * 4;
  return p;
}

}  // namespace

size_t gemv_f4m_workspace_bytes(int64_t m, int64_t K, int64_t B) {
  const Plan p = plan(m, K, B);
  return p.b_bytes + p.p_bytes;
}

namespace {

// The product over the image bws (f4m_image.h) and the split reduction.
hipError_t launch_product(const Plan& p, const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                          const float* s, const uint8_t* bws, int64_t B, float* out,
                          float* partials, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(gemv_f4m_kernel<kT>);
  if (p.lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(p.lds));
    if (e != hipSuccess) return e;
  }
  const dim3 grid(static_cast<unsigned>(p.groups), static_cast<unsigned>(p.S));
  hipLaunchKernelGGL((gemv_f4m_kernel<kT>), grid, dim3(512), p.lds, st, w, static_cast<int>(m),
                     static_cast<int>(ldw), static_cast<int>((K + 31) / 32), bws, p.TW,
                     static_cast<int>(B), partials);
  const int64_t n = B * m;
  const dim3 rgrid(static_cast<unsigned>((n + 255) / 256));
  const int mi = static_cast<int>(m), bi = static_cast<int>(B);
  if (p.S <= 2)
    hipLaunchKernelGGL(gemv_f4m_reduce_kernel<2>, rgrid, dim3(256), 0, st, partials, s, out, mi, bi,
                       p.S);
  else if (p.S <= 4)
    hipLaunchKernelGGL(gemv_f4m_reduce_kernel<4>, rgrid, dim3(256), 0, st, partials, s, out, mi, bi,
                       p.S);
  else if (p.S <= 8)
    hipLaunchKernelGGL(gemv_f4m_reduce_kernel<8>, rgrid, dim3(256), 0, st, partials, s, out, mi, bi,
                       p.S);
  else if (p.S <= 16)
    hipLaunchKernelGGL(gemv_f4m_reduce_kernel<16>, rgrid, dim3(256), 0, st, partials, s, out, mi,
                       bi, p.S);
  else
    hipLaunchKernelGGL(gemv_f4m_reduce_kernel<32>, rgrid, dim3(256), 0, st, partials, s, out, mi,
                       bi, p.S);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_f4m(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                           const float* a_lift, int64_t B, float* out, void* ws, hipStream_t st) {
  const Plan p = plan(m, K, B);
  uint8_t* bws = static_cast<uint8_t*>(ws);
  float* partials = reinterpret_cast<float*>(bws + p.b_bytes);
  const int prep_threads = p.nspans * 4 * 16 * 8;
  hipLaunchKernelGGL(gemv_f4m_prep_kernel, dim3((prep_threads + 255) / 256), dim3(256), 0, st,
                     a_lift, static_cast<int>(B), static_cast<int>(K), p.nspans, bws);
  return launch_product(p, w, m, K, ldw, s, bws, B, out, partials, st);
}

size_t gemv_f4m_parts_workspace_bytes(int64_t m, int64_t K, int64_t B) {
  return plan(m, K, B).p_bytes;
}

hipError_t launch_gemv_f4m_parts(const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                                 const float* s, const void* parts, int64_t B, float* out,
                                 void* ws, hipStream_t st) {
  const Plan p = plan(m, K, B);
  return launch_product(p, w, m, K, ldw, s, static_cast<const uint8_t*>(parts), B, out,
                        static_cast<float*>(ws), st);
}

}  // namespace lq
