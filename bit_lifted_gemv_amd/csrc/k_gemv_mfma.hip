// Product of 1-bit weights with float lifted activations for a few tokens
// (1 <= B <= 16) on the matrix cores:
//   out[b][i] = s[i] * sum_k sigma_ik * a_hat[b][k],  sigma = 2*bit - 1
// (LiftQuant notes, 关键设计 4: after the activation transform the layer is a
// product of 1-bit weights with floats, scaled per row by s).
//
// Operands.  Each float32 a_hat value is split into two bfloat16 parts,
// hi = bf16(x) and lo = bf16(x - hi) (16 significant bits together, a
// relative error below 2^-17), and each token takes two columns of the
// v_mfma_f32_16x16x32_bf16 B operand: hi in column t, lo in column t + 8, so
// one 16-column tile holds 8 tokens (NB = 1 tile for B <= 8, 2 for B <= 16).
// The sign bits become exact bfloat16 +-1 values of the A operand.  The two
// columns of a token are added after the contraction; accumulation is
// float32 throughout.
//
// Position order.  The weights come in spans of 16 words (512 lifted
// positions); lane (i, g) of a tile loads words 4 g .. 4 g + 3 of the span
// of row i (16 bytes, so one load covers 64 contiguous bytes of each row).
// The span is contracted in 16 MFMAs; MFMA 4 u + v takes from lane group g
// bits 4 v + e (low half of dword e) and 4 v + e + 16 (high half) of its word
// u.  The activation parts are laid out in the same order, so each lane's
// 8 sign values are four dwords
//   d_e = ((W << (15 - 4 v - e)) & 0x80008000) | ONE_ONE
// (a set bit sets the sign, so the tile holds -sigma and the epilogue
// multiplies by -s): two vector operations per pair of weights, shifts by
// constants, no byte shuffling and no exchange between lanes.
//
// Kernels.  A small preparation kernel writes the bfloat16 parts once, in
// the order the MFMA B operand is read (per word-block and tile, 64 lanes x
// 16 bytes), to the workspace.  The main kernel gives each wave RT tiles of
// 16 rows; a workgroup of 8 waves (two per SIMD) shares the
// activation parts
// of 16 word-blocks at a time in LDS (double-buffered; each chunk is loaded
// into registers two chunks ahead and written to LDS one chunk ahead) and
// streams its weights from HBM, 16 bytes (4 words) per lane, tile and span,
// two chunks ahead in a register ring.  When
// the lifted dimension is split over S workgroups (so that enough waves run
// for short, wide layers), each split writes float32 partial sums to the
// workspace and a reduction kernel adds them in split order; otherwise the
// scaled sums go straight to the output.  Every result is deterministic.
#include "lq_internal.h"

#include <type_traits>

namespace lq {
namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOneOne = 0x3F803F80u;  // bfloat16 (+1, +1)
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kFar = 0x40000000u;     // past every weight range (<= 2^30 bytes)

// Values the compiler cannot fold (no instruction is emitted for them): a
// scalar, and a per-lane value (kept in a vector register).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// (x & mask) | one for a mask that `one` does not touch, written as a
// bitfield insert so that it is one v_bfi_b32 that the compiler schedules
// (and spaces from the MFMA that reads it) like any other instruction.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t one) {
  return (x & mask) | (one & ~mask);
}

__device__ __forceinline__ f32x4 mfma(const uint4& a, const uint4& b, const f32x4& c) {
  bf8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// The bfloat16 part `lo_part` (0: hi, 1: lo) of x.
__device__ __forceinline__ uint32_t split_part(float x, int lo_part) {
  const uint32_t hi = bf16_rne(x);
  return lo_part ? bf16_rne(x - __uint_as_float(hi << 16)) : hi;
}

// Preparation: bws[(blk * NB + nb) * 64 + l] for MFMA step blk, tile nb,
// lane l = 16 g + j; column j holds token 8 nb + (j & 7), part j >> 3.  Step
// blk = 16 S + 4 u + v takes, from lane group g, bits 4 v + e (low half of
// dword e) and 4 v + e + 16 (high half) of word 16 S + 4 g + u.  Positions
// >= K and tokens >= B are zero.
__global__ void __launch_bounds__(256) gemv_mfma_prep_kernel(const float* __restrict__ ah, int B,
                                                             int K, int NB, int nblk,
                                                             uint4* __restrict__ bws) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nblk * NB * 64) return;
  const int l = idx & 63;
  const int nb = (idx >> 6) % NB;
  const int blk = (idx >> 6) / NB;
  const int j = l & 15;
  const int g = l >> 4;
  const int t = nb * 8 + (j & 7);
  const int part = j >> 3;
  const int word = 16 * (blk >> 4) + 4 * g + ((blk >> 2) & 3);
  const int k0 = word * 32 + 4 * (blk & 3);    // K % 4 == 0: a 4-group is all in or all out
  float4 lo4 = make_float4(0.f, 0.f, 0.f, 0.f), hi4 = lo4;
  if (t < B) {
    const float* row = ah + static_cast<int64_t>(t) * K;
    if (k0 < K) lo4 = *reinterpret_cast<const float4*>(row + k0);
    if (k0 + 16 < K) hi4 = *reinterpret_cast<const float4*>(row + k0 + 16);
  }
  const float lo[4] = {lo4.x, lo4.y, lo4.z, lo4.w};
  const float hi[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
  uint32_t d[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) d[e] = split_part(lo[e], part) | (split_part(hi[e], part) << 16);
  bws[idx] = make_uint4(d[0], d[1], d[2], d[3]);
}

// RT: 16-row tiles per wave; NB: 16-column tiles (8 tokens each); kCB:
// MFMA steps (32 positions each) per chunk; kW: waves per workgroup.
// Grid: x = row groups of 4 waves, y = splits of the lifted dimension (whole
// chunks each).  partials == nullptr: write s-scaled sums to out.
template <int RT, int NB, int kCB, int kW>
__global__ void __launch_bounds__(64 * kW, 1) gemv_mfma_kernel(
    const uint32_t* __restrict__ w, int m, int ldw, int nw, const float* __restrict__ s,
    const uint4* __restrict__ bws, int B, int nchunks, float* __restrict__ out,
    float* __restrict__ partials) {
  constexpr int kThreads = 64 * kW;
  __shared__ u32x4 sb[2][kCB * NB * 64];     // 2 kCB KB per tile of columns

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i = lane & 15;
  const int g = lane >> 4;
  // this split's chunks: a whole number of chunk pairs (nchunks is even)
  const int S = gridDim.y;
  const int c0 = 2 * (blockIdx.y * (nchunks / 2) / S);
  const int c1 = 2 * ((blockIdx.y + 1) * (nchunks / 2) / S);

  // Weights of this workgroup's rows; rows past m read as zero.  Words past
  // a row's end (the last chunk may reach past ldw) pair with zero
  // activations.  Offsets stay below 2^31 (m * ldw * 4 <= 2^30).
  const int wg_row0 = blockIdx.x * kW * 16 * RT;
  const int wg_rows = min(kW * 16 * RT, m - wg_row0);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w + static_cast<int64_t>(wg_row0) * ldw), (short)0,
      static_cast<int>(static_cast<uint32_t>(wg_rows) * static_cast<uint32_t>(ldw) * 4u), kRsrcWord3);
  uint32_t w_off[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
    w_off[t] = static_cast<uint32_t>((wave * 16 * RT + t * 16 + i) * ldw + 4 * g) * 4u;
  // weights of chunk c, span q (16 words), tile t: lane (i, g) takes words
  // 4 g .. 4 g + 3 of the span of row i, so one load covers 64 contiguous
  // bytes of each of the tile's 16 rows
  // Spans past this split (a scalar choice) or words past the row's last
  // one, nw (a per-lane choice), are not fetched: their offsets fall outside
  // the range (each part is 2^30 or more and the range is at most 2^30
  // bytes, the sum stays below 2^32) and read as zero.
  auto load_w = [&](int c, int q, int t) -> uint4 {
    const int word0 = c * kCB + 16 * q + 4 * g;
    const uint32_t vo = word0 < nw ? w_off[t] : kFar;
    const int so = c < c1 ? (c * kCB + 16 * q) * 4 : static_cast<int>(kFar);
    const auto r = __builtin_amdgcn_raw_buffer_load_b128(wres, vo, so, 0);
    uint4 v;
    __builtin_memcpy(&v, &r, 16);
    return v;
  };
  // activation parts of chunk c: kCB * NB * 64 16-byte vectors, kPer per
  // thread (native vector type, so the staging stays in registers)
  constexpr int kPer = kCB * NB * 64 / kThreads;
  const u32x4* bsrc = reinterpret_cast<const u32x4*>(bws);
  auto load_b = [&](int c, u32x4 (&v)[kPer]) {
    const u32x4* src = bsrc + static_cast<int64_t>(c) * kCB * NB * 64;
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = src[tid + k * kThreads];
  };
  auto store_b = [&](int buf, const u32x4 (&v)[kPer]) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) sb[buf][tid + k * kThreads] = v[k];
  };

  f32x4 acc[RT][NB];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t one = opaque_v(kOneOne);
  const uint32_t sgn = opaque(0x80008000u);

  constexpr int kLook = NB == 1 ? 2 : 1;     // LDS reads ahead, in blocks
  // weight ring: two chunks, wv[parity][span][tile]; activation parts:
  // two chunks in registers, nbv[parity]
  constexpr int kG = kCB / 16;               // spans of 16 words per chunk
  uint4 wv[2][kG][RT];
  u32x4 nbv[2][kPer];
#pragma unroll
  for (int q = 0; q < kG; ++q)
#pragma unroll
    for (int t = 0; t < RT; ++t) wv[0][q][t] = load_w(c0, q, t);
#pragma unroll
  for (int q = 0; q < kG; ++q)
#pragma unroll
    for (int t = 0; t < RT; ++t) wv[1][q][t] = load_w(c0 + 1, q, t);
  load_b(c0, nbv[0]);
  load_b(c0 + 1, nbv[1]);
  store_b(0, nbv[0]);
  __syncthreads();

  // One chunk, c % 2 == P (counted from c0): wv[P] holds its weights, LDS
  // buffer P its activation parts, nbv[P ^ 1] the next chunk's parts.  The
  // parts of chunk c + 2 are loaded first (into nbv[P]); each group's weight
  // registers are refilled with chunk c + 2 as soon as the group is done; the
  // next chunk's parts go to the other buffer at the end.
  auto chunk = [&](auto P, int c) {
    constexpr int p = decltype(P)::value;
    load_b(c + 2, nbv[p]);
    // activation fragments of block bb, read kLook blocks ahead
    uint4 bfr[kLook + 1][NB];
    auto read_b = [&](int bb, uint4 (&bf)[NB]) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 v = sb[p][(bb * NB + nb) * 64 + lane];
        bf[nb] = make_uint4(v.x, v.y, v.z, v.w);
      }
    };
#pragma unroll
    for (int x = 0; x < kLook; ++x) read_b(x, bfr[x]);
#pragma unroll
    for (int q = 0; q < kG; ++q) {
      // MFMA 4 u + v of the span: lane group g gives bits 4 v + e and
      // 4 v + e + 16 of its word u (word 4 g + u of the span)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int bb = 16 * q + 4 * u + v;
          if (bb + kLook < kCB) read_b(bb + kLook, bfr[(bb + kLook) % (kLook + 1)]);
          const uint4 (&bf)[NB] = bfr[bb % (kLook + 1)];
#pragma unroll
          for (int t = 0; t < RT; ++t) {
            const uint32_t W = u == 0 ? wv[p][q][t].x : u == 1 ? wv[p][q][t].y
                             : u == 2 ? wv[p][q][t].z : wv[p][q][t].w;
            uint4 a;
            a.x = and_or(W << (15 - 4 * v), sgn, one);
            a.y = and_or(W << (14 - 4 * v), sgn, one);
            a.z = and_or(W << (13 - 4 * v), sgn, one);
            a.w = and_or(W << (12 - 4 * v), sgn, one);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[t][nb] = mfma(a, bf[nb], acc[t][nb]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) wv[p][q][t] = load_w(c + 2, q, t);
    }
    store_b(p ^ 1, nbv[p ^ 1]);
    __syncthreads();
  };
  // Pairs of chunks without branches inside the loop body, so the waits on
  // the loads are the same every turn.  The workspace holds two chunks more
  // than the layer needs, for the activation loads two chunks ahead.
  for (int c = c0; c < c1; c += 2) {
    chunk(std::integral_constant<int, 0>{}, c);
    chunk(std::integral_constant<int, 1>{}, c + 1);
  }

  // Epilogue.  acc[t][nb][e] = D[row 4 g + e][column j = lane & 15] of tile
  // t; column j < 8 is token 8 nb + j's hi part, j + 8 its lo part.
  float* dst = partials ? partials + static_cast<int64_t>(blockIdx.y) * B * m : out;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row0 = wg_row0 + wave * 16 * RT + t * 16 + 4 * g;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int tok = nb * 8 + i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = acc[t][nb][e] + __shfl_xor(acc[t][nb][e], 8);
        const int row = row0 + e;
        if (i < 8 && tok < B && row < m)
          dst[static_cast<int64_t>(tok) * m + row] = partials ? -v : -s[row] * v;
      }
    }
  }
}

// out[b][i] = s[i] * sum over splits of partials[split][b][i], in split order.
__global__ void __launch_bounds__(256) gemv_mfma_reduce_kernel(const float* __restrict__ partials,
                                                               const float* __restrict__ s,
                                                               float* __restrict__ out, int m,
                                                               int B, int S) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(B) * m;
  if (idx >= n) return;
  float v = 0.f;
  for (int y = 0; y < S; ++y) v += partials[static_cast<int64_t>(y) * n + idx];
  out[idx] = s[idx % m] * v;
}

struct Plan {
  int RT, NB, CB, W, S, nblk, nchunks;
  size_t b_bytes, p_bytes;
};

Plan plan(int64_t m, int64_t K, int64_t B) {
  Plan p;
  p.NB = B <= 8 ? 1 : 2;
  p.RT = 4;                                  // 64 rows per wave
  p.CB = 16;                                 // one span per chunk
  p.W = 8;                                   // waves per workgroup (2 per SIMD)
  const int kCB = p.CB;
  // an even number of chunks (a padding chunk of zero activations, if
  // needed, adds nothing)
  const int64_t nblk = (K + 31) / 32;
  p.nchunks = static_cast<int>((nblk + 2 * kCB - 1) / (2 * kCB) * 2);
  p.nblk = p.nchunks * kCB;
  // as many splits of the lifted dimension as keep every workgroup on a CU
  // of its own (no CU runs two of them, which would double its time)
  const int64_t groups = (m + 16 * p.RT * p.W - 1) / (16 * p.RT * p.W);
  const int64_t cus = num_cus();
  int64_t S = cus / groups;
  S = S < 1 ? 1 : S;
  S = S > p.nchunks / 2 ? p.nchunks / 2 : S;
  p.S = static_cast<int>(S);
  // the layer's chunks plus two read ahead of the last (never used)
  p.b_bytes = (static_cast<size_t>(p.nblk + 2 * kCB) * p.NB * 1024 + 255) / 256 * 256;
  p.p_bytes = p.S > 1 ? static_cast<size_t>(p.S) * B * m * 4 : 0;
  return p;
}

template <int RT, int NB, int CB, int W>
void launch_main(const Plan& p, const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                 const float* s, const uint4* bws, int64_t B, float* out, float* partials,
                 hipStream_t st) {
  const int rows_wg = W * 16 * RT;
  const dim3 grid(static_cast<unsigned>((m + rows_wg - 1) / rows_wg), static_cast<unsigned>(p.S));
  hipLaunchKernelGGL((gemv_mfma_kernel<RT, NB, CB, W>), grid, dim3(64 * W), 0, st, w,
                     static_cast<int>(m), static_cast<int>(ldw), static_cast<int>((K + 31) / 32),
                     s, bws, static_cast<int>(B), p.nchunks, out, partials);
}

}  // namespace

size_t gemv_mfma_workspace_bytes(int64_t m, int64_t K, int64_t B) {
  const Plan p = plan(m, K, B);
  return p.b_bytes + p.p_bytes;
}

hipError_t launch_gemv_mfma(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                            const float* a_lift, int64_t B, float* out, void* ws,
                            hipStream_t st) {
  const Plan p = plan(m, K, B);
  uint4* bws = static_cast<uint4*>(ws);
  float* partials = p.S > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.b_bytes) : nullptr;
  const int prep_threads = p.nblk * p.NB * 64;
  hipLaunchKernelGGL(gemv_mfma_prep_kernel, dim3((prep_threads + 255) / 256), dim3(256), 0, st,
                     a_lift, static_cast<int>(B), static_cast<int>(K), p.NB, p.nblk, bws);
  if (p.NB == 1)
    launch_main<4, 1, 16, 8>(p, w, m, K, ldw, s, bws, B, out, partials, st);
  else
    launch_main<4, 2, 16, 8>(p, w, m, K, ldw, s, bws, B, out, partials, st);
  if (p.S > 1) {
    const int64_t n = B * m;
    hipLaunchKernelGGL(gemv_mfma_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, st, partials, s, out, static_cast<int>(m),
                       static_cast<int>(B), p.S);
  }
  return hipGetLastError();
}

}  // namespace lq
