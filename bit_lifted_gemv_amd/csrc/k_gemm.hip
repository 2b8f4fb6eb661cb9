// Large-batch product on the matrix cores:
//   out[b][i] = s[i] * sum_k sigma_ik * a_hat[b][k]
// (LiftQuant notes, 关键设计 4: a product of 1-bit weights with floats; with a
// few hundred tokens it is a dense contraction, so it runs on MFMA).
//
// Signs are expanded in registers to exact 16-bit +-1 values (f16 or bf16,
// matching the lifted activations) and fed as the A operand of
// v_mfma_f32_32x32x16; the lifted activations are the B operand, staged
// through LDS.  Accumulation is float32.
//
// Expansion of one weight byte (8 lifted positions of one row: the A operand
// of one lane for one MFMA) into four dwords of two 16-bit values:
//   rep = byte | byte << 16                (v_perm_b32)
//   h   = rep << (15-2p, 14-2p) per half   (v_pk_lshlrev_b16: bit 2p -> bit 15,
//                                           bit 2p+1 -> bit 31)
//   dword_p = (h & 0x80008000) | ONE_ONE   (v_and_or_b32)
// A set bit sets the sign, so the tile holds -sigma; the epilogue multiplies
// by -s.
//
// Tiling: 128 rows x 128 tokens per workgroup of 8 waves.  The lifted
// dimension advances 256 positions per step; wave w takes rows
// 64 (w % 2) .. +63 of the tile against all 128 tokens (2 x 4 MFMA tiles:
// each expanded weight byte feeds four MFMAs, each activation fragment read
// from LDS two) on quarter w / 2 of every step's positions.  The four
// quarters are summed through LDS at the end, where the tile is also
// transposed so that the output rows are written with consecutive lanes on
// consecutive addresses.
//
// The k order inside a quarter-step is permuted the same way for both
// operands: sub-step c (c < 4) gives lane (row or token, h) positions
// 8 (8 kq + 4 h + c) .. +7 of the step, so a lane's weight bits for a whole
// quarter-step are one dword of its row.  Weight dwords are loaded several
// steps ahead into a ring of registers; the activations of the next step
// (128 tokens x 256 positions) are loaded into registers at the start of a
// step and written at its end to the other of two LDS buffers.  Inside a
// step the expansion of sub-step c + 1's weights and the LDS reads of its
// activations are issued between the MFMAs of sub-step c.  All global loads
// are buffer loads whose range check returns zeros for rows, tokens and
// positions past the end, so the loop has no branches.
//
// Workgroups are ordered so that the ones on one XCD (dispatched round-robin
// over 8) take a contiguous run of tiles in token-tile-major order and share
// the token tile's activations in that XCD's L2.
#include "lq_internal.h"

#include <type_traits>

namespace lq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;                 // rows per workgroup
constexpr int kBN = 128;                 // tokens per workgroup
constexpr int kKS = 256;                 // lifted positions per step
constexpr int kThreads = 512;            // 8 waves: 2 row halves x 4 position quarters
constexpr int kRing = 4;                 // steps of weight dwords held in registers
constexpr int kLdsRow = kKS + 8;         // 16-bit elements per LDS token row (528 B)
constexpr int kBufElems = kBN * kLdsRow; // one activation buffer (66 KB)
constexpr int kOutLd = kBM + 4;          // floats per token row of the epilogue tile
constexpr int kBChunks = kBN * kKS / 8 / kThreads;   // 16-byte activation chunks per thread
constexpr uint32_t kNoLoad = 0x80000000u;  // an offset past every buffer's range
constexpr uint32_t kRsrcWord3 = 0x00020000u;

static_assert(kBN * kOutLd * 4 <= 2 * kBufElems * 2, "epilogue tile must fit the LDS buffers");

template <int DT>
struct Mfma;

template <>
struct Mfma<LQ_F16> {
  static constexpr uint32_t kOneOne = 0x3C003C00u;
  __device__ static f32x16 run(const uint4& a, const uint4& b, const f32x16& c) {
    half8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
  }
};

template <>
struct Mfma<LQ_BF16> {
  static constexpr uint32_t kOneOne = 0x3F803F80u;
  __device__ static f32x16 run(const uint4& a, const uint4& b, const f32x16& c) {
    bf8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
  }
};

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

// Byte `byte_idx` of `word` -> 8 16-bit values -sigma (bit 1 -> -1, bit 0 -> +1).
template <int DT>
__device__ __forceinline__ uint4 expand_byte(uint32_t word, int byte_idx, uint32_t sgn,
                                             uint32_t one) {
  const uint32_t selr = static_cast<uint32_t>(byte_idx) | 0x0C000C00u |
                        (static_cast<uint32_t>(byte_idx) << 16);
  const uint32_t rep = __builtin_amdgcn_perm(0u, word, selr);   // [x, 0, x, 0]
  us2 r;
  __builtin_memcpy(&r, &rep, 4);
  uint32_t d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    us2 sh = {static_cast<unsigned short>(15 - 2 * p), static_cast<unsigned short>(14 - 2 * p)};
    const us2 h = r << sh;
    uint32_t hv;
    __builtin_memcpy(&hv, &h, 4);
    d[p] = and_or(hv, sgn, one);
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

template <int DT>
__global__ void __launch_bounds__(kThreads, 1) gemm_mfma_kernel(
    const uint32_t* __restrict__ w, int m, int K, int ldw, const float* __restrict__ s,
    const uint16_t* __restrict__ ah, int B, float* __restrict__ out, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t sB[2 * kBufElems];   // 132 KB

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave & 1;           // 64-row half of the tile
  const int kq = wave >> 1;          // quarter of each step's positions
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Workgroup wg runs on XCD wg % 8; XCD x takes the tiles
  // [x * per_x, (x + 1) * per_x) in token-tile-major order.
  const int wg = blockIdx.x;
  const int per_x = (tiles_m * tiles_n + 7) / 8;
  const int lin = (wg & 7) * per_x + (wg >> 3);
  if (lin >= tiles_m * tiles_n) return;
  const int tn = lin / tiles_m;
  const int tm = lin - tn * tiles_m;
  const int row0 = tm * kBM;
  const int tok0 = tn * kBN;
  const int rows = min(kBM, m - row0);
  const int toks = min(kBN, B - tok0);

  // Weights: rows row0 .. row0 + rows - 1.  Offsets stay below 2^31
  // (ldw <= 2^22): a dword past the row's end pairs with zero activations,
  // rows past m fall outside the range and read as zero.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w + static_cast<int64_t>(row0) * ldw), (short)0,
      static_cast<int>(static_cast<uint32_t>(rows) * static_cast<uint32_t>(ldw) * 4u), kRsrcWord3);
  uint32_t a_off[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
    a_off[mi] = (static_cast<uint32_t>(wr * 64 + mi * 32 + l32) * ldw + 2 * kq + h) * 4u;
  auto load_a = [&](int step, uint32_t (&a)[2]) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      a[mi] = __builtin_amdgcn_raw_buffer_load_b32(wres, a_off[mi], step * (kKS / 8), 0);
  };

  // Activations: tokens tok0 .. tok0 + toks - 1; a step is 128 tokens x 32
  // chunks of 8 positions, kBChunks per thread.  Chunks at positions >= K
  // (K % 8 == 0) take the out-of-range offset; tokens past B fall outside
  // the range.
  const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(ah + static_cast<int64_t>(tok0) * K), (short)0,
      static_cast<int>(static_cast<uint32_t>(toks) * static_cast<uint32_t>(K) * 2u), kRsrcWord3);
  const int b_kk = (tid & 31) * 8;
  const int b_tok = tid >> 5;
  const uint32_t b_off = (static_cast<uint32_t>(b_tok) * K + b_kk) * 2u;
  const uint32_t b_tok_stride = static_cast<uint32_t>(kThreads / 32) * K * 2u;
  // per lane only the range test; the step and the token stride go in the
  // scalar offset (kNoLoad + soffset stays below 2^32 and out of range)
  auto load_b = [&](int step, uint4 (&v)[kBChunks]) {
    const uint32_t vo = step * kKS + b_kk < K ? b_off : kNoLoad;
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const auto r = __builtin_amdgcn_raw_buffer_load_b128(
          bres, vo, static_cast<int>(i * b_tok_stride + static_cast<uint32_t>(step * kKS * 2)), 0);
      __builtin_memcpy(&v[i], &r, 16);
    }
  };
  uint16_t* const b_st = &sB[b_tok * kLdsRow + b_kk];
  auto store_b = [&](int buf, const uint4 (&v)[kBChunks]) {
#pragma unroll
    for (int i = 0; i < kBChunks; ++i)
      *reinterpret_cast<uint4*>(b_st + buf * kBufElems + i * (kThreads / 32) * kLdsRow) = v[i];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < 4; ++nj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][nj][e] = 0.f;

  // LDS element offset of this lane's activation fragment (token block 0,
  // sub-step 0) in buffer 0
  const uint16_t* const b_frag = &sB[l32 * kLdsRow + 8 * (8 * kq + 4 * h)];
  auto read_b = [&](int buf, int c, uint4 (&bf)[4]) {
#pragma unroll
    for (int nj = 0; nj < 4; ++nj)
      bf[nj] = *reinterpret_cast<const uint4*>(b_frag + buf * kBufElems + nj * 32 * kLdsRow + 8 * c);
  };
  const uint32_t one = opaque_v(Mfma<DT>::kOneOne);
  const uint32_t sgn = opaque(0x80008000u);

  const int steps = (K + kKS - 1) / kKS;
  uint32_t a[kRing][2];
  uint4 nb[kBChunks];
#pragma unroll
  for (int r = 0; r < kRing; ++r) load_a(r, a[r]);
  __builtin_amdgcn_sched_barrier(0);
  load_b(0, nb);
  __builtin_amdgcn_sched_barrier(0);
  store_b(0, nb);
  __syncthreads();

  // One step, st % kRing == P: a[P] holds this step's weight dwords, LDS
  // buffer P % 2 its activations.  The scheduling barriers keep the phases in
  // this order: the next step's activation loads first, then per sub-step the
  // MFMAs with the next sub-step's expansion and LDS reads, the weight
  // loads kRing steps ahead right after the last expansion of a[P] (so they
  // land in its registers), the LDS store of the next step's activations last.
  auto step = [&](auto P, int st) {
    constexpr int p = decltype(P)::value;
    constexpr int buf = p & 1;
    load_b(st + 1, nb);
    uint4 bf[4];
    uint4 af[2], afn[2];
    read_b(buf, 0, bf);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) af[mi] = expand_byte<DT>(a[p][mi], 0, sgn, one);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c == 3) {
        load_a(st + kRing, a[p]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c < 3) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) afn[mi] = expand_byte<DT>(a[p][mi], c + 1, sgn, one);
      }
      // token block nj's fragment is reloaded for sub-step c + 1 as soon as
      // its two MFMAs of sub-step c are issued
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) acc[mi][nj] = Mfma<DT>::run(af[mi], bf[nj], acc[mi][nj]);
        if (c < 3)
          bf[nj] = *reinterpret_cast<const uint4*>(b_frag + buf * kBufElems + nj * 32 * kLdsRow +
                                                   8 * (c + 1));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (c < 3) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) af[mi] = afn[mi];
      }
    }
    store_b(buf ^ 1, nb);
    __syncthreads();
  };
  // A whole number of ring turns, without branches inside the loop body: a
  // step past the end reads zero activations and adds nothing.
  for (int st = 0; st < steps; st += kRing) {
    step(std::integral_constant<int, 0>{}, st);
    step(std::integral_constant<int, 1>{}, st + 1);
    step(std::integral_constant<int, 2>{}, st + 2);
    step(std::integral_constant<int, 3>{}, st + 3);
  }

  // Epilogue: D[i][j] of a 32 x 32 MFMA tile, i = row, j = token; lane holds
  // j = l32 and rows 8 (e / 4) + 4 h + (e % 4), e = 0..15.  Quarter 0 writes
  // its sums to the [token][row] tile in LDS, quarters 1..3 add theirs in
  // turn, then every thread scales and stores one row of the output for
  // every fourth token.
  float* tile = reinterpret_cast<float*>(&sB[0]);
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    if (kq == qt) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
          const int tok = nj * 32 + l32;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int row = wr * 64 + mi * 32 + 8 * g + 4 * h;
            float4* dst = reinterpret_cast<float4*>(&tile[tok * kOutLd + row]);
            float4 v = make_float4(acc[mi][nj][4 * g], acc[mi][nj][4 * g + 1],
                                   acc[mi][nj][4 * g + 2], acc[mi][nj][4 * g + 3]);
            if (qt > 0) {
              const float4 o = *dst;
              v.x += o.x;
              v.y += o.y;
              v.z += o.z;
              v.w += o.w;
            }
            *dst = v;
          }
        }
    }
    __syncthreads();
  }
  const int row = tid & (kBM - 1);
  if (row < rows) {
    const float ns = -s[row0 + row];
    float* orow = out + static_cast<int64_t>(tok0) * m + row0 + row;
#pragma unroll 4
    for (int t = tid >> 7; t < toks; t += kThreads / kBM)
      orow[static_cast<int64_t>(t) * m] = ns * tile[t * kOutLd + row];
  }
}

}  // namespace

hipError_t launch_gemm(const uint32_t* w, int64_t m, int64_t K, int64_t ldw, const float* s,
                       const void* a_lift, lq_dtype dt, int64_t B, float* out, hipStream_t st) {
  const int tiles_m = static_cast<int>((m + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((B + kBN - 1) / kBN);
  const int per_x = (tiles_m * tiles_n + 7) / 8;
  const dim3 grid(static_cast<unsigned>(8 * per_x));
  const uint16_t* ah = static_cast<const uint16_t*>(a_lift);
  if (dt == LQ_F16)
    hipLaunchKernelGGL(gemm_mfma_kernel<LQ_F16>, grid, dim3(kThreads), 0, st, w,
                       static_cast<int>(m), static_cast<int>(K), static_cast<int>(ldw), s, ah,
                       static_cast<int>(B), out, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(gemm_mfma_kernel<LQ_BF16>, grid, dim3(kThreads), 0, st, w,
                       static_cast<int>(m), static_cast<int>(K), static_cast<int>(ldw), s, ah,
                       static_cast<int>(B), out, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace lq
