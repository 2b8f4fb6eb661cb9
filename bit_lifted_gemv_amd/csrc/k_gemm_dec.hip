// Decode-weights product for large batches: instead of contracting the 1-bit
// signs with the lifted activations over K = n D / d (关键设计 4's lifted
// GEMM), the weights are reconstructed, W_hat[i][g d + c] = sum_j M[c][j]
// sigma_{i, g D + j} (关键设计 1: w = M y), and contracted over n with the
// whitened activations u = T^-1 a:
//   out[b][i] = s_i sum_{k<n} W_hat[i][k] u[b][k].
// The two are the same linear map (y . (M^T x) = (M y) . x); this one costs
// 2 m n B flops for the product plus the reconstruction, against 2 m K B.
//
// One kernel, on the matrix cores (v_mfma_f32_16x16x32_f16), with the decoded
// weights never leaving the compute unit.  A workgroup of 8 waves owns 64
// rows x 256 tokens.  The decoded dimension is cut into tiles of 16 weights
// (tile t: group g = t / NT, weights c = 16 (t % NT) .. + 15 of it, zero past
// d); a k step of the product is two tiles, a stage four tiles.  Per stage:
//   decode: wave w reconstructs rows 16 (w % 4) .. + 15 of tiles 2 (w / 4)
//     and 2 (w / 4) + 1, W_hat^T[c][rows] = sum_kb (-M)[c][32 kb ..]
//     (-sigma)[32 kb ..][rows] (A = -M fragments, zero past d and D; B = the
//     rows' sign bytes expanded to float16 -sigma in registers).  The
//     result lane (row l % 16, q = l / 16) holds weights
//     4 q .. 4 q + 3 of the tile, which is what lane l of the product's A
//     operand holds for its k positions 8 q .. 8 q + 7 when a k step is
//     (tile 2j: 4 q .. + 3, tile 2j + 1: 4 q .. + 3); the two tiles' float16
//     weights go to LDS as one 16-byte run per lane.
//   product: wave (wr, wn) accumulates rows 32 wr .. + 31 x tokens 64 wn ..
//     + 63 (2 x 4 tiles of 16 x 16) from the LDS tiles of the decoded
//     weights and the activations (a row of 64 slots per token: weight c of
//     tile t at 32 (t / 2) + 8 (c / 4) + 4 (t % 2) + c % 4, so that a lane's
//     B operand of a k step is one 16-byte run of its token's row).
// The sign words (through a per-wave LDS window) and the activations of
// stages s + 1 .. s + P are in flight while stage s multiplies; the stage's
// LDS buffers alternate, one barrier per stage.  s_i scales the float32 sums
// in the epilogue.
#include <type_traits>

#include "lq_internal.h"

namespace lq {
namespace {

// f(0), ..., f(N - 1) with compile-time arguments (register arrays indexed by
// them stay in registers).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTM = 64;                     // rows per workgroup
constexpr int kTN = 256;                    // tokens per workgroup
constexpr int kThreads = 2 * kTN;           // a wave per 32 rows x 64 tokens
constexpr int kWavesD = kThreads / 64;
constexpr int kPairs = 8 / kWavesD;         // tile pairs a wave decodes per stage
constexpr int kStageTiles = 4;              // tiles of 16 decoded weights per stage
constexpr uint32_t kNoLoad = 0x80000000u;   // past every buffer range: loads give 0
constexpr uint32_t kRsrcWord3 = 0x00020000u;
// LDS in 16-byte units: sA [2 buf][2 k steps][4 row tiles][64 lanes], sB [2
// buf][256 tokens][kRowPitch halves], the per-wave sign windows [8][16
// rows][SP words] (SP odd), then the -M fragments.
constexpr int kRowPitch = 72;               // halves per token row: 64 slots + pad
constexpr int kAUnits = 2 * 4 * 64;
constexpr int kBUnits = kTN * kRowPitch * 2 / 16;
constexpr int kSA = 0;
constexpr int kSB = 2 * kAUnits;
constexpr int kSG = kSB + 2 * kBUnits;
// sign words per row and stage held in the window: the stage's GS groups of
// D <= 32 KB bits from an arbitrary bit offset
constexpr int sign_words(int NT, int KB) { return (kStageTiles / NT) * KB + 2; }
// every lane writes its words unconditionally: the window holds 4 SL words
constexpr int sign_loads(int NT, int KB) { return (sign_words(NT, KB) + 3) / 4; }
constexpr int sign_pitch(int NT, int KB) { return (4 * sign_loads(NT, KB)) | 1; }
constexpr int mf_unit(int NT, int KB) { return kSG + (8 * 16 * sign_pitch(NT, KB) + 3) / 4; }

// The low byte of `byte` -> 8 float16 values -sigma (bit i -> value i; 1:
// -1, 0: +1): one byte permute, then per pair a packed 16-bit shift that puts
// the two bits at the sign positions and a bit select against +1.0.
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ f16x8 expand_signs(uint32_t byte, uint32_t sgn, uint32_t one) {
  const uint32_t rep = __builtin_amdgcn_perm(0u, byte, 0x0C000C00u);   // [x, 0, x, 0]
  us2 r;
  __builtin_memcpy(&r, &rep, 4);
  uint32_t d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const us2 sh = {static_cast<unsigned short>(15 - 2 * p),
                    static_cast<unsigned short>(14 - 2 * p)};
    const us2 h = r << sh;
    uint32_t hv;
    __builtin_memcpy(&hv, &h, 4);
    d[p] = (hv & sgn) | (one & ~sgn);
  }
  f16x8 y;
  __builtin_memcpy(&y, d, 16);
  return y;
}

__device__ __forceinline__ f32x4 mfma(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &ha, 2);
  __builtin_memcpy(&ub, &hb, 2);
  return ua | (static_cast<uint32_t>(ub) << 16);
}

// NT = ceil(d / 16) tiles per group (1, 2 or 4), KB = ceil(D / 32) blocks of
// 32 signs (1, 2, 4 or 8; fragments past d and D are zero).  VEC: d % 4 == 0
// and u rows 8-byte aligned, so four consecutive activations load as one.
template <int NT, int KB, bool VEC>
__global__ void __launch_bounds__(kThreads, 512 / kThreads) gemm_dec_kernel(
    const uint32_t* __restrict__ w, int m, int n, int ldw, const float* __restrict__ M, int d,
    int D, const float* __restrict__ s, const uint16_t* __restrict__ u, int B,
    float* __restrict__ out, int tiles_m, int tiles_n) {
  constexpr int GS = kStageTiles / NT;          // groups per stage
  constexpr int SW = sign_words(NT, KB);
  constexpr int SP = sign_pitch(NT, KB);
  constexpr int SL = sign_loads(NT, KB);        // window words loaded per lane and stage
  constexpr int kMF = mf_unit(NT, KB);
  constexpr bool kMfragRegs = KB * NT <= (VEC ? 8 : 4);
  // stages of sign words and activations in flight in registers
  constexpr int P = KB * NT <= 2 ? 4 : 2;
  extern __shared__ uint4 lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 1, wn = wave >> 1;     // product: 32 rows x 64 tokens
  const int drt = wave & 3;                     // decode: row tile,
  const int dtp0 = (wave >> 2) * kPairs;        // first tile pair
  const int q = lane >> 4;
  const int l16 = lane & 15;

  // -M fragments: lane (c = 16 nt + l % 16, j = 32 kb + 8 (l / 16) + 0..7)
  for (int e = tid; e < KB * NT * 64; e += kThreads) {
    const int l = e & 63;
    const int f = e >> 6;                       // kb * NT + nt
    const int kb = f / NT;
    const int nt = f - kb * NT;
    const int c = 16 * nt + (l & 15);
    uint32_t v[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int j = 32 * kb + 8 * (l >> 4) + 2 * h;
      const float x0 = (c < d && j < D) ? -M[c * D + j] : 0.f;
      const float x1 = (c < d && j + 1 < D) ? -M[c * D + j + 1] : 0.f;
      v[h] = pack_f16(x0, x1);
    }
    lds[kMF + e] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  // Workgroup wg runs on XCD wg % 8; XCD x takes the tiles [x per_x, (x + 1)
  // per_x) in token-tile-major order, so that its workgroups share a token
  // tile's activations in that XCD's L2.
  const int per_x = (tiles_m * tiles_n + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_x + (blockIdx.x >> 3);
  if (lin >= tiles_m * tiles_n) return;         // before any barrier: the whole workgroup
  const int tn = lin / tiles_m;
  const int tm = lin - tn * tiles_m;
  const int row0 = tm * kTM;
  const int tok0 = tn * kTN;
  const int rows = min(kTM, m - row0);
  const int toks = min(kTN, B - tok0);
  const int G = n / d;                          // groups per row
  const int T = G * NT;                         // tiles
  const int stages = (T + kStageTiles - 1) / kStageTiles;

  // signs: rows row0 .. row0 + rows - 1; a past-the-end word reads as zero
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w + static_cast<int64_t>(row0) * ldw), (short)0,
      static_cast<int>(static_cast<uint32_t>(rows) * static_cast<uint32_t>(ldw) * 4u),
      kRsrcWord3);
  // activations: tokens tok0 .. tok0 + toks - 1
  const __amdgpu_buffer_rsrc_t ures = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(u + static_cast<int64_t>(tok0) * n), (short)0,
      static_cast<int>(static_cast<uint32_t>(toks) * static_cast<uint32_t>(n) * 2u), kRsrcWord3);

  // -- sign window of the wave: its 16 rows x the SW words from the stage's
  // first group's first bit (word (g0 D) >> 5); lane (row l % 16, q) loads
  // words q, q + 4, ...
  uint32_t* const swin = reinterpret_cast<uint32_t*>(&lds[kSG]) + wave * 16 * SP;
  uint32_t sreg[P][SL];
  auto load_signs = [&](auto pc, int st) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    const uint32_t wb = static_cast<uint32_t>((static_cast<int64_t>(st) * GS * D) >> 5);
    const uint32_t ro = static_cast<uint32_t>(16 * drt + l16) * static_cast<uint32_t>(ldw);
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const int j = q + 4 * i;
      const uint32_t off = (j < SW && st * GS < G) ? (ro + wb + j) * 4u : kNoLoad;
      sreg[p][i] = __builtin_amdgcn_raw_buffer_load_b32(wres, off, 0, 0);
    }
  };
  auto store_signs = [&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
#pragma unroll
    for (int i = 0; i < SL; ++i) swin[l16 * SP + q + 4 * i] = sreg[p][i];
  };

  // -- activations: kTN tokens x 4 tiles x 4 lane groups of 4 values per
  // stage, 8 units per thread (unit i * kThreads + tid: lane group unit % 4, tile
  // (unit / 4) % 4, token unit / 16: 16 consecutive threads cover a token's
  // run of the stage, and write it to consecutive LDS slots)
  u32x2 av[P][8];
  auto load_acts = [&](auto pc, int st) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int un = i * kThreads + tid;
      const int kq = un & 3;
      const int tl = (un >> 2) & 3;
      const int tok = un >> 4;
      const int t = st * kStageTiles + tl;
      const int g = t / NT;
      const int c0 = 16 * (t - g * NT) + 4 * kq;
      const uint32_t base = static_cast<uint32_t>(tok) * static_cast<uint32_t>(n) +
                            static_cast<uint32_t>(g * d + c0);
      if constexpr (VEC) {
        const uint32_t off = (t < T && c0 < d) ? base * 2u : kNoLoad;
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(ures, off, 0, 0);
        __builtin_memcpy(&av[p][i], &v, 8);
      } else {
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off = (t < T && c0 + e < d) ? (base + e) * 2u : kNoLoad;
          h[e] = __builtin_amdgcn_raw_buffer_load_b16(ures, off, 0, 0);
        }
        av[p][i][0] = h[0] | (h[1] << 16);
        av[p][i][1] = h[2] | (h[3] << 16);
      }
    }
  };
  auto store_acts = [&](auto pc, int buf) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int un = i * kThreads + tid;
      const int kq = un & 3;
      const int tl = (un >> 2) & 3;
      const int tok = un >> 4;
      char* row = reinterpret_cast<char*>(&lds[kSB + buf * kBUnits]) + tok * (2 * kRowPitch);
      *reinterpret_cast<u32x2*>(row + 2 * (32 * (tl >> 1) + 8 * kq + 4 * (tl & 1))) = av[p][i];
    }
  };

  __syncthreads();                              // the -M fragments
  const uint32_t sgn = opaque(0x80008000u);
  const uint32_t one = opaque_v(0x3C003C00u);
  f16x8 mreg[kMfragRegs ? KB : 1][kMfragRegs ? NT : 1];
  if constexpr (kMfragRegs) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        mreg[kb][nt] = __builtin_bit_cast(f16x8, lds[kMF + (kb * NT + nt) * 64 + lane]);
  }
  auto mfrag = [&](int kb, int nt) __attribute__((always_inline)) -> f16x8 {
    if constexpr (kMfragRegs)
      return mreg[kb][nt];
    else
      return __builtin_bit_cast(f16x8, lds[kMF + (kb * NT + nt) * 64 + lane]);
  };

  // -- decode of stage st into buffer buf: row tile drt, tile pairs dtp0 ..
  // dtp0 + kPairs - 1 (pair j: tiles 2 j and 2 j + 1, k step j).  First the
  // 32-sign windows from the stage's sign window in LDS, then the products.
  auto decode_words = [&](int st, uint32_t (&win)[kPairs][2][KB]) __attribute__((always_inline)) {
    const int bsh = static_cast<int>((static_cast<int64_t>(st) * GS * D) & 31);
    const uint32_t* srow = swin + l16 * SP;
#pragma unroll
    for (int pr = 0; pr < kPairs; ++pr)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int gi = (2 * (dtp0 + pr) + h) / NT;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int ob = bsh + gi * D + 32 * kb;  // bit offset in the window
          win[pr][h][kb] = __builtin_amdgcn_alignbit(srow[(ob >> 5) + 1], srow[ob >> 5],
                                                     static_cast<uint32_t>(ob & 31));
        }
      }
  };
  auto decode_mfma = [&](const uint32_t (&win)[kPairs][2][KB], int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int pr = 0; pr < kPairs; ++pr) {
      const int dtp = dtp0 + pr;
      uint32_t v[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tl = 2 * dtp + h;
        const int nt = tl - (tl / NT) * NT;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          acc = mfma(mfrag(kb, nt), expand_signs((win[pr][h][kb] >> (8 * q)) & 0xFFu, sgn, one),
                     acc);
        v[2 * h] = pack_f16(acc[0], acc[1]);
        v[2 * h + 1] = pack_f16(acc[2], acc[3]);
      }
      lds[kSA + buf * kAUnits + (dtp * 4 + drt) * 64 + lane] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage st's sign words and activations sit in register slot st % P from P
  // stages ahead; every slot is refilled (loads past the end read zeros) as
  // soon as it is consumed, so each step issues the same loads and the waits
  // are for the oldest ones only.
  using Z = std::integral_constant<int, 0>;
  static_for<P>([&](auto pc) __attribute__((always_inline)) {
    load_signs(pc, decltype(pc)::value);
    load_acts(pc, decltype(pc)::value);
  });
  store_signs(Z{});
  {
    uint32_t win[kPairs][2][KB];
    decode_words(0, win);
    decode_mfma(win, 0);
  }
  store_acts(Z{}, 0);
  load_signs(Z{}, P);
  load_acts(Z{}, P);
  __syncthreads();

  // whole turns of the ring (stages past the last multiply zeros), so that
  // every step issues its loads and the waits stay exact across the loop
  for (int st0 = 0; st0 < stages; st0 += P) {
    static_for<P>([&](auto pc) __attribute__((always_inline)) {
      constexpr int p = decltype(pc)::value;
      constexpr int buf = p & 1;                // st0 % P == 0 and P is even
      constexpr int nx = (p + 1) % P;           // slot of stage st + 1
      const int st = st0 + p;
      // stage st + 1's activations and sign window into LDS and the decode's
      // sign words read back ahead of stage st's product, so that their LDS
      // latency hides under its MFMAs (past the last stage: zeros, never read)
      store_acts(std::integral_constant<int, nx>{}, buf ^ 1);
      store_signs(std::integral_constant<int, nx>{});
      uint32_t win[kPairs][2][KB];
      decode_words(st + 1, win);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f16x8 af[2], bf[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = __builtin_bit_cast(f16x8, lds[kSA + buf * kAUnits + (ks * 4 + 2 * wr + i) * 64 + lane]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const char* row = reinterpret_cast<const char*>(&lds[kSB + buf * kBUnits]) +
                            (64 * wn + 16 * j + l16) * (2 * kRowPitch) + 2 * (32 * ks + 8 * q);
          bf[j] = *reinterpret_cast<const f16x8*>(row);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma(af[i], bf[j], acc[i][j]);
      }
      decode_mfma(win, buf ^ 1);
      // the slot takes stage st + 1 + P
      load_signs(std::integral_constant<int, nx>{}, st + 1 + P);
      load_acts(std::integral_constant<int, nx>{}, st + 1 + P);
      __syncthreads();
    });
  }

  // Epilogue: lane holds token 16 j + l % 16 and rows 16 i + 4 q .. + 3 of
  // the wave's 32 x 64 block.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = 64 * wn + 16 * j + l16;
    if (tok >= toks) continue;
    float* orow = out + static_cast<int64_t>(tok0 + tok) * m;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = row0 + 32 * wr + 16 * i + 4 * q;
      if (r + 3 < m && (m & 3) == 0) {
        const float4 sv = *reinterpret_cast<const float4*>(s + r);
        *reinterpret_cast<float4*>(orow + r) =
            make_float4(sv.x * acc[i][j][0], sv.y * acc[i][j][1], sv.z * acc[i][j][2],
                        sv.w * acc[i][j][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (r + e < m) orow[r + e] = s[r + e] * acc[i][j][e];
      }
    }
  }
}

template <int NT, int KB>
hipError_t launch_nk(const uint32_t* w, int64_t m, int64_t n, int64_t ldw, const float* M, int d,
                     int D, const float* s, const uint16_t* u, int64_t B, float* out,
                     hipStream_t st) {
  const int tiles_m = static_cast<int>((m + kTM - 1) / kTM);
  const int tiles_n = static_cast<int>((B + kTN - 1) / kTN);
  const int per_x = (tiles_m * tiles_n + 7) / 8;
  const size_t lds = (static_cast<size_t>(mf_unit(NT, KB)) + KB * NT * 64) * 16;
  const bool vec = d % 4 == 0 && n % 4 == 0 && reinterpret_cast<uintptr_t>(u) % 8 == 0;
  auto go = [&](auto kern) -> hipError_t {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(8 * per_x)), dim3(kThreads), lds, st, w,
                       static_cast<int>(m), static_cast<int>(n), static_cast<int>(ldw), M, d, D,
                       s, u, static_cast<int>(B), out, tiles_m, tiles_n);
    return hipGetLastError();
  };
  return vec ? go(gemm_dec_kernel<NT, KB, true>) : go(gemm_dec_kernel<NT, KB, false>);
}

template <int NT>
hipError_t launch_n(const uint32_t* w, int64_t m, int64_t n, int64_t ldw, const float* M, int d,
                    int D, const float* s, const uint16_t* u, int64_t B, float* out,
                    hipStream_t st) {
  const int kb = (D + 31) / 32;
  if (kb <= 1) return launch_nk<NT, 1>(w, m, n, ldw, M, d, D, s, u, B, out, st);
  if (kb <= 2) return launch_nk<NT, 2>(w, m, n, ldw, M, d, D, s, u, B, out, st);
  if (kb <= 4) return launch_nk<NT, 4>(w, m, n, ldw, M, d, D, s, u, B, out, st);
  return launch_nk<NT, 8>(w, m, n, ldw, M, d, D, s, u, B, out, st);
}

}  // namespace

bool gemm_decoded_shape_ok(int d, int D) { return d >= 1 && d <= 64 && D >= 1 && D <= 256; }

size_t gemm_decoded_workspace_bytes(int64_t, int64_t) { return 0; }

hipError_t launch_gemm_decoded(const uint32_t* w, int64_t m, int64_t n, int64_t ldw,
                               const float* M, int d, int D, const float* s, const void* u,
                               int64_t B, float* out, void*, hipStream_t st, const char**) {
  const uint16_t* uh = static_cast<const uint16_t*>(u);
  const int nt = (d + 15) / 16;
  if (nt <= 1) return launch_n<1>(w, m, n, ldw, M, d, D, s, uh, B, out, st);
  if (nt <= 2) return launch_n<2>(w, m, n, ldw, M, d, D, s, uh, B, out, st);
  return launch_n<4>(w, m, n, ldw, M, d, D, s, uh, B, out, st);
}

}  // namespace lq
