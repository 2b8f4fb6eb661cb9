// Activation lift for many tokens on the matrix cores (LiftQuant notes,
// 关键设计 4: the small transform of the activations; 关键设计 1 for the
// per-group M):
//   u[b][128q + r]     = sum_c T_q[r][c] * a[b][128q + c]      (block q of T^-1)
//   a_hat[b][g D + j]  = sum_{r<d} M[r][j] * u[b][g d + r]
//
// With a and T^-1 in the same 16-bit type the first step is a product of
// exact 16-bit operands, so it runs on v_mfma_f32_32x32x16 with float32
// accumulation: per 128-block q it is U_q = A_q T_q^T over 128 positions.
// A workgroup of 4 waves takes one block and 32 tokens; wave w takes
// channels 32 w .. 32 w + 31 (one MFMA tile of 32 x 32, 8 steps of 16
// positions).  Both operands come straight from global memory: lane
// (l, h) of an MFMA reads 8 consecutive 16-bit values of a token row of a, or
// of a row of T_q, which are contiguous in their layouts.  u goes through LDS
// (float32, token-major) to the second step, which runs on the vector ALU:
// a lane takes whole groups of one token (consecutive lanes, consecutive
// groups, so the writes of a_hat are contiguous) and multiplies its d values
// of u by M, read 8 columns at a time as scalars (the same for every lane);
// a last chunk of fewer than 8 columns reads a zero-padded copy in LDS.
// When D % 8 != 0 a lane's run of D values cannot be written as 16-byte
// vectors; then, if the workgroup's slab of a_hat (32 tokens x 128 D / d
// values) fits in LDS beside the rest and its rows are 16-byte aligned, the
// lanes write it there and the workgroup stores it to memory in whole
// 16-byte pieces of consecutive addresses.  Used when 128 % d == 0, so no group straddles two blocks.
#include "lq_internal.h"

namespace lq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTB = 128;                 // transform block
constexpr int kWaves = 4;                // each takes 32 of the block's 128 channels
constexpr int kThreads = 64 * kWaves;
constexpr int kTok = 32;                 // tokens per workgroup
constexpr int kChW = kTB / kWaves;       // channels per wave
constexpr int kUld = kChW + 4;           // floats per token row of a wave's u in LDS
constexpr uint32_t kRsrcWord3 = 0x00020000u;

template <int DT>
__device__ __forceinline__ f32x16 mfma16(const uint4& a, const uint4& b, const f32x16& c);

template <>
__device__ __forceinline__ f32x16 mfma16<LQ_F16>(const uint4& a, const uint4& b, const f32x16& c) {
  half8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma16<LQ_BF16>(const uint4& a, const uint4& b, const f32x16& c) {
  bf8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

template <int O_DT>
__device__ __forceinline__ void store8(void* out, int64_t idx, const float* v, bool vec, int cnt);

template <>
__device__ __forceinline__ void store8<LQ_F32>(void* out, int64_t idx, const float* v, bool vec,
                                               int cnt) {
  float* o = static_cast<float*>(out) + idx;
  if (vec) {
    reinterpret_cast<float4*>(o)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(o)[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < cnt) o[e] = v[e];
  }
}

template <int O_DT>
__device__ __forceinline__ void store8_16(void* out, int64_t idx, const float* v, bool vec,
                                          int cnt) {
  uint16_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    h[e] = O_DT == LQ_F16 ? float_to_f16_bits_rne(v[e]) : float_to_bf16_bits_rne(v[e]);
  uint16_t* o = static_cast<uint16_t*>(out) + idx;
  if (vec) {
    uint4 q;
    q.x = h[0] | (static_cast<uint32_t>(h[1]) << 16);
    q.y = h[2] | (static_cast<uint32_t>(h[3]) << 16);
    q.z = h[4] | (static_cast<uint32_t>(h[5]) << 16);
    q.w = h[6] | (static_cast<uint32_t>(h[7]) << 16);
    *reinterpret_cast<uint4*>(o) = q;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < cnt) o[e] = h[e];
  }
}

template <>
__device__ __forceinline__ void store8<LQ_F16>(void* out, int64_t idx, const float* v, bool vec,
                                               int cnt) {
  store8_16<LQ_F16>(out, idx, v, vec, cnt);
}

template <>
__device__ __forceinline__ void store8<LQ_BF16>(void* out, int64_t idx, const float* v, bool vec,
                                                int cnt) {
  store8_16<LQ_BF16>(out, idx, v, vec, cnt);
}

// Bytes of dynamic LDS before the staged a_hat slab: M as [d][Dpad] floats.
__host__ __device__ constexpr int m_lds_bytes(int d, int D) { return (d * ((D + 7) & ~7) * 4 + 15) & ~15; }

// DT: type of a and T^-1 (LQ_F16 or LQ_BF16); O_DT: type of a_hat; DD = d.
// vec: D % 8 == 0 and out 16-byte aligned (every 8-value run of a_hat then
// starts 16-byte aligned).  staged: the slab goes through LDS (see above).
template <int DT, int O_DT, int DD>
__global__ void __launch_bounds__(kThreads) lift_mfma_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ t_inv,
    const float* __restrict__ M, void* __restrict__ out, int B, int n, int D, int K, bool vec,
    bool staged) {
  __shared__ __attribute__((aligned(16))) float su[kWaves][kTok * kUld];   // 18 KB
  extern __shared__ float4 sM4[];                 // M, [d][Dpad], zero padded; then the slab
  float* sM = reinterpret_cast<float*>(sM4);
  const int Dpad = (D + 7) & ~7;
  constexpr int kOB = O_DT == LQ_F32 ? 4 : 2;     // bytes per a_hat value
  const int per_tok = (kTB / DD) * D;             // a_hat values of this workgroup per token
  char* const slab = reinterpret_cast<char*>(sM4) + m_lds_bytes(DD, D);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int q = blockIdx.x;                 // 128-block
  const int t0 = blockIdx.y * kTok;         // first token
  const int c0 = wave * kChW;               // this wave's first channel in the block

  // ---- step 1: U = A_q T_q^T on MFMA, one 32 x 32 tile per wave (tokens x
  // channels c0 .. c0 + 31) over the block's 128 positions.  Tokens past B
  // read as zero (buffer range of the workgroup's token rows).
  const int toks = min(kTok, B - t0);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a + static_cast<int64_t>(t0) * n), (short)0,
      static_cast<int>(static_cast<uint32_t>(toks) * static_cast<uint32_t>(n) * 2u), kRsrcWord3);
  const uint32_t a_off = (static_cast<uint32_t>(l32) * n + q * kTB + 8 * h) * 2u;
  const uint16_t* trow = t_inv + (static_cast<int64_t>(q) * kTB + c0 + l32) * kTB + 8 * h;
  uint4 af[kTB / 16], bt[kTB / 16];
#pragma unroll
  for (int ks = 0; ks < kTB / 16; ++ks) {
    const auto r = __builtin_amdgcn_raw_buffer_load_b128(ares, a_off + 32u * ks, 0, 0);
    __builtin_memcpy(&af[ks], &r, 16);
    bt[ks] = *reinterpret_cast<const uint4*>(trow + 16 * ks);
  }

  for (int i = threadIdx.x; i < DD * Dpad; i += kThreads) {
    const int r = i / Dpad;
    const int j = i - r * Dpad;
    sM[i] = j < D ? M[r * D + j] : 0.f;
  }

  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int ks = 0; ks < kTB / 16; ++ks) acc = mfma16<DT>(af[ks], bt[ks], acc);
  // D[i][j]: i = token 8 (e / 4) + 4 h + (e % 4), j = channel c0 + l32
  float* u = su[wave];
#pragma unroll
  for (int e = 0; e < 16; ++e) u[(8 * (e >> 2) + 4 * h + (e & 3)) * kUld + l32] = acc[e];
  __syncthreads();

  // ---- step 2: a_hat = M^T u per group, on the vector ALU.  The wave's 32
  // channels hold 32 / d whole groups; a lane takes (token, group) pairs
  // (consecutive lanes, consecutive groups of a token) and the d rows of M
  // kRB at a time; each broadcast read of 8 entries of a row of M feeds 8
  // multiply-adds per pair.
  constexpr int kGw = kChW / DD;                          // groups per wave
  constexpr int kPairs = kTok * kGw;                      // (token, group) pairs per wave
  constexpr int kPC = kPairs >= 64 ? kPairs / 64 : 1;     // pairs per lane
  constexpr int kRB = DD < 8 ? DD : 8;
  int ubase[kPC];
  int64_t obase[kPC];
  int sbase[kPC];
  bool live[kPC];
#pragma unroll
  for (int pc = 0; pc < kPC; ++pc) {
    const int pidx = lane + 64 * pc;
    const int tt = pidx / kGw;
    const int g = pidx - tt * kGw;
    live[pc] = pidx < kPairs && t0 + tt < B;
    ubase[pc] = live[pc] ? tt * kUld + g * DD : 0;
    obase[pc] = static_cast<int64_t>(t0 + tt) * K +
                static_cast<int64_t>(q * (kTB / DD) + wave * kGw + g) * D;
    sbase[pc] = tt * per_tok + (wave * kGw + g) * D;
  }
  // later pairs of a lane are dead when its first is; without the slab no
  // barrier follows
  if (!live[0] && !staged) return;
  // Whole chunks of 8 columns read M from global memory at addresses that are
  // the same for every lane (scalar loads, an SGPR operand per multiply-add);
  // a last chunk of fewer than 8 columns reads the zero-padded copy in LDS.
  const int Dfull = D & ~7;
#pragma unroll 1
  for (int j0 = 0; j0 < D; j0 += 8) {
    const bool full = j0 < Dfull;
    float o[kPC][8];
#pragma unroll
    for (int pc = 0; pc < kPC; ++pc)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[pc][e] = 0.f;
#pragma unroll 1
    for (int r0 = 0; r0 < DD; r0 += kRB) {
      float uv[kPC][kRB];
#pragma unroll
      for (int pc = 0; pc < kPC; ++pc)
#pragma unroll
        for (int r = 0; r < kRB; ++r) uv[pc][r] = u[ubase[pc] + r0 + r];
      if (full) {
#pragma unroll
        for (int r = 0; r < kRB; ++r) {
          const float* mr = M + (r0 + r) * D + j0;
#pragma unroll
          for (int pc = 0; pc < kPC; ++pc)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[pc][e] = fmaf(mr[e], uv[pc][r], o[pc][e]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < kRB; ++r) {
          const float4 m0 = sM4[((r0 + r) * Dpad + j0) / 4];
          const float4 m1 = sM4[((r0 + r) * Dpad + j0) / 4 + 1];
          const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
          for (int pc = 0; pc < kPC; ++pc)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[pc][e] = fmaf(mv[e], uv[pc][r], o[pc][e]);
        }
      }
    }
#pragma unroll
    for (int pc = 0; pc < kPC; ++pc) {
      if (!live[pc]) continue;
      if (staged)
        store8<O_DT>(slab, sbase[pc] + j0, o[pc], vec, D - j0);
      else
        store8<O_DT>(out, obase[pc] + j0, o[pc], vec, D - j0);
    }
  }
  if (staged) {
    // the slab, row by row (token rows of per_tok values), in 16-byte pieces
    __syncthreads();
    const int rows = min(kTok, B - t0);
    const int cpr = per_tok * kOB / 16;
    char* const gbase = static_cast<char*>(out) +
                        (static_cast<int64_t>(t0) * K + static_cast<int64_t>(q) * per_tok) * kOB;
    for (int i = threadIdx.x; i < rows * cpr; i += kThreads) {
      const int r = i / cpr;
      const int c = i - r * cpr;
      const uint4 v = *reinterpret_cast<const uint4*>(slab + (r * per_tok) * kOB + 16 * c);
      *reinterpret_cast<uint4*>(gbase + static_cast<int64_t>(r) * K * kOB + 16 * c) = v;
    }
  }
}

template <int DT, int O_DT, int DD>
hipError_t launch_dd(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M,
                     int D, void* out, hipStream_t st) {
  const int K = static_cast<int>(n / DD * D);
  const dim3 grid(static_cast<unsigned>(n / kTB), static_cast<unsigned>((B + kTok - 1) / kTok));
  // The slab goes through LDS when the lanes' own runs cannot be written as
  // 16-byte vectors (D % 8 != 0: value-by-value stores), the slab's rows and
  // their places in a_hat are 16-byte aligned, and everything stays within
  // 64 KB of LDS.  (With 16-byte runs the direct stores measured faster: the
  // larger LDS footprint costs more resident workgroups than the partly
  // filled lines cost.)
  const int ob = O_DT == LQ_F32 ? 4 : 2;
  const int64_t per_tok = static_cast<int64_t>(kTB / DD) * D;
  const bool aligned16 = reinterpret_cast<uintptr_t>(out) % 16 == 0;
  const size_t static_lds = sizeof(float) * kWaves * kTok * kUld;
  const size_t slab_bytes = static_cast<size_t>(kTok * per_tok * ob);
  const bool staged = D % 8 != 0 && aligned16 && (per_tok * ob) % 16 == 0 &&
                      (int64_t{K} * ob) % 16 == 0 &&
                      static_lds + m_lds_bytes(DD, D) + slab_bytes <= 65536;
  const size_t lds = m_lds_bytes(DD, D) + (staged ? slab_bytes : 0);
  // within the slab a lane's 8-value runs are 16-byte aligned when D % 8 == 0
  hipLaunchKernelGGL((lift_mfma_kernel<DT, O_DT, DD>), grid, dim3(kThreads), lds, st,
                     static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(t_inv), M, out,
                     static_cast<int>(B), static_cast<int>(n), D, K,
                     D % 8 == 0 && (staged || aligned16), staged);
  return hipGetLastError();
}

template <int DT, int O_DT>
hipError_t launch_o(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M, int d,
                    int D, void* out, hipStream_t st) {
  switch (d) {
    case 4: return launch_dd<DT, O_DT, 4>(a, B, n, t_inv, M, D, out, st);
    case 8: return launch_dd<DT, O_DT, 8>(a, B, n, t_inv, M, D, out, st);
    case 16: return launch_dd<DT, O_DT, 16>(a, B, n, t_inv, M, D, out, st);
    default: return launch_dd<DT, O_DT, 32>(a, B, n, t_inv, M, D, out, st);
  }
}

template <int DT>
hipError_t launch_t(const void* a, int64_t B, int64_t n, const void* t_inv, const float* M, int d,
                    int D, void* out, lq_dtype out_dt, hipStream_t st) {
  switch (out_dt) {
    case LQ_F32: return launch_o<DT, LQ_F32>(a, B, n, t_inv, M, d, D, out, st);
    case LQ_F16: return launch_o<DT, LQ_F16>(a, B, n, t_inv, M, d, D, out, st);
    default: return launch_o<DT, LQ_BF16>(a, B, n, t_inv, M, d, D, out, st);
  }
}

}  // namespace

bool lift_mfma_applies(lq_dtype a_dt, lq_dtype t_dt, int64_t B, int64_t n, int d, int D) {
  const bool enough = B >= 8 || (B >= 4 && n >= 12288);
  return enough && a_dt == t_dt && (a_dt == LQ_F16 || a_dt == LQ_BF16) &&
         (d == 4 || d == 8 || d == 16 || d == 32) && D <= 256 &&
         static_cast<int64_t>(kTok) * n * 2 < (int64_t{1} << 31);
}

hipError_t launch_lift_mfma(const void* a, lq_dtype dt, int64_t B, int64_t n, const void* t_inv,
                            const float* M, int d, int D, void* out, lq_dtype out_dt,
                            hipStream_t st) {
  if (dt == LQ_F16) return launch_t<LQ_F16>(a, B, n, t_inv, M, d, D, out, out_dt, st);
  return launch_t<LQ_BF16>(a, B, n, t_inv, M, d, D, out, out_dt, st);
}

}  // namespace lq
