// Device pieces shared by the table-driven GEMV kernels (k_gemv.hip,
// k_gemv1.hip): the float32 activation-sum table of one 1024-bit slice of the
// lifted dimension, its LDS layout, and the lane reductions.
//
// Table of slice sl: for each byte position p < 128 of the slice and each
// weight-byte value v < 256,
//   E_p[v] = sum_{t<8} (2*bit_t(v) - 1) * a_hat[1024 sl + 8p + t]
// (zero activations past K).  LDS layout (128 KB): entry (slot, v) at byte
// 65536*(slot >> 6) + 256*v + 4*(slot & 63), slot = slot_of(p).  A weight byte
// becomes its entry's address with one v_perm_b32: the byte goes to address
// byte 1, a per-lane constant supplies bytes 0 and 2.
#pragma once

#include "lq_internal.h"

namespace lq {

constexpr int kSliceBits = 1024;
constexpr int kSliceBytes = kSliceBits / 8;    // 128
constexpr int kTableFloats = 128 * 256;        // 128 KB
constexpr uint32_t kNoLoad = 0x80000000u;      // outside every buffer resource: loads give 0,
                                               // stores are dropped

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

// Slot of byte position p (and back: the map is an involution).  Byte b of
// dword d of 16-byte chunk c: p = 16c + 4d + b -> 16c + 4(d ^ (c >> 1)) + b.
// Lanes (row r, chunk c) that read byte (i + r) & 3 of dword d at step i then
// hit 32 different banks per half-wave.
__host__ __device__ constexpr int slot_of(int p) {
  return (p & ~12) | ((((p >> 2) & 3) ^ ((p >> 5) & 3)) << 2);
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

// Table of one slice and token, built by WAVES waves.  Wave w: slot half
// h = w & 1 (slots 64h .. 64h + 63, one per lane), entry block q = w >> 1
// (v in [E*q, E*q + E), E = 512 / WAVES entries), low bits of v visited in
// Gray-code order: one add per entry.  x0, x1: the 8 activations of byte
// position slot_of(64h + lane).
template <int WAVES>
__device__ __forceinline__ void build_table(float* __restrict__ table, const float4& x0,
                                            const float4& x1, int wave, int lane) {
  constexpr int E = 512 / WAVES;                 // entries per lane: 64 or 32
  constexpr int LB = E == 64 ? 6 : 5;            // Gray-coded low bits
  const int h = wave & 1;
  const int q = wave >> 1;
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  float val = 0.f;
#pragma unroll
  for (int t = 0; t < LB; ++t) val -= x[t];
#pragma unroll
  for (int t = LB; t < 8; ++t) val += ((q >> (t - LB)) & 1) ? x[t] : -x[t];
  float tw[LB];
#pragma unroll
  for (int t = 0; t < LB; ++t) tw[t] = 2.f * x[t];
  float* base = table + h * 16384 + (E * q) * 64 + lane;
  base[0] = val;
#pragma unroll
  for (int i = 1; i < E; ++i) {
    const int t = ctz6(i);
    const bool up = (gray(i) >> t) & 1;
    val = up ? val + tw[t] : val - tw[t];
    base[gray(i) * 64] = val;
  }
}

// Per-lane address constants for the lookups of lane (row r, chunk c): at
// step i the lane reads byte b = (i + r) & 3 of each of its 4 dwords d.
struct LaneConsts {
  uint32_t lc[4][4];   // [d][i]: bytes 0 and 2 of the entry address
  uint32_t sel[4];     // [i]: v_perm_b32 selector placing weight byte b at byte 1
};

__device__ __forceinline__ LaneConsts lane_consts(int r, int c) {
  LaneConsts k;
  const int r4 = r & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (i + r4) & 3;
    k.sel[i] = 0u | ((4u + b) << 8) | (2u << 16) | (0x0Cu << 24);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int sl = slot_of(16 * c + 4 * d + static_cast<int>(b));
      k.lc[d][i] = static_cast<uint32_t>(4 * (sl & 63)) | (static_cast<uint32_t>(sl >> 6) << 16);
    }
  }
  return k;
}

// Sum of the table entries of one lane's 16 weight bytes.
__device__ __forceinline__ float lookup16(const char* __restrict__ tb, const uint4& wv,
                                          const LaneConsts& k) {
  const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
  float a[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
    a[d] = *reinterpret_cast<const float*>(tb + __builtin_amdgcn_perm(wd[d], k.lc[d][0], k.sel[0]));
#pragma unroll
  for (int i = 1; i < 4; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d)
      a[d] += *reinterpret_cast<const float*>(tb + __builtin_amdgcn_perm(wd[d], k.lc[d][i],
                                                                         k.sel[i]));
  return (a[0] + a[1]) + (a[2] + a[3]);
}

}  // namespace lq
