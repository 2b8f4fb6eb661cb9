// Operands of the few-token products on v_mfma_scale_f32_16x16x128_f8f6f4
// (LiftQuant notes, 关键设计 4: a product of 1-bit weights with floats),
// shared by the slice-major kernel (k_gemv_f4.hip) and the one-launch kernel
// (k_gemv_f4r.hip).
//
// A (16 rows x 128 lifted positions) holds sign bits as float4 (E2M1):
// dword q of a lane's operand takes bits q, q + 4, ..., q + 28 of a word of
// 32 signs, each left in place inside its nibble, so nibble t (slot 8 q + t)
// is 0 or c_q (0.5, 1, 2 for q = 0, 1, 2; bit 3 moves one place down, so
// c_3 = 2).  B (128 positions x 16 columns) holds the activations of up to
// five tokens as three float8 (E4M3) parts each, in columns 3 b + p, every
// position pre-scaled by 1 / c_q of its slot; a step therefore yields
// R = sum_k bit_k a_k, and with sigma = 2 bit - 1 a slice contributes
// 2 R - sum_k a_k.
//
// Parts of a 1024-position slice: with f the biased exponent of the slice's
// largest |x| and e = 133 - f (at most 118), x 2^e lies in [-128, 128); the
// position's 1 / c_q (at most 2) keeps it below 256, inside float8's range.
// p0 = fp8(y), p1 = fp8(16 (y - p0)), p2 = fp8(16 (y - p0 - p1 / 16) ...)
// (the remainders are exact in float32); column (b, p)'s hardware scale is
// 2^(-e - 4 p), so a token's three columns add up to x with a relative error
// of about 2^-12 of the slice's largest |x| at worst.  Products are exact
// and accumulate in float32.
//
// Position order.  Each slice of a row is 128 bytes; lane (r, G) of a
// 16-row tile loads bytes 16 G .. 16 G + 15 and 64 + 16 G .. 64 + 16 G + 15
// of row r (words 4 G + u and 16 + 4 G + u, u < 4).  MFMA step u < 4 takes
// word 4 G + u from lane group G, step 4 + u word 16 + 4 G + u.  Bit 4 t + q
// of a word sits at A slot 8 q + t, which in the float8 B operand is lane
// group (32 G + 8 q + t) % 64 / 16, byte (8 q + t) % 16 (+ 16 past slot 63);
// a slice's parts are stored [step][column][lane group][32 bytes].
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lq {
namespace f4 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSliceBits = 1024;
constexpr int kSteps = kSliceBits / 128;        // MFMA steps per slice

constexpr int part_bytes(int nb) { return kSteps * 3 * nb * 4 * 32; }   // per slice

// The A operand of one step from a word of sign bits (see above).
__device__ __forceinline__ i32x8 expand(uint32_t w) {
  i32x8 a;
  a[0] = static_cast<int>(w & 0x11111111u);
  a[1] = static_cast<int>(w & 0x22222222u);
  a[2] = static_cast<int>(w & 0x44444444u);
  a[3] = static_cast<int>((w >> 1) & 0x44444444u);
  a[4] = a[5] = a[6] = a[7] = 0;               // unused with a float4 A operand
  return a;
}

__device__ __forceinline__ f32x4 mfma(const i32x8& a, const i32x8& b, const f32x4& c, int sc) {
  // A: E2M1 (cbsz 4), scale 2^0; B: E4M3 (blgp 0), scale 2^(sc - 127)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, 127, 0, sc);
}

template <int CTRL>
__device__ __forceinline__ float dpp_from(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// A slice's sum for the rows of result element c: the token's three part
// columns (lanes 3 b, 3 b + 1, 3 b + 2 of the 16-lane row) added, doubled,
// less the slice's activation sum.
__device__ __forceinline__ float slice_sum(float c, float asum) {
  return fmaf(2.f, c + dpp_from<0x101>(c) + dpp_from<0x102>(c), -asum);
}

// Largest of v over the wave (every lane gets it, in a scalar register).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  const uint32_t a = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
  const uint32_t b = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
  const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
  const uint32_t d = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
  return max(max(a, b), max(c, d));
}

// Sum of v over the wave in a fixed order (every lane gets it).
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Three float8 parts of four values (already scaled), packed in byte order:
// d[p] byte j holds part p of y[j].
__device__ __forceinline__ void split3(float y0a, float y0b, float y0c, float y0d, int d[3]) {
  float y[4] = {y0a, y0b, y0c, y0d};
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    int q = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    q = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], q, true);
    d[p] = q;
    if (p < 2) {
      y[0] = 16.f * (y[0] - __builtin_amdgcn_cvt_f32_fp8(q, 0));
      y[1] = 16.f * (y[1] - __builtin_amdgcn_cvt_f32_fp8(q, 1));
      y[2] = 16.f * (y[2] - __builtin_amdgcn_cvt_f32_fp8(q, 2));
      y[3] = 16.f * (y[3] - __builtin_amdgcn_cvt_f32_fp8(q, 3));
    }
  }
}

// One wave's view of a slice: lane l holds positions 16 l .. 16 l + 15 of
// each token as four float4 vectors.  The largest |x| (as bits, over the
// wave) and the sum of the slice per token.
template <int NB>
__device__ __forceinline__ void slice_stats(const f32x4 (&xv)[NB][4], uint32_t (&mb)[NB],
                                            float (&sum)[NB]) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    uint32_t v = 0;
    float sm = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v = max(v, __float_as_uint(xv[b][c].x) & 0x7FFFFFFFu);
      v = max(v, __float_as_uint(xv[b][c].y) & 0x7FFFFFFFu);
      v = max(v, __float_as_uint(xv[b][c].z) & 0x7FFFFFFFu);
      v = max(v, __float_as_uint(xv[b][c].w) & 0x7FFFFFFFu);
      sm += (xv[b][c].x + xv[b][c].y) + (xv[b][c].z + xv[b][c].w);
    }
    mb[b] = wave_max(v);
    sum[b] = wave_sum(sm);
  }
}

// The slice's scale exponent from its largest |x| (bits): 0 for a zero slice.
__device__ __forceinline__ int slice_exponent(uint32_t mb) {
  return mb == 0 ? 0 : min(133 - static_cast<int>(mb >> 23), 118);
}

// The parts of one wave's slice into dst (the slice's [step][column][lane
// group][32] bytes): per part and per q = position mod 4 a lane writes the
// dword of its positions q, q + 4, q + 8, q + 12 (consecutive slots of one
// B lane).
template <int NB>
__device__ __forceinline__ void slice_parts(const f32x4 (&xv)[NB][4], const int (&e)[NB],
                                            uint8_t* dst, int lane) {
  constexpr int NCOL = 3 * NB;
  const int xw = lane >> 1, xh = lane & 1;      // word of the slice, half of it
  const int xu = xw < 16 ? (xw & 3) : 4 + ((xw - 16) & 3);
  const int xG = xw < 16 ? (xw >> 2) : ((xw - 16) >> 2);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kap = 32 * xG + 8 * q + 4 * xh;
      const int off = (xu * NCOL * 4 + ((kap & 63) >> 4)) * 32 + (kap & 15) + (kap >= 64 ? 16 : 0) +
                      (3 * b) * 128;
      const int eq = e[b] + (q == 0 ? 1 : q == 1 ? 0 : -1);   // 1 / c_q
      int d[3];
      split3(ldexpf(xv[b][0][q], eq), ldexpf(xv[b][1][q], eq), ldexpf(xv[b][2][q], eq),
             ldexpf(xv[b][3][q], eq), d);
      *reinterpret_cast<int*>(dst + off) = d[0];
      *reinterpret_cast<int*>(dst + off + 128) = d[1];
      *reinterpret_cast<int*>(dst + off + 256) = d[2];
    }
  }
}

}  // namespace f4
}  // namespace lq
