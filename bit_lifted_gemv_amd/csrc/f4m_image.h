// The operand image of the several-token GEMV (k_gemv_f4m.hip): float8
// parts of the lifted activations in the order each lane holds its B
// operand, written either by the GEMV's own preparation kernel from float32
// lifted activations or directly by the parts lift (k_lift_parts.hip).
//
// Per span c of 16 words (512 lifted positions): parts [step u < 4][part p
// < 3][half 2][lane 64][16 bytes], then the exponents [step][token 16] as
// int.  Step u of a span covers words 16 c + 4 g + u (g < 4); per (step,
// token), with f the biased exponent of the largest |x| over those 128
// positions and e = min(134 - f, 119) (0 when all are zero), y = x 2^e lies
// below 256 in magnitude; p0 = fp8(y), p1 = fp8(16 (y - p0)),
// p2 = fp8(16 (y - p0 - p1 / 16)) (E4M3; the remainders are exact in
// float32) and part p's hardware scale is 2^(-e - 4 p).  In the B operand a
// lane group holds slots 16 h' .. 16 h' + 15 of two words: a word's slots 0
// .. 15 go to lane group 2 (g % 2), slots 16 .. 31 to lane group
// 2 (g % 2) + 1, in bytes 16 (g / 2) .. 16 (g / 2) + 15; slot 8 q + t of a
// word is its position 4 t + q.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lq {
namespace f4m {

constexpr int kSpanWords = 16;
constexpr int kSpanPositions = 32 * kSpanWords;
constexpr int kPartBytes = 4 * 3 * 64 * 32;            // per span
constexpr int kSpanBytes = kPartBytes + 4 * 16 * 4;    // parts, then exponents
constexpr int kSpansPerSplit = 8;                      // spans per GEMV workgroup (one per wave)

// Spans of the image for K lifted positions: whole splits of eight, the
// padding spans zero.
inline int64_t image_spans(int64_t K) {
  const int64_t nsp = ((K + 31) / 32 + kSpanWords - 1) / kSpanWords;
  return (nsp + kSpansPerSplit - 1) / kSpansPerSplit * kSpansPerSplit;
}

// Thread (u, n, g, h) of a span (h = bit 0 of the lane, g = bits 1 - 2, so
// the eight threads of a (step, token) are consecutive lanes): x holds the
// 32 values of token n's word 4 g + u of the span.  Shares the (step, token)
// exponent over the eight lanes, then writes the parts of slots 16 h .. 16 h
// + 15 and, from thread (g, h) = (0, 0), the exponent.  Every lane of the
// wave must call it; only `live` ones write.
__device__ __forceinline__ void write_span_parts(const float (&x)[32], bool live, int u, int n,
                                                 int g, int h, uint8_t* span) {
  uint32_t mb = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) mb = max(mb, __float_as_uint(x[j]) & 0x7FFFFFFFu);
  mb = max(mb, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mb), 1)));
  mb = max(mb, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mb), 2)));
  mb = max(mb, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mb), 4)));
  if (!live) return;
  const int e = mb == 0 ? 0 : min(134 - static_cast<int>(mb >> 23), 119);
  // this half's positions 4 t + 2 h + qq, picked with one select each (an
  // index computed from h would make every access a 32-way select chain)
  float xs[2][8];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int t = 0; t < 8; ++t) xs[qq][t] = h ? x[4 * t + 2 + qq] : x[4 * t + qq];
  // dword (q', hh) of this half holds slots 8 q + 4 hh .. + 3 (q = 2 h + q'),
  // i.e. positions 4 t + q for t = 4 hh .. 4 hh + 3
  uint32_t d[3][4];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = ldexpf(xs[qq][4 * hh + j], e);
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
  const int blane = 16 * (2 * (g & 1) + h) + n;  // B lane group 2 (g % 2) + h
  const int byte0 = 16 * (g >> 1);
#pragma unroll
  for (int p = 0; p < 3; ++p)
    *reinterpret_cast<uint4*>(span + (((u * 3 + p) * 2 + (byte0 >> 4)) * 64 + blane) * 16) =
        make_uint4(d[p][0], d[p][1], d[p][2], d[p][3]);
  if (g == 0 && h == 0) reinterpret_cast<int*>(span + kPartBytes)[u * 16 + n] = e;
}

}  // namespace f4m
}  // namespace lq
