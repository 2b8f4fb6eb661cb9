// Activation lift with the Kronecker-factored whitening of the LiftQuant
// notes (关键设计 3: T = diag(s1) (P1 (x) P2) diag(s2), P1 n1 x n1 and P2
// n2 x n2 with n = n1 n2, s2 constant over each lift group so that it folds
// into M; 关键设计 4 applies T^-1 to the activations before the 1-bit product):
//   u     = diag(1/s2) (P1^-1 (x) P2^-1) diag(1/s1) a
//   a_hat = (I (x) M^T) u
// With channel c = i n2 + j of a token as entry (i, j) of an n1 x n2 matrix
// X, (P1^-1 (x) P2^-1) vec(X) = vec(P1^-1 X P2^-T): two small products per
// token instead of one n x n one.
//
// Both products run on the float32 matrix cores (16 x 16 x 4 steps, exact
// float32 products, float32 sums), each operand read as per-lane runs of
// consecutive k:
//   rows:    Z = (X / s1) P2^-T over the B n1 rows (token b, row i) of all
//            tokens, A = X / s1 (row-major, k = j'), B = P2^-1 (row j holds
//            its k = j' run).  Z goes to the workspace transposed per token,
//            Zt[b][j][i], so that the next product reads runs too.
//   columns: Y = P1^-1 Z per token, A = P1^-1 (row i, k = i'), B = Zt (row j,
//            k = i'); the wave's Y slab (16 rows i x a slab of columns j that
//            holds whole d-wide groups, n2 % d == 0) goes to LDS, group-major,
//            and the per-group step a_hat[g D + jj] = (1/s2[g]) sum_r
//            M[r][jj] Y[g d + r] is a third matrix-core product, groups x d
//            times d x D.
// Lane (l % 16, q = l / 16) of a 16 x 16 x 4 step holds A[l % 16][q] and
// B[q][l % 16]; over the KQ steps of a run lane q supplies k = KQ q + t, so a
// run is KQ consecutive elements and loads as 16-byte vectors.  The result
// lane holds rows 4 q + e (e < 4) of column l % 16.
#include <numeric>

#include "lq_internal.h"

namespace lq {
namespace {

using f32x4 = float __attribute__((ext_vector_type(4)));
using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kFar = 0x80000000u;     // past every range used here (< 2^31 bytes)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxN2 = 128;
constexpr int kMaxN1 = 256;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           static_cast<int>(bytes), kRsrcWord3);
}

template <int DT>
constexpr uint32_t kES = DT == LQ_F32 ? 4u : 2u;

template <int DT>
__device__ __forceinline__ float half_to_float(uint32_t h) {
  return DT == LQ_F16 ? f16_bits_to_float(static_cast<uint16_t>(h))
                      : bf16_bits_to_float(static_cast<uint16_t>(h));
}

// v[t] = element k0 + t of the row that starts `row` bytes into the
// resource, 0 where k0 + t >= len (such lanes take an offset past the range,
// which reads as zero, so there is no branch).  vec: len % 4 == 0 and rows
// start on 4-element boundaries, so a 4-element chunk is wholly in or out
// and loads as one 16-byte (float32) or 8-byte (16-bit) vector.
template <int DT, int KQ>
__device__ __forceinline__ void load_run(__amdgpu_buffer_rsrc_t r, uint32_t row, int k0, int len,
                                         bool vec, float (&v)[KQ]) {
  constexpr uint32_t es = kES<DT>;
  if (vec) {
#pragma unroll
    for (int u = 0; u < KQ / 4; ++u) {
      const int k = k0 + 4 * u;
      const uint32_t off = k < len ? row + static_cast<uint32_t>(k) * es : kFar;
      // (the loaded vector is bit-cast to a named vector type before its
      // elements are read: indexing the builtin's value directly lowered to
      // a single 4-byte load)
      if constexpr (DT == LQ_F32) {
        const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
#pragma unroll
        for (int c = 0; c < 4; ++c) v[4 * u + c] = x[c];
      } else {
        const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
        v[4 * u + 0] = half_to_float<DT>(x[0] & 0xffffu);
        v[4 * u + 1] = half_to_float<DT>(x[0] >> 16);
        v[4 * u + 2] = half_to_float<DT>(x[1] & 0xffffu);
        v[4 * u + 3] = half_to_float<DT>(x[1] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < KQ; ++t) {
      const int k = k0 + t;
      const uint32_t off = k < len ? row + static_cast<uint32_t>(k) * es : kFar;
      if constexpr (DT == LQ_F32)
        v[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
      else
        v[t] = half_to_float<DT>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
    }
  }
}

// One 16 x 16 block over a run pair: two interleaved accumulation chains.
template <int KQ>
__device__ __forceinline__ f32x4 mfma_run(const float (&a)[KQ], const float (&b)[KQ]) {
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f};
  f32x4 c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < KQ; t += 2) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t + 1], b[t + 1], c1, 0, 0, 0);
  }
  return c0 + c1;
}

// floor(x / y) for 0 <= x < 2^20, 1 <= y (float estimate, one correction).
__device__ __forceinline__ int small_div(int x, int y, float inv_y) {
  int r = static_cast<int>(static_cast<float>(x) * inv_y);
  if (r * y > x) --r;
  if ((r + 1) * y <= x) ++r;
  return r;
}

// Four consecutive outputs at element i (i % 4 == 0): one 16-byte (float32)
// or 8-byte (16-bit) store.
template <int O_DT>
__device__ __forceinline__ void store4(void* out, int64_t i, f32x4 v) {
  if constexpr (O_DT == LQ_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + i) = v;
  } else {
    u32x2 w;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t lo, hi;
      if constexpr (O_DT == LQ_F16) {
        lo = float_to_f16_bits_rne(v[2 * h]);
        hi = float_to_f16_bits_rne(v[2 * h + 1]);
      } else {
        lo = float_to_bf16_bits_rne(v[2 * h]);
        hi = float_to_bf16_bits_rne(v[2 * h + 1]);
      }
      w[h] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + i) = w;
  }
}

// Rows: wave w of workgroup x takes flat rows rho0 .. rho0 + 15 (rho = b n1
// + i over all tokens) and column blocks jb0 .. jb0 + nbj - 1 of Z (16
// columns each).  Its A run stays in registers; the B runs of the next
// column block load while the current one multiplies.
template <int A_DT, int KQ>
__global__ void __launch_bounds__(kThreads) kron_rows_kernel(
    const void* __restrict__ a, const float* __restrict__ s1, const float* __restrict__ p2_inv,
    float* __restrict__ zt, int n1, int n2, int rtot, int nbj, int vec) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int k0 = KQ * q;
  // the wave index is uniform: read it into a scalar register so that the
  // buffer resources built from it are scalar too
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int rho0 = (blockIdx.x * kWaves + wave) * 16;
  if (rho0 >= rtot) return;                         // no barriers in this kernel
  constexpr uint32_t es = kES<A_DT>;
  const uint32_t rows = static_cast<uint32_t>(min(16, rtot - rho0));
  const auto ra = rsrc(static_cast<const char*>(a) + static_cast<int64_t>(rho0) * n2 * es,
                       rows * static_cast<uint32_t>(n2) * es);
  const auto rs = rsrc(s1, static_cast<uint32_t>(n1 * n2) * 4u);
  const auto rp = rsrc(p2_inv, static_cast<uint32_t>(n2 * n2) * 4u);
  float x[KQ];
  {
    float s[KQ];
    const int i = (rho0 + r16) % n1;
    load_run<A_DT, KQ>(ra, static_cast<uint32_t>(r16 * n2) * es, k0, n2, vec, x);
    load_run<LQ_F32, KQ>(rs, static_cast<uint32_t>(i * n2) * 4u, k0, n2, vec, s);
#pragma unroll
    for (int t = 0; t < KQ; ++t) x[t] = k0 + t < n2 ? x[t] * __builtin_amdgcn_rcpf(s[t]) : 0.f;
  }
  const int jb0 = blockIdx.y * nbj;
  const int jb1 = min(jb0 + nbj, (n2 + 15) / 16);
  // row j of P2^-1 for column block jb (rows past n2 lie past the range)
  auto prow = [&](int jb) -> uint32_t {
    return jb < jb1 ? static_cast<uint32_t>((16 * jb + r16) * n2) * 4u : kFar;
  };
  auto store = [&](int jb, f32x4 acc) {
    const int j = 16 * jb + r16;
    if (j >= n2) return;
    const int rho = rho0 + 4 * q;
    if (vec && (n1 & 3) == 0) {
      // the four rows are i .. i + 3 of one token (rho0 % 16 == 0, n1 % 4 == 0)
      if (rho < rtot) {
        const int b = rho / n1;
        const int i = rho - b * n1;
        *reinterpret_cast<f32x4*>(zt + (static_cast<int64_t>(b) * n2 + j) * n1 + i) = acc;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (rho + e < rtot) {
          const int b = (rho + e) / n1;
          const int i = rho + e - b * n1;
          zt[(static_cast<int64_t>(b) * n2 + j) * n1 + i] = acc[e];
        }
      }
    }
  };
  float pb0[KQ], pb1[KQ];
  load_run<LQ_F32, KQ>(rp, prow(jb0), k0, n2, vec, pb0);
  for (int jb = jb0; jb < jb1; jb += 2) {
    load_run<LQ_F32, KQ>(rp, prow(jb + 1), k0, n2, vec, pb1);
    store(jb, mfma_run<KQ>(x, pb0));
    if (jb + 1 >= jb1) break;
    load_run<LQ_F32, KQ>(rp, prow(jb + 2), k0, n2, vec, pb0);
    store(jb + 1, mfma_run<KQ>(x, pb1));
  }
}

// Columns: workgroup (x, y, b) takes column slab x (16 nbj columns, whole
// groups) of token b; its wave w rows i0 = 16 (4 y + w) .. i0 + 15.  LDS:
// M [d][D], 1 / s2 of the workgroup's groups, then per wave the slab's Y
// group-major, yg[k][group] with
// group = row * (W / d) + (column / d) and k = column % d, rows padded to an
// odd length.
template <int O_DT, int KQ>
__global__ void __launch_bounds__(kThreads) kron_cols_kernel(
    const float* __restrict__ zt, const float* __restrict__ p1_inv,
    const float* __restrict__ s2, const float* __restrict__ M, void* __restrict__ out, int n1,
    int n2, int nbj, int d, int D, int vec, int vec_out) {
  extern __shared__ float4 lds4[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int b = blockIdx.z;
  const int i0 = (blockIdx.y * kWaves + wave) * 16;
  const int j0 = blockIdx.x * 16 * nbj;
  const int W = min(16 * nbj, n2 - j0);             // a multiple of d
  const int gpr = W / d;                            // groups per row of the slab
  const int gp = 16 * (16 * nbj / d) + 1;           // padded group count (odd)
  const int gsl = 16 * nbj / d;                     // groups per row of a full slab
  float* ms = reinterpret_cast<float*>(lds4);
  float* rs2s = ms + ((d * D + 3) & ~3);            // [kWaves * 16][gsl]: 1 / s2
  float* yg = rs2s + ((kWaves * 16 * gsl + 3) & ~3) + wave * d * gp;
  for (int e = threadIdx.x; e < d * D; e += kThreads) ms[e] = M[e];
  {
    // 1 / s2 of the workgroup's groups (rows 64 y .. 64 y + 63 of the slab)
    const int gpr_w = min(16 * nbj, n2 - j0) / d;
    const int ib = blockIdx.y * kWaves * 16;
    for (int e = threadIdx.x; e < kWaves * 16 * gsl; e += kThreads) {
      const int r = e / gsl;
      const int c = e - r * gsl;
      if (c < gpr_w && ib + r < n1)
        rs2s[e] = 1.f / s2[(ib + r) * (n2 / d) + j0 / d + c];
    }
  }

  if (i0 < n1) {
    const int n = n1 * n2;
    const auto rp = rsrc(p1_inv, static_cast<uint32_t>(n1 * n1) * 4u);
    const auto rz = rsrc(zt + static_cast<int64_t>(b) * n, static_cast<uint32_t>(n) * 4u);
    const int k0 = KQ * q;
    float pa[KQ];
    load_run<LQ_F32, KQ>(rp, static_cast<uint32_t>((i0 + r16) * n1) * 4u, k0, n1, vec, pa);
    const int nb = (W + 15) / 16;
    const float inv_d = 1.f / static_cast<float>(d);
    // column j0 + 16 jb + r16 of Zt; blocks past the slab take no loads
    auto zrow = [&](int jb) -> uint32_t {
      return jb < nb ? static_cast<uint32_t>((j0 + 16 * jb + r16) * n1) * 4u : kFar;
    };
    auto keep = [&](int jb, f32x4 acc) {
      const int c = 16 * jb + r16;                  // slab column
      if (c >= W) return;
      const int gq = small_div(c, d, inv_d);
      const int k = c - gq * d;
#pragma unroll
      for (int e = 0; e < 4; ++e) yg[k * gp + (4 * q + e) * gpr + gq] = acc[e];
    };
    float pb0[KQ], pb1[KQ];
    load_run<LQ_F32, KQ>(rz, zrow(0), k0, n1, vec, pb0);
    for (int jb = 0; jb < nb; jb += 2) {
      load_run<LQ_F32, KQ>(rz, zrow(jb + 1), k0, n1, vec, pb1);
      keep(jb, mfma_run<KQ>(pa, pb0));
      if (jb + 1 >= nb) break;
      load_run<LQ_F32, KQ>(rz, zrow(jb + 2), k0, n1, vec, pb0);
      keep(jb + 1, mfma_run<KQ>(pa, pb1));
    }
  }
  __syncthreads();
  if (i0 >= n1) return;

  // a_hat^T tile: D (16 a block) x groups of the wave's rows (16 a block), k
  // = r < d in steps of 4 (lane q supplies k = 4 s + q; k >= d adds zero).
  // A = M^T (lane: jj = jb + l % 16), B = the groups (lane: group gb + l %
  // 16); the result lane holds jj = jb + 4 q + e of group gb + l % 16, four
  // consecutive outputs of one group.
  const int rows = min(16, n1 - i0);
  const int G = rows * gpr;
  const int ks = (d + 3) / 4;
  const int64_t K = static_cast<int64_t>(n1 * n2 / d) * D;
  const int gpt = n2 / d;                           // groups per row of the token
  const float inv_gpr = 1.f / static_cast<float>(gpr);
  for (int gb = 0; gb < G; gb += 16) {
    const int gl = gb + r16;                        // this lane's group
    const bool ok = gl < G;
    const int row = small_div(gl, gpr, inv_gpr);
    const int g = (i0 + row) * gpt + j0 / d + (gl - row * gpr);
    const int64_t obase = static_cast<int64_t>(b) * K + static_cast<int64_t>(g) * D;
    const float rs2 = ok ? rs2s[(wave * 16 + row) * gsl + (gl - row * gpr)] : 0.f;
    for (int jb = 0; jb < D; jb += 16) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < ks; ++s) {
        const int k = 4 * s + q;
        const float mv = (k < d && jb + r16 < D) ? ms[k * D + jb + r16] : 0.f;
        const float yv = (k < d && ok) ? yg[k * gp + gl] : 0.f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mv, yv, acc, 0, 0, 0);
      }
      const int jj = jb + 4 * q;
      if (!ok || jj >= D) continue;
      acc *= rs2;
      if (vec_out)                                  // D % 4 == 0: jj .. jj + 3 < D, aligned
        store4<O_DT>(out, obase + jj, acc);
      else
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (jj + e < D) store_from_float<O_DT>(out, obase + jj + e, acc[e]);
    }
  }
}

int kq_for(int len) { return len <= 32 ? 8 : len <= 64 ? 16 : len <= 128 ? 32 : 64; }

// Column blocks per workgroup of the rows kernel: the most (dividing the
// row's blocks evenly) that still leave four workgroups per compute unit (loads of the next block wait on L2 while
// the current one multiplies; other waves cover the rest), else one.
int rows_blocks(int64_t B, int n1, int n2, int cus) {
  const int nbt = (n2 + 15) / 16;
  const int64_t rg = (B * n1 + 16 * kWaves - 1) / (16 * kWaves);
  for (int nbj = nbt; nbj > 1; --nbj)
    if (nbt % nbj == 0 && rg * (nbt / nbj) >= 4 * cus) return nbj;
  return 1;
}

// Column blocks per slab of the columns kernel: a slab (16 nbj columns)
// holds whole d-wide groups, or is the whole row; the widest slab (dividing
// the row evenly) that still leaves four workgroups per compute unit, else
// the narrowest.
int cols_blocks(int64_t B, int n1, int n2, int d, int cus) {
  const int nbt = (n2 + 15) / 16;
  const int step = d / std::gcd(16, d);
  if (step >= nbt) return nbt;
  const int64_t rg = B * ((n1 + 16 * kWaves - 1) / (16 * kWaves));
  if (rg >= 4 * cus) return nbt;
  int best = step;
  for (int nbj = step; nbj < nbt; nbj += step)
    if (nbt % nbj == 0 && rg * (nbt / nbj) >= 4 * cus) best = nbj;
  return best;
}

size_t cols_lds_bytes(int nbj, int d, int D) {
  const size_t gsl = 16 * static_cast<size_t>(nbj) / d;
  const size_t gp = 16 * gsl + 1;
  return sizeof(float) * (((static_cast<size_t>(d) * D + 3) & ~size_t{3}) +
                          ((kWaves * 16 * gsl + 3) & ~size_t{3}) +
                          static_cast<size_t>(kWaves) * d * gp);
}

template <int A_DT, int KQ>
hipError_t launch_rows_kq(const void* a, int64_t B, int n1, int n2, const float* s1,
                          const float* p2_inv, float* zt, int vec, hipStream_t st) {
  const int rtot = static_cast<int>(B * n1);
  const int nbt = (n2 + 15) / 16;
  const int nbj = rows_blocks(B, n1, n2, num_cus());
  hipLaunchKernelGGL((kron_rows_kernel<A_DT, KQ>),
                     dim3(static_cast<unsigned>((rtot + 16 * kWaves - 1) / (16 * kWaves)),
                          static_cast<unsigned>((nbt + nbj - 1) / nbj)),
                     dim3(kThreads), 0, st, a, s1, p2_inv, zt, n1, n2, rtot, nbj, vec);
  return hipGetLastError();
}

template <int A_DT>
hipError_t launch_rows(const void* a, int64_t B, int n1, int n2, const float* s1,
                       const float* p2_inv, float* zt, hipStream_t st) {
  const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const int vec = (n2 % 4 == 0) && al16(a) && al16(s1) && al16(p2_inv);
  switch (kq_for(n2)) {
    case 8: return launch_rows_kq<A_DT, 8>(a, B, n1, n2, s1, p2_inv, zt, vec, st);
    case 16: return launch_rows_kq<A_DT, 16>(a, B, n1, n2, s1, p2_inv, zt, vec, st);
    default: return launch_rows_kq<A_DT, 32>(a, B, n1, n2, s1, p2_inv, zt, vec, st);
  }
}

template <int O_DT, int KQ>
hipError_t launch_cols_kq(const float* zt, int64_t B, int n1, int n2, const float* p1_inv,
                          const float* s2, const float* M, int d, int D, void* out, int vec,
                          hipStream_t st) {
  const int nbt = (n2 + 15) / 16;
  const int nbj = cols_blocks(B, n1, n2, d, num_cus());
  const size_t lds = cols_lds_bytes(nbj, d, D);
  // four consecutive outputs of a group as one vector store
  const int vec_out = (D % 4 == 0) &&
                      (reinterpret_cast<uintptr_t>(out) % (O_DT == LQ_F32 ? 16 : 8)) == 0;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kron_cols_kernel<O_DT, KQ>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((kron_cols_kernel<O_DT, KQ>),
                     dim3(static_cast<unsigned>((nbt + nbj - 1) / nbj),
                          static_cast<unsigned>((n1 + 16 * kWaves - 1) / (16 * kWaves)),
                          static_cast<unsigned>(B)),
                     dim3(kThreads), lds, st, zt, p1_inv, s2, M, out, n1, n2, nbj, d, D, vec,
                     vec_out);
  return hipGetLastError();
}

template <int O_DT>
hipError_t launch_cols(const float* zt, int64_t B, int n1, int n2, const float* p1_inv,
                       const float* s2, const float* M, int d, int D, void* out, hipStream_t st) {
  const int vec = (n1 % 4 == 0) && (reinterpret_cast<uintptr_t>(p1_inv) & 15) == 0;
  switch (kq_for(n1)) {
    case 8: return launch_cols_kq<O_DT, 8>(zt, B, n1, n2, p1_inv, s2, M, d, D, out, vec, st);
    case 16: return launch_cols_kq<O_DT, 16>(zt, B, n1, n2, p1_inv, s2, M, d, D, out, vec, st);
    case 32: return launch_cols_kq<O_DT, 32>(zt, B, n1, n2, p1_inv, s2, M, d, D, out, vec, st);
    default: return launch_cols_kq<O_DT, 64>(zt, B, n1, n2, p1_inv, s2, M, d, D, out, vec, st);
  }
}

// ---- one launch for many tokens (small enough factors).  A workgroup of 8
// waves stages P2^-1, P1^-1, M and 1/s2 in LDS once, then takes tokens b =
// blockIdx.x, blockIdx.x + gridDim.x, ...: X = a_b / s1 into LDS, Z = X
// P2^-T and then Y = P1^-1 Z as 16 x 16 float32 MFMA tiles with both operands
// read from LDS (two tiles per wave at a time, so that two accumulation
// chains interleave), and the per-group M^T step as a third MFMA product
// whose result lanes hold four consecutive outputs of one group.  No Zt
// round trip through memory.  Row strides: n2 + 4 floats for X, Y and
// P2^-1 and n1 + 4 for P1^-1 (the 16 rows x 4 k of an operand read land in
// distinct banks), n2 + 16 for Z (read as 4 rows x 16 columns).
// Eight consecutive activations as float (i % 8 == 0, 16-byte aligned).
template <int DT>
__device__ __forceinline__ void load8_as_float(const void* base, int64_t i, float (&v)[8]) {
  if constexpr (DT == LQ_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
    const float4 x = p[0], y = p[1];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = half_to_float<DT>(w[e] & 0xFFFFu);
      v[2 * e + 1] = half_to_float<DT>(w[e] >> 16);
    }
  }
}

// Four consecutive outputs (i % 4 == 0, aligned) as one vector store.
template <int O_DT>
__device__ __forceinline__ void store4_out(void* out, int64_t i, const float* v) {
  if constexpr (O_DT == LQ_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + i) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint16_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      h[e] = O_DT == LQ_F16 ? float_to_f16_bits_rne(v[e]) : float_to_bf16_bits_rne(v[e]);
    uint2 q;
    q.x = h[0] | (static_cast<uint32_t>(h[1]) << 16);
    q.y = h[2] | (static_cast<uint32_t>(h[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + i) = q;
  }
}

constexpr int kFWaves = 8;
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFJT = 4;                    // D <= 64: at most 4 16-wide output tiles
constexpr int kFKS = 8;                    // d <= 32: at most 8 4-deep k steps

__host__ __device__ constexpr size_t fused_lds_floats(int n1, int n2, int d, int D) {
  return static_cast<size_t>(n1) * (n2 + 4) + static_cast<size_t>(n1) * (n2 + 16) +
         static_cast<size_t>(n2) * (n2 + 4) + static_cast<size_t>(n1) * (n1 + 4) +
         static_cast<size_t>(d) * D + static_cast<size_t>(n1) * n2 / d;
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// JT = ceil(D / 16) output tiles and KS >= ceil(d / 4) k steps of the
// per-group product, fixed at compile time so that its MFMAs run without
// branches between them (operands past d or D are zero).
template <int JT, int KS>
__global__ void __launch_bounds__(kFThreads, 1) kron_fused_kernel(
    const void* __restrict__ a, const float* __restrict__ s1, const float* __restrict__ p1,
    const float* __restrict__ p2, const float* __restrict__ s2, const float* __restrict__ M,
    void* __restrict__ out, int B, int n1, int n2, int d, int D, int a_dt, int out_dt) {
  extern __shared__ float lds[];
  const int n = n1 * n2;
  const int ldx = n2 + 4, ldz = n2 + 16, ldp2 = n2 + 4, ldp1 = n1 + 4;
  float* sX = lds;                          // [n1][ldx]: X, then Y
  float* sZ = sX + n1 * ldx;                // [n1][ldz]
  float* sP2 = sZ + n1 * ldz;               // [n2][ldp2]
  float* sP1 = sP2 + n2 * ldp2;             // [n1][ldp1]
  float* sM = sP1 + n1 * ldp1;              // [d][D]
  float* sR2 = sM + d * D;                  // [n / d]: 1 / s2
  const int tid = threadIdx.x;
  for (int i = tid; i < n2 * n2; i += kFThreads) sP2[(i / n2) * ldp2 + i % n2] = p2[i];
  for (int i = tid; i < n1 * n1; i += kFThreads) sP1[(i / n1) * ldp1 + i % n1] = p1[i];
  for (int i = tid; i < d * D; i += kFThreads) sM[i] = M[i];
  for (int i = tid; i < n / d; i += kFThreads) sR2[i] = 1.f / s2[i];

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int kq = lane >> 4;
  const int tj_n = n2 / 16;
  const int tiles = (n1 / 16) * tj_n;
  const int64_t K = static_cast<int64_t>(n / d) * D;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    __syncthreads();                        // staging done / the previous token's Y read
    // eight consecutive values per thread and pass (n2 % 8 == 0: a run stays
    // in one row of X)
    for (int c = 8 * tid; c < n; c += 8 * kFThreads) {
      float v[8];
      const int64_t ai = static_cast<int64_t>(b) * n + c;
      if (a_dt == LQ_F32)
        load8_as_float<LQ_F32>(a, ai, v);
      else if (a_dt == LQ_F16)
        load8_as_float<LQ_F16>(a, ai, v);
      else
        load8_as_float<LQ_BF16>(a, ai, v);
      const float4 r0 = *reinterpret_cast<const float4*>(s1 + c);
      const float4 r1 = *reinterpret_cast<const float4*>(s1 + c + 4);
      const float sv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
      float* xr = sX + (c / n2) * ldx + c % n2;
      float4 o0, o1;
      o0.x = v[0] / sv[0]; o0.y = v[1] / sv[1]; o0.z = v[2] / sv[2]; o0.w = v[3] / sv[3];
      o1.x = v[4] / sv[4]; o1.y = v[5] / sv[5]; o1.z = v[6] / sv[6]; o1.w = v[7] / sv[7];
      reinterpret_cast<float4*>(xr)[0] = o0;
      reinterpret_cast<float4*>(xr)[1] = o1;
    }
    __syncthreads();
    // Z = X P2^-T: A[i][k] = X[i][k], B[k][j] = P2^-1[j][k]; the result lane
    // holds column l16 and rows 4 kq + e of its tile
#pragma unroll 1
    for (int t0 = 2 * wave; t0 < tiles; t0 += 2 * kFWaves) {
      const int t1 = t0 + 1 < tiles ? t0 + 1 : t0;
      const float* xa0 = sX + ((t0 / tj_n) * 16 + l16) * ldx + kq;
      const float* xa1 = sX + ((t1 / tj_n) * 16 + l16) * ldx + kq;
      const float* pb0 = sP2 + ((t0 % tj_n) * 16 + l16) * ldp2 + kq;
      const float* pb1 = sP2 + ((t1 % tj_n) * 16 + l16) * ldp2 + kq;
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll 1
      for (int k = 0; k < n2; k += 16) {        // n2 % 16 == 0: operands of 4 steps first
        float a0[4], b0[4], a1[4], b1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a0[u] = xa0[k + 4 * u];
          b0[u] = pb0[k + 4 * u];
          a1[u] = xa1[k + 4 * u];
          b1[u] = pb1[k + 4 * u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          c0 = mfma4(a0[u], b0[u], c0);
          c1 = mfma4(a1[u], b1[u], c1);
        }
      }
      float* z0 = sZ + ((t0 / tj_n) * 16 + 4 * kq) * ldz + (t0 % tj_n) * 16 + l16;
      float* z1 = sZ + ((t1 / tj_n) * 16 + 4 * kq) * ldz + (t1 % tj_n) * 16 + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z0[e * ldz] = c0[e];
        z1[e * ldz] = c1[e];
      }
    }
    __syncthreads();
    // Y = P1^-1 Z into sX: A[i][k] = P1^-1[i][k], B[k][j] = Z[k][j]
#pragma unroll 1
    for (int t0 = 2 * wave; t0 < tiles; t0 += 2 * kFWaves) {
      const int t1 = t0 + 1 < tiles ? t0 + 1 : t0;
      const float* pa0 = sP1 + ((t0 / tj_n) * 16 + l16) * ldp1 + kq;
      const float* pa1 = sP1 + ((t1 / tj_n) * 16 + l16) * ldp1 + kq;
      const float* zb0 = sZ + kq * ldz + (t0 % tj_n) * 16 + l16;
      const float* zb1 = sZ + kq * ldz + (t1 % tj_n) * 16 + l16;
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll 1
      for (int k = 0; k < n1; k += 16) {        // n1 % 16 == 0
        float a0[4], b0[4], a1[4], b1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a0[u] = pa0[k + 4 * u];
          b0[u] = zb0[(k + 4 * u) * ldz];
          a1[u] = pa1[k + 4 * u];
          b1[u] = zb1[(k + 4 * u) * ldz];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          c0 = mfma4(a0[u], b0[u], c0);
          c1 = mfma4(a1[u], b1[u], c1);
        }
      }
      float* y0 = sX + ((t0 / tj_n) * 16 + 4 * kq) * ldx + (t0 % tj_n) * 16 + l16;
      float* y1 = sX + ((t1 / tj_n) * 16 + 4 * kq) * ldx + (t1 % tj_n) * 16 + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y0[e * ldx] = c0[e];
        y1[e * ldx] = c1[e];
      }
    }
    __syncthreads();
    // a_hat[b][g D + jj] = (1 / s2[g]) sum_r M[r][jj] Y[channel g d + r] as a
    // third product, C = M^T U^T (D x groups): A[i][k] = M[k][jt 16 + i],
    // B[k][j] = Y of group gt 16 + j at r = k (a group lies in one row of Y,
    // n2 % d == 0).  A wave takes whole tiles of 16 groups: its results go to
    // its own part of the (now free) Z buffer as [group][jj], then the wave
    // writes the tile's 16 D consecutive outputs in 4-value pieces.
    const int gtiles = n / d / 16;
    float* stage = sZ + wave * (16 * D);
    // the A operand (M) is the same for every group tile: load it once
    float av[JT][KS];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r = 4 * ks + kq;
        const int jm = jt * 16 + l16;
        // clamped address, then zeroed: no per-lane branch around the load
        const float v = sM[min(r, d - 1) * D + min(jm, D - 1)];
        av[jt][ks] = (r < d && jm < D) ? v : 0.f;
      }
#pragma unroll 1
    for (int gt = wave; gt < gtiles; gt += kFWaves) {
      const int g = gt * 16 + l16;                        // this lane's B column / group
      const int c0 = g * d;
      const float* yr = sX + (c0 / n2) * ldx + c0 % n2;
      float bv[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r = 4 * ks + kq;
        const float v = yr[min(r, d - 1)];
        bv[ks] = r < d ? v : 0.f;
      }
      const float sc = sR2[g];
      f32x4 c[JT];
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) c[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) c[jt] = mfma4(av[jt][ks], bv[ks], c[jt]);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const int jj0 = jt * 16 + 4 * kq;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (jj0 + e < D) stage[l16 * D + jj0 + e] = c[jt][e] * sc;
      }
      // the wave's own LDS writes are seen by its later reads in order
      const int64_t o = static_cast<int64_t>(b) * K + static_cast<int64_t>(gt) * 16 * D;
      for (int q = lane; q < 4 * D; q += 64) {
        if (out_dt == LQ_F32)
          store4_out<LQ_F32>(out, o + 4 * q, stage + 4 * q);
        else if (out_dt == LQ_F16)
          store4_out<LQ_F16>(out, o + 4 * q, stage + 4 * q);
        else
          store4_out<LQ_BF16>(out, o + 4 * q, stage + 4 * q);
      }
    }
  }
}

bool fused_applies(int64_t B, int n1, int n2, int d, int D, const void* a, const float* s1,
                   const void* out) {
  const bool aligned = reinterpret_cast<uintptr_t>(a) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(s1) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(out) % 16 == 0;
  return aligned && B >= 64 && d <= 4 * kFKS && D <= 16 * kFJT && n1 % 16 == 0 &&
         n2 % 16 == 0 && n2 % d == 0 &&
         (n1 * n2 / d) % 16 == 0 && 16 * D <= n1 * (n2 + 16) / kFWaves &&
         fused_lds_floats(n1, n2, d, D) * sizeof(float) <= 160 * 1024;
}

template <int JT, int KS>
hipError_t launch_fused_jk(const void* a, lq_dtype a_dt, int64_t B, int n1, int n2,
                           const float* s1, const float* p1, const float* p2, const float* s2,
                           const float* M, int d, int D, void* out, lq_dtype out_dt,
                           hipStream_t st) {
  const size_t lds = fused_lds_floats(n1, n2, d, D) * sizeof(float);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kron_fused_kernel<JT, KS>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  int cus = num_cus();
  const int grid = static_cast<int>(B < cus ? B : cus);
  hipLaunchKernelGGL((kron_fused_kernel<JT, KS>), dim3(static_cast<unsigned>(grid)),
                     dim3(kFThreads), lds, st, a, s1, p1, p2, s2, M, out, static_cast<int>(B),
                     n1, n2, d, D, static_cast<int>(a_dt), static_cast<int>(out_dt));
  return hipGetLastError();
}

template <int JT>
hipError_t launch_fused_j(const void* a, lq_dtype a_dt, int64_t B, int n1, int n2,
                          const float* s1, const float* p1, const float* p2, const float* s2,
                          const float* M, int d, int D, void* out, lq_dtype out_dt,
                          hipStream_t st) {
  if (d <= 4) return launch_fused_jk<JT, 1>(a, a_dt, B, n1, n2, s1, p1, p2, s2, M, d, D, out, out_dt, st);
  if (d <= 8) return launch_fused_jk<JT, 2>(a, a_dt, B, n1, n2, s1, p1, p2, s2, M, d, D, out, out_dt, st);
  if (d <= 16) return launch_fused_jk<JT, 4>(a, a_dt, B, n1, n2, s1, p1, p2, s2, M, d, D, out, out_dt, st);
  return launch_fused_jk<JT, 8>(a, a_dt, B, n1, n2, s1, p1, p2, s2, M, d, D, out, out_dt, st);
}

hipError_t launch_fused(const void* a, lq_dtype a_dt, int64_t B, int n1, int n2,
                        const float* s1, const float* p1, const float* p2, const float* s2,
                        const float* M, int d, int D, void* out, lq_dtype out_dt,
                        hipStream_t st) {
  switch ((D + 15) / 16) {
    case 1: return launch_fused_j<1>(a, a_dt, B, n1, n2, s1, p1, p2, s2, M, d, D, out, out_dt, st);
    case 2: return launch_fused_j<2>(a, a_dt, B, n1, n2, s1, p1, p2, s2, M, d, D, out, out_dt, st);
    case 3: return launch_fused_j<3>(a, a_dt, B, n1, n2, s1, p1, p2, s2, M, d, D, out, out_dt, st);
    default: return launch_fused_j<4>(a, a_dt, B, n1, n2, s1, p1, p2, s2, M, d, D, out, out_dt, st);
  }
}

}  // namespace

bool lift_kron_shape_ok(int64_t n, int n1, int d, int D) {
  if (n1 < 1 || n1 > kMaxN1 || n % n1) return false;
  const int64_t n2 = n / n1;
  if (n2 < 1 || n2 > kMaxN2 || n2 % d) return false;
  // the widest slab any batch size can pick
  return cols_lds_bytes((static_cast<int>(n2) + 15) / 16, d, D) <= 160 * 1024;
}

size_t lift_kron_workspace_bytes(int64_t B, int64_t n) {
  return (static_cast<size_t>(B) * n * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_lift_kron(const void* a, lq_dtype a_dt, int64_t B, int64_t n, int n1,
                            const float* s1, const float* p1_inv, const float* p2_inv,
                            const float* s2, const float* M, int d, int D, void* out,
                            lq_dtype out_dt, void* ws, hipStream_t st) {
  const int n2 = static_cast<int>(n / n1);
#ifndef LQ_KRON_FUSED
#define LQ_KRON_FUSED 1
#endif
  if (LQ_KRON_FUSED && fused_applies(B, n1, n2, d, D, a, s1, out))
    return launch_fused(a, a_dt, B, n1, n2, s1, p1_inv, p2_inv, s2, M, d, D, out, out_dt, st);
  float* zt = static_cast<float*>(ws);
  hipError_t e;
  switch (a_dt) {
    case LQ_F32: e = launch_rows<LQ_F32>(a, B, n1, n2, s1, p2_inv, zt, st); break;
    case LQ_F16: e = launch_rows<LQ_F16>(a, B, n1, n2, s1, p2_inv, zt, st); break;
    default: e = launch_rows<LQ_BF16>(a, B, n1, n2, s1, p2_inv, zt, st); break;
  }
  if (e != hipSuccess) return e;
  switch (out_dt) {
    case LQ_F32: return launch_cols<LQ_F32>(zt, B, n1, n2, p1_inv, s2, M, d, D, out, st);
    case LQ_F16: return launch_cols<LQ_F16>(zt, B, n1, n2, p1_inv, s2, M, d, D, out, st);
    default: return launch_cols<LQ_BF16>(zt, B, n1, n2, p1_inv, s2, M, d, D, out, st);
  }
}

}  // namespace lq
