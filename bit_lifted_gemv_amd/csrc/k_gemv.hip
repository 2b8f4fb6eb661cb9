// Small-batch product of 1-bit weights with float lifted activations:
//   out[b][i] = s[i] * sum_k sigma_ik * a_hat[b][k],  sigma = 2*bit - 1
// (LiftQuant notes, 关键设计 4: after the activation transform the layer is a
// product of 1-bit weights with floats, scaled per row by s).
//
// The weights stream from HBM once; the kernel is bound by HBM bandwidth as
// long as the work per weight bit stays small.  One vector op per bit would
// already be too slow on gfx950 (64 lanes x 4 SIMDs x 2.4 GHz = 39 T lane-ops/s
// against 64 T weight bits/s at 8 TB/s), so the sign-select is done a byte at a
// time through a table of activation sums:
//   E_p[v] = sum_{t<8} (2*bit_t(v) - 1) * a_hat[8p + t]     (v = 0..255)
// for the 64 byte positions p of a 512-bit slice of the lifted dimension.
// The sum over a weight row is then one table read and one add per byte.
// The tables hold activation sums, rebuilt from a_hat on every call; nothing
// about the weights is tabulated.
//
// LDS layout: entry (slot, v) at byte 256*v + 4*slot, 64 slots x 256 entries
// = 64 KB per workgroup (two workgroups per CU).  A byte of weights turns into
// its table address with a single v_perm_b32 (weight byte -> address byte 1,
// lane constant 4*slot -> address byte 0).  Lanes are laid out so that the 32
// lanes of each half-wave read 32 different slots whose banks (slot mod 32)
// are all distinct: reads are free of bank conflicts.
//
// Work split: a workgroup owns 64*JR rows and a run of slices (a K-part).  Per
// slice it loads its weights (8 bytes per lane per 8-row group), builds the
// table for each token (8 waves x 32 entries, Gray-code order: one add per
// entry), and accumulates.  With more than one K-part the partial sums go to
// a workspace and the last workgroup of a row block (arrival counter) adds
// them in part order, so the result is deterministic.
#include "lq_internal.h"

namespace lq {
namespace {

constexpr int kThreads = 512;              // 8 waves
constexpr int kWaves = kThreads / 64;
constexpr int kSliceBits = 512;
constexpr int kSliceWords = kSliceBits / 32;   // 16
constexpr int kTableFloats = 64 * 256;         // 64 KB

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
__host__ __device__ constexpr int ctz5(int i) {
  return (i & 1) ? 0 : (i & 2) ? 1 : (i & 4) ? 2 : (i & 8) ? 3 : 4;
}

// Lifted activations of byte position `lane` of slice `sl` for one token
// (zero past K; K is a multiple of 4).
__device__ __forceinline__ void load_x(const float* __restrict__ ah_tok, int64_t K, int sl,
                                       int lane, float4& x0, float4& x1) {
  const int64_t k0 = (int64_t)sl * kSliceBits + 8 * lane;
  x0 = make_float4(0.f, 0.f, 0.f, 0.f);
  x1 = x0;
  if (k0 + 4 <= K) x0 = *reinterpret_cast<const float4*>(ah_tok + k0);
  if (k0 + 8 <= K) x1 = *reinterpret_cast<const float4*>(ah_tok + k0 + 4);
}

// Build the 64 x 256 table of one slice and token: wave w writes entries
// v in [32w, 32w + 32) of every slot, lane p owns byte position p.
__device__ __forceinline__ void build_table(float* __restrict__ table, const float4& x0,
                                            const float4& x1, int wave, int lane) {
  const int p = lane;
  const int slot = p ^ ((p >> 5) << 2);
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  // v0 = 32*wave: bits 0..4 clear, bits 5..7 = wave bits 0..2
  float val = -(x[0] + x[1] + x[2] + x[3] + x[4]);
  val += (wave & 1) ? x[5] : -x[5];
  val += (wave & 2) ? x[6] : -x[6];
  val += (wave & 4) ? x[7] : -x[7];
  float tw[5];
#pragma unroll
  for (int t = 0; t < 5; ++t) tw[t] = 2.f * x[t];
  float* base = table + (32 * wave) * 64 + slot;
  base[0] = val;
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    const int t = ctz5(i);
    const bool up = (gray(i) >> t) & 1;
    val = up ? val + tw[t] : val - tw[t];
    base[gray(i) * 64] = val;
  }
}

template <int NT, int JR>
__global__ void __launch_bounds__(kThreads, 2) gemv_lut_kernel(
    const uint32_t* __restrict__ w, int64_t m, int64_t K, int64_t ldw, const float* __restrict__ s,
    const float* __restrict__ ah, int B, float* __restrict__ out, float* __restrict__ partials,
    unsigned* __restrict__ counters, int slices_per_part, int parts, int slices,
    uint32_t w_bytes) {
  __shared__ float table[kTableFloats];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rb = blockIdx.x / parts;
  const int part = blockIdx.x - rb * parts;
  constexpr int R = 64 * JR;
  const int64_t row0 = (int64_t)rb * R;
  const int sl0 = part * slices_per_part;
  const int sl1 = min(sl0 + slices_per_part, slices);

  // lane -> (row within an 8-row group, 8-byte chunk of the 64-byte slice row)
  const int rsub = lane >> 3;
  const int c = lane & 7;
  const int r4 = rsub & 3;
  // address bytes 4*slot for byte b of dword dd: slot = 8c + 4(dd ^ [c>=4]) + b
  uint32_t lc[2];
#pragma unroll
  for (int dd = 0; dd < 2; ++dd) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t a4 = 4u * (8u * c + 4u * (dd ^ (c >= 4 ? 1 : 0)) + b);
      v |= a4 << (8 * b);
    }
    lc[dd] = v;
  }
  // selector of step i: byte b = (i + r4) & 3 of the weight dword goes to the
  // address byte 1, byte b of the lane constant to byte 0, zeros above.
  uint32_t sel[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (i + r4) & 3;
    sel[i] = b | ((4u + b) << 8) | 0x0C0C0000u;
  }

  float acc[NT][JR];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < JR; ++j) acc[t][j] = 0.f;

  // Software pipeline over steps (slice, token): the activations of the next
  // step and the weights of the next slice are requested before the current
  // table is built, so their latency hides behind the build and the lookups.
  // Weight loads go through a buffer resource sized to the whole weight array:
  // lanes past the last row read zeros without a branch.  Words past K (and
  // past ldw, which would belong to the next row) multiply table entries that
  // are zero, because the activations past K are zero.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w), (short)0, static_cast<int>(w_bytes), 0x00020000);
  const uint32_t lane_off = static_cast<uint32_t>(((row0 + wave * 8 + rsub) * ldw + 2 * c) * 4);
  const uint32_t jstride = static_cast<uint32_t>(kWaves * 8 * ldw * 4);
  auto load_w = [&](int sl, uint2* wv) {
    const uint32_t soff = static_cast<uint32_t>(sl) * (kSliceWords * 4);
#pragma unroll
    for (int j = 0; j < JR; ++j) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(wres, lane_off + j * jstride, soff, 0);
      __builtin_memcpy(&wv[j], &v, 8);
    }
  };
  uint2 wv[JR], wn[JR];
  float4 xc0, xc1, xn0, xn1;
  if (sl0 < sl1) {
    load_x(ah, K, sl0, lane, xc0, xc1);
    load_w(sl0, wv);
  }
  const char* tb = reinterpret_cast<const char*>(table);
  for (int sl = sl0; sl < sl1; ++sl) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < B) {
        // next step's activations first, then the next slice's weights
        const bool last_tok = (t + 1 >= B) || (t + 1 >= NT);
        if (!last_tok) load_x(ah + (int64_t)(t + 1) * K, K, sl, lane, xn0, xn1);
        else if (sl + 1 < sl1) load_x(ah, K, sl + 1, lane, xn0, xn1);
        if (t == 0 && sl + 1 < sl1) load_w(sl + 1, wn);
        __syncthreads();                       // previous readers of the table are done
        build_table(table, xc0, xc1, wave, lane);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < JR; ++j) {
          float a0 = *reinterpret_cast<const float*>(
              tb + __builtin_amdgcn_perm(wv[j].x, lc[0], sel[0]));
          float a1 = *reinterpret_cast<const float*>(
              tb + __builtin_amdgcn_perm(wv[j].y, lc[1], sel[0]));
#pragma unroll
          for (int i = 1; i < 4; ++i) {
            a0 += *reinterpret_cast<const float*>(tb + __builtin_amdgcn_perm(wv[j].x, lc[0], sel[i]));
            a1 += *reinterpret_cast<const float*>(tb + __builtin_amdgcn_perm(wv[j].y, lc[1], sel[i]));
          }
          acc[t][j] += a0 + a1;
        }
        xc0 = xn0;
        xc1 = xn1;
      }
    }
#pragma unroll
    for (int j = 0; j < JR; ++j) wv[j] = wn[j];
  }

  // reduce the 8 lanes of each row; lane c == 0 holds the row's partial sum
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < JR; ++j) acc[t][j] = sum8(acc[t][j]);

  if (parts == 1) {
    if (c == 0) {
#pragma unroll
      for (int j = 0; j < JR; ++j) {
        const int64_t row = row0 + (j * kWaves + wave) * 8 + rsub;
        if (row < m) {
          const float sc = s[row];
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (t < B) out[(int64_t)t * m + row] = sc * acc[t][j];
        }
      }
    }
    return;
  }

  if (c == 0) {
#pragma unroll
    for (int j = 0; j < JR; ++j) {
      const int64_t row = row0 + (j * kWaves + wave) * 8 + rsub;
      if (row < m) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t < B) partials[((int64_t)part * B + t) * m + row] = acc[t][j];
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(&counters[rb], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == static_cast<unsigned>(parts - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int64_t nrows = (m - row0) < R ? (m - row0) : R;
  for (int64_t i = tid; i < nrows * B; i += kThreads) {
    const int t = static_cast<int>(i / nrows);
    const int64_t row = row0 + (i - (int64_t)t * nrows);
    float sum = 0.f;
    for (int p = 0; p < parts; ++p)
      sum += __hip_atomic_load(&partials[((int64_t)p * B + t) * m + row], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    out[(int64_t)t * m + row] = s[row] * sum;
  }
  if (tid == 0)
    __hip_atomic_store(&counters[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Rows per workgroup are 64*JR.  JR = 8 keeps every variant under 128 VGPRs,
// so two 512-thread workgroups (64 KB of table each) share a CU.
constexpr int kMaxJR = 8;

}  // namespace

GemvPlan plan_gemv(int64_t m, int64_t K, int64_t B) {
  GemvPlan p{};
  p.slices = static_cast<int>((K + kSliceBits - 1) / kSliceBits);
  const int target = 512;                       // 2 workgroups per CU
  // Largest row block that still leaves enough workgroups once K is split.
  int best_jr = 1, best_spp = 1;
  double best_cost = 1e300;
  for (int jr = 1; jr <= kMaxJR; jr *= 2) {
    const int64_t R = 64 * jr;
    const int64_t rbs = (m + R - 1) / R;
    for (int spp = 1; spp <= p.slices; ++spp) {
      const int64_t parts = (p.slices + spp - 1) / spp;
      const int64_t nwg = rbs * parts;
      const int64_t rounds = (nwg + target - 1) / target;
      // cost per workgroup in "bytes of HBM time": weights + table builds
      // (about 6.5 KB each) + partial sums written and read back.
      const double wg = (double)R * spp * 64.0 + (double)spp * B * 6656.0 +
                        (parts > 1 ? (double)R * B * 8.0 : 0.0);
      const double cost = rounds * wg;
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        best_jr = jr;
        best_spp = spp;
      }
    }
  }
  p.rows_per_wg = 64 * best_jr;
  p.slices_per_part = best_spp;
  p.parts = (p.slices + best_spp - 1) / best_spp;
  p.row_blocks = static_cast<int>((m + p.rows_per_wg - 1) / p.rows_per_wg);
  p.ws_bytes = 0;
  if (p.parts > 1)
    p.ws_bytes = gemv_counter_bytes(m) + sizeof(float) * (size_t)p.parts * (size_t)B * (size_t)m;
  return p;
}

size_t gemv_counter_bytes(int64_t m) {
  // one arrival counter per possible row block (row blocks are >= 64 rows)
  return ((size_t)((m + 63) / 64) * sizeof(unsigned) + 255) / 256 * 256;
}

size_t gemv_workspace_bytes(int64_t m, int64_t K, int64_t B) {
  size_t mx = 0;
  for (int64_t bt = 1; bt <= (B < 4 ? B : 4); ++bt) {
    const size_t b = plan_gemv(m, K, bt).ws_bytes;
    if (b > mx) mx = b;
  }
  return mx;
}

template <int NT, int JR>
static hipError_t launch_t(const GemvPlan& p, const uint32_t* w, int64_t m, int64_t K,
                           int64_t ldw, const float* s, const float* ah, int64_t B, float* out,
                           void* ws, hipStream_t st) {
  // workspace: [arrival counters][partial sums]; counters stay zero between calls
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (p.parts > 1) {
    counters = static_cast<unsigned*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + gemv_counter_bytes(m));
  }
  hipLaunchKernelGGL((gemv_lut_kernel<NT, JR>), dim3(p.row_blocks * p.parts), dim3(kThreads), 0,
                     st, w, m, K, ldw, s, ah, static_cast<int>(B), out, partials, counters,
                     p.slices_per_part, p.parts, p.slices,
                     static_cast<uint32_t>(m * ldw * 4));
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_nt(const GemvPlan& p, const uint32_t* w, int64_t m, int64_t K,
                            int64_t ldw, const float* s, const float* ah, int64_t B, float* out,
                            void* ws, hipStream_t st) {
  switch (p.rows_per_wg / 64) {
    case 1: return launch_t<NT, 1>(p, w, m, K, ldw, s, ah, B, out, ws, st);
    case 2: return launch_t<NT, 2>(p, w, m, K, ldw, s, ah, B, out, ws, st);
    case 4: return launch_t<NT, 4>(p, w, m, K, ldw, s, ah, B, out, ws, st);
    case 8: return launch_t<NT, 8>(p, w, m, K, ldw, s, ah, B, out, ws, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const GemvPlan& p, const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                       const float* s, const float* ah, int64_t B, float* out, void* ws,
                       hipStream_t st) {
  if (B <= 1) return launch_nt<1>(p, w, m, K, ldw, s, ah, B, out, ws, st);
  if (B <= 2) return launch_nt<2>(p, w, m, K, ldw, s, ah, B, out, ws, st);
  if (B <= 4) return launch_nt<4>(p, w, m, K, ldw, s, ah, B, out, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace lq
