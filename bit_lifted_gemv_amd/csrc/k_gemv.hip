// Small-batch product of 1-bit weights with float lifted activations:
//   out[b][i] = s[i] * sum_k sigma_ik * a_hat[b][k],  sigma = 2*bit - 1
// (LiftQuant notes, 关键设计 4: after the activation transform the layer is a
// product of 1-bit weights with floats, scaled per row by s).
//
// The weights stream from HBM once, so the kernel is bound by HBM bandwidth
// as long as the work per weight bit stays small.  One vector op per bit
// would already be too slow on gfx950 (64 lanes x 4 SIMDs x 2.4 GHz = 39 T
// lane-ops/s against 64 T weight bits/s at 8 TB/s), so the sign-select is done
// a byte at a time through tables of activation sums:
//   E_p[v] = sum_{t<8} (2*bit_t(v) - 1) * a_hat[8p + t]     (v = 0..255)
// for the 128 byte positions p of a 1024-bit slice of the lifted dimension.
// A row's sum is then one table read and one add per weight byte.  The tables
// hold activation sums rebuilt from a_hat on every call; nothing about the
// weights is tabulated.
//
// LDS layout (128 KB, one workgroup per CU): entry (slot, v) at byte
// 65536*(slot >> 6) + 256*v + 4*(slot & 63).  A weight byte becomes its
// table address with one v_perm_b32: the weight byte goes to address byte 1,
// a per-lane constant supplies bytes 0 and 2.  Lanes are arranged so that the
// 32 lanes of each half-wave hit 32 different banks on every read.
//
// Work split (persistent, stream-K): the iteration space is ordered
// (row block, slice, 64-row step) and cut into one equal range per CU, so the
// load is balanced to one 64-row step.  A workgroup walks its range a unit
// (row block x slice) at a time: it requests the next unit's weights (8
// rows x 128 B per wave per step, 16 B per lane) two units ahead, builds the
// current unit's table, and does the lookups.  A row block owned by one workgroup is written
// straight to the output; a row block split over several workgroups leaves
// one partial sum per workgroup in the workspace, and the last of them to
// arrive (arrival counter) adds them in workgroup order, so the result is
// deterministic.
#include "lut_common.h"

namespace lq {
namespace {

struct Sched {
  int64_t T;        // 64-row steps in the iteration space (row blocks x slices x JR)
  int G;            // workgroups
  int S;            // slices
  int rbs;          // row blocks
  int kmax;         // most workgroups sharing one row block
};

// Workgroup whose range holds step g: the largest w with floor(w*T/G) <= g.
__host__ __device__ __forceinline__ int owner(int64_t g, int64_t T, int G) {
  return static_cast<int>(((g + 1) * G + T - 1) / T - 1);
}

// THREADS: workgroup size (8 or 16 waves); NT: tokens per launch (tables are
// rebuilt per token, weights stay in registers); JR: row steps per unit (a
// row step is 8 rows per wave); DEPTH: units of weights held in registers
// (DEPTH - 1 of them in flight behind the current one).
template <int THREADS, int NT, int JR, int DEPTH>
__global__ void __launch_bounds__(THREADS, 1) gemv_lut_kernel(
    const uint32_t* __restrict__ w, int64_t m, int64_t K, int64_t ldw, const float* __restrict__ s,
    const float* __restrict__ ah, int B, float* __restrict__ out, float* __restrict__ partials,
    unsigned* __restrict__ counters, Sched sc, uint32_t w_bytes, uint32_t a_bytes) {
  __shared__ float table[kTableFloats];
  __shared__ float4 xstage[2][256];   // activations of a slice, by slot (double-buffered)
  __shared__ int s_last;

  constexpr int kThreads = THREADS;
  constexpr int kWaves = THREADS / 64;
  constexpr int kRowsPerStep = kWaves * 8;
  constexpr int R = kRowsPerStep * JR;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wg = blockIdx.x;
  const int64_t g_begin = (int64_t)wg * sc.T / sc.G;
  const int64_t g_end = (int64_t)(wg + 1) * sc.T / sc.G;
  if (g_begin >= g_end) return;
  const int64_t u_begin = g_begin / JR;
  const int64_t u_last = (g_end - 1) / JR;

  // lane -> (row r of the wave's 8 rows, 16-byte chunk c of the 128-byte slice row)
  const int r = lane >> 3;
  const int c = lane & 7;
  const int r4 = r & 3;
  uint32_t lc[4][4];
  uint32_t sel[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (i + r4) & 3;
    sel[i] = 0u | ((4u + b) << 8) | (2u << 16) | (0x0Cu << 24);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int sl = slot_of(16 * c + 4 * d + static_cast<int>(b));
      lc[d][i] = static_cast<uint32_t>(4 * (sl & 63)) | (static_cast<uint32_t>(sl >> 6) << 16);
    }
  }
  // byte position whose table entries this lane writes (slot 64h + lane)
  const int my_pos = slot_of(64 * (wave & 1) + lane);

  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(w), (short)0, static_cast<int>(w_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ah), (short)0, static_cast<int>(a_bytes), 0x00020000);
  const uint32_t row_bytes = static_cast<uint32_t>(ldw * 4);

  // Weights of unit u, 64-row steps [j_lo, j_hi) only (the rest load nothing).
  auto load_unit = [&](int64_t u, uint4* wv) {
    const bool ok = u <= u_last;
    const int64_t rb = u / sc.S;
    const int sl = static_cast<int>(u - rb * sc.S);
    const int j_lo = (ok && u == u_begin) ? static_cast<int>(g_begin - u * JR) : 0;
    const int j_hi = (ok && u == u_last) ? static_cast<int>(g_end - u * JR) : JR;
    const uint32_t base = static_cast<uint32_t>(
        (rb * R + wave * 8 + r) * (int64_t)row_bytes + (int64_t)sl * kSliceBytes + 16 * c);
#pragma unroll
    for (int j = 0; j < JR; ++j) {
      const uint32_t off = (ok && j >= j_lo && j < j_hi)
                               ? base + static_cast<uint32_t>(j * kRowsPerStep) * row_bytes
                               : kNoLoad;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(wres, off, 0, 0);
      __builtin_memcpy(&wv[j], &v, 16);
    }
  };

  float acc[NT][JR];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < JR; ++j) acc[t][j] = 0.f;

  // Flush row block rb (all of its rows this workgroup touched).
  auto flush = [&](int64_t rb) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < JR; ++j) acc[t][j] = sum8(acc[t][j]);
    const int64_t g0 = rb * sc.S * JR;
    const int w_first = owner(g0, sc.T, sc.G);
    const int w_last = owner(g0 + (int64_t)sc.S * JR - 1, sc.T, sc.G);
    const int n = w_last - w_first + 1;
    if (n == 1) {
      if (c == 0) {
#pragma unroll
        for (int j = 0; j < JR; ++j) {
          const int64_t row = rb * R + j * kRowsPerStep + wave * 8 + r;
          if (row < m) {
            const float scale = s[row];
#pragma unroll
            for (int t = 0; t < NT; ++t)
              if (t < B) out[(int64_t)t * m + row] = scale * acc[t][j];
          }
        }
      }
    } else {
      // partials[rb][k][t][R], k = this workgroup's place among the n sharers;
      // written and read with device-scope accesses (no cache-wide fences)
      const int k = wg - w_first;
      float* pb = partials + ((rb * sc.kmax + k) * (int64_t)NT) * R;
      if (c == 0) {
#pragma unroll
        for (int j = 0; j < JR; ++j) {
          const int rr = j * kRowsPerStep + wave * 8 + r;
#pragma unroll
          for (int t = 0; t < NT; ++t)
            __hip_atomic_store(pb + t * R + rr, acc[t][j], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&counters[rb], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == static_cast<unsigned>(n - 1)) ? 1 : 0;
      }
      __syncthreads();
      if (s_last) {
        const float* p0 = partials + (rb * sc.kmax * (int64_t)NT) * R;
        for (int i = tid; i < NT * R; i += kThreads) {
          const int t = i / R;
          const int rr = i - t * R;
          const int64_t row = rb * R + rr;
          if (t < B && row < m) {
            // batches of 8 independent loads, added in part order
            const float* pp = p0 + (int64_t)t * R + rr;
            const int64_t stride = (int64_t)NT * R;
            float sum = 0.f;
            for (int k0 = 0; k0 < n; k0 += 8) {
              float v[8];
#pragma unroll
              for (int e = 0; e < 8; ++e)
                v[e] = (k0 + e < n) ? __hip_atomic_load(pp + (k0 + e) * stride, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                    : 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) sum += v[e];
            }
            out[(int64_t)t * m + row] = s[row] * sum;
          }
        }
        if (tid == 0)
          __hip_atomic_store(&counters[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < JR; ++j) acc[t][j] = 0.f;
  };

  const char* tb = reinterpret_cast<const char*>(table);
  uint4 wbuf[DEPTH][JR];
  // Activations of the next table travel through LDS: waves 0 and 1 load a
  // slice (one byte position per lane) into registers, store it to the free
  // half of `xstage` once the current lookups are issued, and every wave
  // reads its 8 values from there when it builds the table.
  const bool x_loader = wave < 2;
  const int my_slot = 64 * (wave & 1) + lane;
  float4 xn0 = make_float4(0.f, 0.f, 0.f, 0.f), xn1 = xn0;
  int xb = 0;                                   // xstage half of the current step
  if (x_loader) {
    const int64_t rb = u_begin / sc.S;
    load_x(ares, K, 0, static_cast<int>(u_begin - rb * sc.S), my_pos, xn0, xn1);
  }
#pragma unroll
  for (int k = 0; k + 1 < DEPTH; ++k) load_unit(u_begin + k, wbuf[k]);
  if (x_loader) {
    xstage[0][2 * my_slot] = xn0;
    xstage[0][2 * my_slot + 1] = xn1;
  }

  // One unit: its weights are in `cur`; the weights DEPTH - 1 units ahead go
  // to `ahead`, so DEPTH - 1 units of loads stay in flight behind this one.
  // Steps past the end (active == false) still issue their (empty) loads and
  // register moves, so every pass of the unrolled loop has the same register
  // flow and the compiler never has to drain the loads in flight.
  auto do_unit = [&](int64_t u, bool active, const uint4* cur, uint4* ahead) {
    const int64_t rb = u / sc.S;
    const int sl = static_cast<int>(u - rb * sc.S);
    const int j_lo = (u == u_begin) ? static_cast<int>(g_begin - u * JR) : 0;
    const int j_hi = (u == u_last) ? static_cast<int>(g_end - u * JR) : JR;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // next step's activations (loader waves), then once per unit the
      // weights DEPTH - 1 units on
      if (x_loader) {
        if (t + 1 < B && t + 1 < NT) {
          load_x(ares, K, t + 1, active ? sl : sc.S, my_pos, xn0, xn1);
        } else {
          const int64_t un = u + 1;
          const int64_t rbn = un / sc.S;
          load_x(ares, K, 0, un <= u_last ? static_cast<int>(un - rbn * sc.S) : sc.S, my_pos,
                 xn0, xn1);
        }
      }
      if (t == 0) load_unit(u + DEPTH - 1, ahead);
      if (active && t < B) {
        __syncthreads();                       // table readers done, xstage[xb] written
        const float4 xc0 = xstage[xb][2 * my_slot];
        const float4 xc1 = xstage[xb][2 * my_slot + 1];
        build_table<kWaves>(table, xc0, xc1, wave, lane);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < JR; ++j) {
          if (j >= j_lo && j < j_hi) {
            const uint32_t wd[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
            float a[4];
#pragma unroll
            for (int d = 0; d < 4; ++d)
              a[d] = *reinterpret_cast<const float*>(tb + __builtin_amdgcn_perm(wd[d], lc[d][0],
                                                                               sel[0]));
#pragma unroll
            for (int i = 1; i < 4; ++i)
#pragma unroll
              for (int d = 0; d < 4; ++d)
                a[d] += *reinterpret_cast<const float*>(
                    tb + __builtin_amdgcn_perm(wd[d], lc[d][i], sel[i]));
            acc[t][j] += (a[0] + a[1]) + (a[2] + a[3]);
          }
        }
        xb ^= 1;
      }
      // the other half was last read before this step's second barrier
      if (x_loader) {
        xstage[xb][2 * my_slot] = xn0;
        xstage[xb][2 * my_slot + 1] = xn1;
      }
    }
    if (active && (u == u_last || (u + 1) / sc.S != rb)) flush(rb);
  };

  for (int64_t u = u_begin; u <= u_last; u += DEPTH) {
#pragma unroll
    for (int k = 0; k < DEPTH; ++k)
      do_unit(u + k, u + k <= u_last, wbuf[k], wbuf[(k + DEPTH - 1) % DEPTH]);
  }
}

constexpr int kUnitRows = 512;                  // rows per unit
constexpr int kGemvThreads = 1024;              // 16 waves: 4 per SIMD
constexpr int kJR = kUnitRows / (kGemvThreads / 8);

Sched make_sched(int64_t m, int64_t K, int jr, int G, int rows_per_step = kGemvThreads / 8) {
  Sched sc{};
  const int64_t R = (int64_t)rows_per_step * jr;
  sc.S = static_cast<int>((K + kSliceBits - 1) / kSliceBits);
  sc.rbs = static_cast<int>((m + R - 1) / R);
  sc.T = (int64_t)sc.rbs * sc.S * jr;
  sc.G = static_cast<int>(sc.T < G ? sc.T : G);
  int kmax = 1;
  for (int rb = 0; rb < sc.rbs; ++rb) {
    const int64_t g0 = (int64_t)rb * sc.S * jr;
    const int n = owner(g0 + (int64_t)sc.S * jr - 1, sc.T, sc.G) - owner(g0, sc.T, sc.G) + 1;
    if (n > kmax) kmax = n;
  }
  sc.kmax = kmax;
  return sc;
}


}  // namespace

static int g_num_cus[64] = {0};

int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_num_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_num_cus[dev] = n;
  }
  return g_num_cus[dev];
}

size_t gemv_counter_bytes(int64_t m) {
  // One 128-byte line per 16 rows: the one-token kernel keeps one counter
  // per block of 16, 32 or 64 rows at the head of a line, this one a counter
  // per row block (>= 512 rows) at the start of the region.  Both kernels put
  // their partial sums after the same counter region and leave every counter
  // at zero, so one workspace serves either.
  return ((size_t)((m + 15) / 16) * 128 + 255) / 256 * 256;
}

GemvPlan plan_gemv(int64_t m, int64_t K, int64_t B) {
  GemvPlan p{};
  const int nt = B <= 1 ? 1 : B <= 2 ? 2 : 4;
  const Sched sc = make_sched(m, K, kJR, num_cus());
  p.rows_per_wg = kUnitRows;
  p.slices = sc.S;
  p.row_blocks = sc.rbs;
  p.parts = sc.kmax;
  p.slices_per_part = 0;
  p.ws_bytes = 0;
  if (sc.kmax > 1)
    p.ws_bytes = gemv_counter_bytes(m) +
                 sizeof(float) * (size_t)sc.rbs * sc.kmax * nt * (size_t)p.rows_per_wg;
  return p;
}

size_t gemv_workspace_bytes(int64_t m, int64_t K, int64_t B) {
  size_t mx = 0;
  for (int64_t bt = 1; bt <= (B < 4 ? B : 4); ++bt) {
    const size_t b = plan_gemv(m, K, bt).ws_bytes;
    if (b > mx) mx = b;
  }
  return mx;
}

template <int NT>
static hipError_t launch_nt(const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                            const float* s, const float* ah, int64_t B, float* out, void* ws,
                            hipStream_t st) {
  const Sched sc = make_sched(m, K, kJR, num_cus());
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (sc.kmax > 1) {
    counters = static_cast<unsigned*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + gemv_counter_bytes(m));
  }
  // two units in flight for one token; with more tokens the per-unit work
  // hides the latency with one (and the registers go to accumulators)
  constexpr int DEPTH = 2;
  hipLaunchKernelGGL((gemv_lut_kernel<kGemvThreads, NT, kJR, DEPTH>), dim3(sc.G),
                     dim3(kGemvThreads), 0, st, w, m, K, ldw,
                     s, ah, static_cast<int>(B), out, partials, counters, sc,
                     static_cast<uint32_t>(m * ldw * 4), static_cast<uint32_t>(B * K * 4));
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvPlan&, const uint32_t* w, int64_t m, int64_t K, int64_t ldw,
                       const float* s, const float* ah, int64_t B, float* out, void* ws,
                       hipStream_t st) {
  if (B <= 1) return launch_nt<1>(w, m, K, ldw, s, ah, B, out, ws, st);
  if (B <= 2) return launch_nt<2>(w, m, K, ldw, s, ah, B, out, ws, st);
  if (B <= 4) return launch_nt<4>(w, m, K, ldw, s, ah, B, out, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace lq
