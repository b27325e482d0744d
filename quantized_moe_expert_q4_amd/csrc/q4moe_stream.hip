// Grouped Q4 gate/up + SwiGLU over routed expert slots: two launches.
//
// Arithmetic: GATE_UP_SOURCE of the @mlx-bun/inference 1.0.0 diff, page 52
// (kernels/glm52/streamed-experts.ts), made exact as in q4moe_device.h; pair
// (t, j) is token t on slot ids[t][j], independent of every other pair.
//
// 1. prep_kernel (M+1 work-groups): work-group t splits token t's activations
//    into the six int8 digits once, in the byte order of the MFMA B operand,
//    into the workspace; the last work-group builds the routing plan -- a
//    counting sort of the (t, j) pairs by slot, the count of "virtual tiles"
//    (slot, token group of up to G, 32 rows) -- and zero-fills pairs with
//    out-of-range ids.
// 2. stream_kernel (persistent, one wave per unit range): the virtual tiles
//    times the K-steps of 128 positions form U units; wave w of W takes the
//    contiguous range [wU/W, (w+1)U/W), so every wave streams the same number
//    of weight bytes whatever the slot count.  Each wave keeps D K-steps of
//    weights and digits in flight (a register ring), reads its B fragments
//    from L2 (no LDS staging, no barriers), and accumulates exactly in int32.
//    A tile cut by a range boundary has two contributors: each publishes its
//    partial sums (exact int64) and bumps a counter with release order; the
//    second to arrive adds the other's partial and finishes the tile.  Nobody
//    waits, and integer addition makes the result independent of the order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4moe_device.h"
#include "q4moe_launch.h"

namespace q4 {

namespace {

constexpr int kStreamThreads = 256;       // four waves per work-group
constexpr int kDigitStepBytes = 768;      // one K-step of 128 positions: [par 2][g 4][digit 6][16 B]

struct Plan {
  int nt, rw, d, g, rtc, nsteps;
  bool vec;
};

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

}  // namespace

__global__ __launch_bounds__(kStreamThreads) void prep_kernel(const StreamParams a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint8_t* ws = a.ws;
  if ((int)blockIdx.x < a.M) {
    // ---- token t: largest |x|, then every digit of the token ----
    const int t = blockIdx.x;
    __shared__ int s_max;
    if (tid == 0) s_max = 0;
    __syncthreads();
    const uint4* xr = (const uint4*)(a.x + (uint64_t)t * a.H);
    uint32_t mx = 0;
    for (int w8 = tid; w8 < a.H / 8; w8 += kStreamThreads) mx = max(mx, max_mag8(xr[w8]));
    const int wm = wave_max((int)mx);
    if (lane == 0 && wm) atomicMax(&s_max, wm);
    __syncthreads();
    const int xm = s_max;
    if (tid == 0) ((int32_t*)(ws + a.off_xmax))[t] = xm;
    const int etop1 = max((xm >> 7) & 0xFF, 1);
    uint8_t* dst = ws + a.off_digits + (uint64_t)t * a.tok_stride;
    const int units = a.nsteps * 16;  // eight positions per unit
    for (int u = tid; u < units; u += kStreamThreads) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (8 * u < a.H) v = xr[u];
      uint32_t lo[8], hi[8];
      x8_digits(v, etop1, lo, hi);
      const int tl = u >> 4, gg = (u >> 2) & 3, i = u & 3;
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        uint32_t d[6];
        digit_words(lo, hi, par, d);
        uint8_t* base = dst + (uint64_t)tl * kDigitStepBytes + (par * 4 + gg) * 96 + 4 * i;
#pragma unroll
        for (int s = 0; s < 6; ++s) *(uint32_t*)(base + s * 16) = d[s];
      }
    }
    return;
  }

  // ---- routing plan (one work-group) ----
  int32_t* hdr = (int32_t*)ws;
  int32_t* cnt = (int32_t*)(ws + a.off_count);      // [E] counts, then cursors
  int32_t* off = (int32_t*)(ws + a.off_offset);     // [E+1] first pair of each slot
  int32_t* vpre = (int32_t*)(ws + a.off_vprefix);   // [E+1] first virtual tile of each slot
  int32_t* pairs = (int32_t*)(ws + a.off_pairs);    // [P] pair indices grouped by slot
  int32_t* bad = (int32_t*)(ws + a.off_bad);        // [P] out-of-range pairs (any order)
  int32_t* fixc = (int32_t*)(ws + a.off_fixcnt);    // [W] tile-split counters
  const int E = a.num_slots;
  const int P = a.M * a.K;
  __shared__ int s_bad;
  __shared__ int s_sum[kStreamThreads];
  __shared__ int s_vsum[kStreamThreads];
  if (tid == 0) s_bad = 0;
  for (int e = tid; e < E; e += kStreamThreads) cnt[e] = 0;
  for (int w = tid; w < a.W; w += kStreamThreads) fixc[w] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kStreamThreads) {
    const int e = a.ids[p];
    if (e >= 0 && e < E) {
      atomicAdd(&cnt[e], 1);
    } else {
      bad[atomicAdd(&s_bad, 1)] = p;
    }
  }
  __syncthreads();
  // exclusive scans of pair counts and virtual-tile counts over the slots
  const int chunk = (E + kStreamThreads - 1) / kStreamThreads;
  const int e0 = min(E, tid * chunk), e1 = min(E, e0 + chunk);
  int ls = 0, lv = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    ls += c;
    lv += (c + a.G - 1) / a.G * a.rtc;
  }
  s_sum[tid] = ls;
  s_vsum[tid] = lv;
  __syncthreads();
  if (tid == 0) {
    int run = 0, vrun = 0;
    for (int i = 0; i < kStreamThreads; ++i) {
      const int c = s_sum[i], v = s_vsum[i];
      s_sum[i] = run;
      s_vsum[i] = vrun;
      run += c;
      vrun += v;
    }
    off[E] = run;
    vpre[E] = vrun;
    hdr[1] = vrun;
  }
  __syncthreads();
  ls = s_sum[tid];
  lv = s_vsum[tid];
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    off[e] = ls;
    vpre[e] = lv;
    ls += c;
    lv += (c + a.G - 1) / a.G * a.rtc;
  }
  __syncthreads();
  for (int e = e0; e < e1; ++e) cnt[e] = off[e];
  __syncthreads();
  // place the pairs of each slot after its offset; the order inside a slot
  // only decides which tokens share a tile, and the exact sums make every
  // output independent of that, so plain atomic cursors suffice
  for (int p = tid; p < P; p += kStreamThreads) {
    const int e = a.ids[p];
    if (e >= 0 && e < E) pairs[atomicAdd(&cnt[e], 1)] = p;
  }
  __syncthreads();
  // zero outputs of out-of-range pairs
  const int nbad = s_bad;
  for (int i = 0; i < nbad; ++i) {
    const uint64_t o = (uint64_t)bad[i] * a.I;
    for (int r = tid; r < a.I; r += kStreamThreads) {
      a.out[o + r] = 0;
      if (a.gate_probe) a.gate_probe[o + r] = 0.0f;
      if (a.up_probe) a.up_probe[o + r] = 0.0f;
    }
  }
  if (tid == 0) hdr[0] = nbad;
}

template <int NT, int RW, int D, bool VEC>
__global__ __launch_bounds__(kStreamThreads, 4) void stream_kernel(const StreamParams a) {
  constexpr int G = (16 * NT) / 6;
  constexpr int ROWS = 16 * RW;
  constexpr int CMAX = 6 * G;
  constexpr int ITEMS = ROWS * G;                 // (row, token) results of one tile
  constexpr int IPL = (ITEMS + 63) / 64;          // items per lane
  __shared__ int32_t s_epi[kStreamThreads / 64][2][ROWS * CMAX];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, cc = lane & 15;
  const int w = blockIdx.x * (kStreamThreads / 64) + wave;
  const uint8_t* ws = a.ws;
  const int total_vt = ((const int32_t*)ws)[1];
  const int W = min(a.W, total_vt);
  if (w >= W) return;
  const int S = a.nsteps;
  const uint64_t U = (uint64_t)total_vt * S;
  const uint64_t u0 = (uint64_t)w * U / W, u1 = (uint64_t)(w + 1) * U / W;
  const int32_t* off = (const int32_t*)(ws + a.off_offset);
  const int32_t* vpre = (const int32_t*)(ws + a.off_vprefix);
  const int32_t* pairs = (const int32_t*)(ws + a.off_pairs);
  const int32_t* xmax = (const int32_t*)(ws + a.off_xmax);
  const uint8_t* digits = ws + a.off_digits;
  int32_t* fixc = (int32_t*)(ws + a.off_fixcnt);
  uint8_t* fixrec = (uint8_t*)ws + a.off_fixrec;
  const int H = a.H, I = a.I, E = a.num_slots;
  const uint32_t wbytes = (uint32_t)((uint64_t)I * (uint32_t)(H / 2));
  int32_t* eg = s_epi[wave][0];
  int32_t* eu = s_epi[wave][1];

  struct Stage {
    v4u ga[RW], ua[RW];
    v4i be[NT], bo[NT];
  };

  uint64_t u = u0;
  while (u < u1) {
    const int v = (int)(u / S);
    const int s0 = (int)(u - (uint64_t)v * S);
    const int s1 = (int)min((uint64_t)S, (uint64_t)s0 + (u1 - u));
    u += (uint64_t)(s1 - s0);
    // virtual tile -> slot (last e with vpre[e] <= v), token group, row tile
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (vpre[mid] <= v) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int r = v - vpre[e];
    const int gi = r / a.rtc;
    const int rt = r - gi * a.rtc;
    const int pbase = off[e] + gi * G;
    const int count = min(G, off[e + 1] - pbase);
    const int C = 6 * count;
    const int ntiles = (C + 15) >> 4;

    // B operand: lane (g4, cc) of tile n reads column 16n+cc (clamped to C-1):
    // digit (col % 6) of token (col / 6), 16 bytes per (step, parity, g4).
    const uint8_t* bptr[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int col = min(16 * n + cc, C - 1);
      const int ti = col / 6;
      const int tok = pairs[pbase + ti] / a.K;
      bptr[n] = digits + (uint64_t)tok * a.tok_stride + g4 * 96 + (col - 6 * ti) * 16;
    }
    const uint8_t* slot = a.slots + (uint64_t)e * a.slot_stride;
    const __amdgpu_buffer_rsrc_t gsrc = make_rsrc(slot + a.gate_w_off, wbytes);
    const __amdgpu_buffer_rsrc_t usrc = make_rsrc(slot + a.up_w_off, wbytes);
    uint32_t row_off[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      const int row = rt * ROWS + q * 16 + cc;
      row_off[q] = (uint32_t)(row < I ? row : I - 1) * (uint32_t)(H / 2) + (uint32_t)(g4 * 16);
    }

    v4i accg[RW][NT], accu[RW][NT];
#pragma unroll
    for (int q = 0; q < RW; ++q)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        accg[q][n] = v4i{0, 0, 0, 0};
        accu[q][n] = v4i{0, 0, 0, 0};
      }

    auto load_stage = [&](Stage& st, int s) {
      const uint32_t soff = (uint32_t)s * 64u;
#pragma unroll
      for (int q = 0; q < RW; ++q) {
        st.ga[q] = load16<VEC>(gsrc, row_off[q] + soff);
        st.ua[q] = load16<VEC>(usrc, row_off[q] + soff);
      }
      const uint64_t boff = (uint64_t)s * kDigitStepBytes;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (n < ntiles) {
          st.be[n] = *(const v4i*)(bptr[n] + boff);
          st.bo[n] = *(const v4i*)(bptr[n] + boff + 384);
        }
      }
    };
    auto compute = [&](const Stage& st) {
#pragma unroll
      for (int q = 0; q < RW; ++q) {
        v4i ge, go, ue, uo;
        split_weights(st.ga[q], ge, go);
        split_weights(st.ua[q], ue, uo);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          if (n < ntiles) {
            accg[q][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ge, st.be[n], accg[q][n], 0, 0, 0);
            accu[q][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ue, st.be[n], accu[q][n], 0, 0, 0);
            accg[q][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(go, st.bo[n], accg[q][n], 0, 0, 0);
            accu[q][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(uo, st.bo[n], accu[q][n], 0, 0, 0);
          }
        }
      }
    };

    Stage R[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (s0 + d < s1) load_stage(R[d], s0 + d);
    for (int s = s0; s < s1; s += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (s + d < s1) {
          compute(R[d]);
          if (s + d + D < s1) load_stage(R[d], s + d + D);
        }
      }
    }

    // ---- digit matrix of this wave's tile, then per (row, token) int64 sums ----
#pragma unroll
    for (int q = 0; q < RW; ++q)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int col = 16 * n + cc;
        if (col < C) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = q * 16 + 4 * g4 + i;
            eg[row * C + col] = accg[q][n][i];
            eu[row * C + col] = accu[q][n][i];
          }
        }
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int64_t sums[IPL][4];
#pragma unroll
    for (int k = 0; k < IPL; ++k) {
      const int item = lane + 64 * k;
      const int rr = item % ROWS, ti = item / ROWS;
      sums[k][0] = sums[k][1] = sums[k][2] = sums[k][3] = 0;
      if (ti < count) {
        const int32_t* gd = eg + rr * C + ti * 6;
        const int32_t* ud = eu + rr * C + ti * 6;
        sums[k][0] = (int64_t)gd[0] + ((int64_t)gd[1] << 8) + ((int64_t)gd[2] << 16);
        sums[k][1] = (int64_t)gd[3] + ((int64_t)gd[4] << 8) + ((int64_t)gd[5] << 16);
        sums[k][2] = (int64_t)ud[0] + ((int64_t)ud[1] << 8) + ((int64_t)ud[2] << 16);
        sums[k][3] = (int64_t)ud[3] + ((int64_t)ud[4] << 8) + ((int64_t)ud[5] << 16);
      }
    }
    __builtin_amdgcn_wave_barrier();   // LDS reads done before the next tile's writes

    bool finish = (s0 == 0 && s1 == S);
    if (!finish) {
      // two contributors: the left one ends at s1 < S (boundary w), the right
      // one starts at s0 > 0 (boundary w-1)
      const int side = s0 > 0 ? 1 : 0;
      const int b = side ? w - 1 : w;
      int64_t* mine = (int64_t*)(fixrec + ((uint64_t)b * 2 + side) * a.rec_bytes);
      const int64_t* other = (const int64_t*)(fixrec + ((uint64_t)b * 2 + (1 - side)) * a.rec_bytes);
#pragma unroll
      for (int k = 0; k < IPL; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) mine[(k * 4 + j) * 64 + lane] = sums[k][j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      int prev = 0;
      if (lane == 0) prev = __hip_atomic_fetch_add(&fixc[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __shfl(prev, 0);
      if (prev == 1) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
        for (int k = 0; k < IPL; ++k)
#pragma unroll
          for (int j = 0; j < 4; ++j) sums[k][j] += __builtin_nontemporal_load(&other[(k * 4 + j) * 64 + lane]);
        finish = true;
      }
    }
    if (finish) {
      const float* gscale = (const float*)(slot + a.gate_s_off);
      const float* uscale = (const float*)(slot + a.up_s_off);
#pragma unroll
      for (int k = 0; k < IPL; ++k) {
        const int item = lane + 64 * k;
        const int rr = item % ROWS, ti = item / ROWS;
        const int row = rt * ROWS + rr;
        if (ti < count && row < I) {
          const int p = pairs[pbase + ti];
          const int xm = xmax[p / a.K];
          const int e2 = sum_exponent(xm);
          float gate = round_scaled(sums[k][1], sums[k][0], e2, gscale[row]);
          float up = round_scaled(sums[k][3], sums[k][2], e2, uscale[row]);
          if (xm >= 0x7F80) {
            gate = __builtin_nanf("");
            up = __builtin_nanf("");
          }
          const uint64_t o = (uint64_t)p * I + row;
          a.out[o] = swiglu_tail(gate, up);
          if (a.gate_probe) a.gate_probe[o] = gate;
          if (a.up_probe) a.up_probe[o] = up;
        }
      }
    }
  }
}

// ---- host side ----

template <int NT, int RW, int D, bool VEC>
static int waves_for(int device) {
  static int cached[64] = {0};
  if (device < 0 || device >= 64) device = 0;
  if (!cached[device]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&stream_kernel<NT, RW, D, VEC>), kStreamThreads, 0) !=
            hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    cached[device] = cus * per_cu * (kStreamThreads / 64);
  }
  return cached[device];
}

StreamPlan plan_stream(int M, int K, int H, int I, int num_slots) {
  StreamPlan sp;
  sp.nt = M <= 2 ? 1 : (M <= 5 ? 2 : 3);
  sp.g = (16 * sp.nt) / 6;
  sp.rw = 2;
  sp.d = sp.nt == 1 ? 3 : 2;
  sp.vec = (H % 32) == 0;
  sp.nsteps = (H + 127) / 128;
  sp.rtc = (I + 16 * sp.rw - 1) / (16 * sp.rw);
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
#define Q4_WAVES(NT_, D_)                                                                   \
  (sp.vec ? waves_for<NT_, 2, D_, true>(device) : waves_for<NT_, 2, D_, false>(device))
  sp.waves = sp.nt == 1 ? Q4_WAVES(1, 3) : (sp.nt == 2 ? Q4_WAVES(2, 2) : Q4_WAVES(3, 2));
#undef Q4_WAVES
  const uint64_t P = (uint64_t)M * K;
  auto up256 = [](uint64_t n) { return (n + 255) / 256 * 256; };
  uint64_t o = 256;  // header: [0] invalid count, [1] virtual tiles
  sp.off_xmax = o;    o += up256(4ull * M);
  sp.off_count = o;   o += up256(4ull * num_slots);
  sp.off_offset = o;  o += up256(4ull * (num_slots + 1));
  sp.off_vprefix = o; o += up256(4ull * (num_slots + 1));
  sp.off_pairs = o;   o += up256(4 * P);
  sp.off_bad = o;     o += up256(4 * P);
  sp.off_fixcnt = o;  o += up256(4ull * sp.waves);
  const int items = 16 * sp.rw * sp.g;
  sp.rec_bytes = (uint32_t)(((items + 63) / 64) * 64 * 4 * 8);
  sp.off_fixrec = o;  o += up256((uint64_t)sp.waves * 2 * sp.rec_bytes);
  sp.tok_stride = (uint32_t)sp.nsteps * kDigitStepBytes;
  sp.off_digits = o;  o += up256((uint64_t)M * sp.tok_stride);
  sp.workspace = o;
  return sp;
}

template <int NT, int D, bool VEC>
static hipError_t launch_stream_t(const StreamParams& p, const StreamPlan& sp, hipStream_t stream) {
  StreamParams arg = p;
  void* args[] = {&arg};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&prep_kernel), dim3((unsigned)p.M + 1),
                                 dim3(kStreamThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(sp.waves / (kStreamThreads / 64));
  return hipLaunchKernel(reinterpret_cast<const void*>(&stream_kernel<NT, 2, D, VEC>), dim3(grid),
                         dim3(kStreamThreads), args, 0, stream);
}

hipError_t launch_stream(const StreamParams& p, const StreamPlan& sp, hipStream_t stream) {
  if (sp.nt == 1) return sp.vec ? launch_stream_t<1, 3, true>(p, sp, stream) : launch_stream_t<1, 3, false>(p, sp, stream);
  if (sp.nt == 2) return sp.vec ? launch_stream_t<2, 2, true>(p, sp, stream) : launch_stream_t<2, 2, false>(p, sp, stream);
  return sp.vec ? launch_stream_t<3, 2, true>(p, sp, stream) : launch_stream_t<3, 2, false>(p, sp, stream);
}

}  // namespace q4
