// Q4 gate/up + SwiGLU for narrow token sets (decode and verify widths): the
// digits of every token of the call stay resident in LDS for the launch.
//
// Arithmetic: GATE_UP_SOURCE of the @mlx-bun/inference 1.0.0 diff, page 52
// (kernels/glm52/streamed-experts.ts), made exact as in q4moe_device.h.
//
// Digit columns: each token of a pass owns W adjacent columns of the MFMA B
// operand, W = 4 when every token of the call allows four digits per value
// (digits_for) and W = 8 otherwise, laid out [d0 d1 d2 0 d3 d4 d5 0].  Either
// way the digits of one (row, token) sum fill whole lane quads of the MFMA
// result and recombine with quad shuffles, without LDS.  NT 16-column tiles
// hold 16*NT/W tokens; a call with more tokens than that takes several passes
// over its weights (only with W = 8 and more than 16*NT/8 tokens).
//  * One persistent launch, one 8-wave work-group per CU: work-group b takes
//    the whole tiles [bT/NB, (b+1)T/NB) of the T = slots x tiles-per-slot tiles.
//  * Inside a work-group the (tile, K-step) units of a slot segment are cut
//    into eight wave ranges (multiples of D steps; the first wave of each
//    SIMD takes a little more, see wave_share).  Each wave streams its own
//    units with D K-steps of weights in flight in a register ring; the first
//    loads of a segment go out before its routing scan and, in the first
//    segment, before x is split.
//  * A tile cut by a wave boundary has several contributors; each adds its
//    exact quad sums into an LDS fix-up slot with LDS atomics and bumps the
//    slot's counter; the last one to arrive finishes the tile.  No wave waits
//    on another inside a segment.
//  * K-steps per tile are padded to a multiple of D; the padding steps meet
//    zero digits, so they add nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4moe_device.h"
#include "q4moe_launch.h"

namespace q4 {

namespace {

constexpr int kResWaves = 8;
constexpr int kResThreads = kResWaves * 64;
#ifndef Q4_RES_DEPTH
#define Q4_RES_DEPTH 4
#endif
// K-steps of weights in flight per wave (1, 2 or 4).
__host__ __device__ constexpr int res_depth(int nt, bool q8) { return (void)nt, (void)q8, Q4_RES_DEPTH; }
// K-steps per pass of the step loop: the B-fragment swizzle repeats every
// four steps, so four steps per pass keep its offsets fixed.
constexpr int kResU = 4;
constexpr int kResLds = 150 * 1024;        // digits, then the fix-up slots
constexpr int kResXRegs = 8;               // 16-byte chunks of x held per thread while splitting
constexpr int kResMaxTokens = 8;           // tokens per call
constexpr int kResMaxPairs = 16;           // routed pairs finished per pass over a slot
constexpr int kResFixSlots = kResWaves - 1;
constexpr int kResIdRegs = 4;              // routing ids held per thread (2048 pairs)

// One K-step of digits: [parity 2][column tile n][k-group g 4][16 x 16 bytes]
// ([plane 4][...] for wide steps).
// The 16-byte chunk of column c sits at position c ^ (4g + step % 4) of its
// k-group row, so that both the B-fragment reads (the sixteen lanes of one
// k-group read sixteen distinct chunks) and the digit stores of one wave
// (lanes spread over dwords, k-groups and four steps) hit distinct banks.
__host__ __device__ constexpr int res_step_bytes(int nt, int planes = 2) { return planes * nt * 1024; }
__host__ __device__ constexpr int res_chunk(int g, int c, int step) { return g * 16 + (c ^ (4 * g + (step & 3))); }
// One fix-up slot: int64 [tile][gate, up][lane] (quad sums).
__host__ __device__ constexpr int res_fix_words(int nt) { return nt * 2 * 64; }
// K-steps per tile, padded to whole passes of the step loop.
__host__ __device__ constexpr int res_steps(int H, int kps = 128) { return ((H + kps - 1) / kps + kResU - 1) / kResU * kResU; }
// Wide K-steps (256 packed nibbles per row, four operand planes) for one
// column tile of Q4 weights and bf16 activations: rows are read 128 bytes per
// step (measured: the same bytes stream ~3-6% faster than 64 bytes per step).
__host__ __device__ constexpr bool res_wide(int nt, bool q8, bool xf) { return (void)nt, !q8 && !xf; }
// Column tiles for a call of M tokens: one up to two tokens, else two.
__host__ __device__ constexpr int res_tiles(int M) { return M <= 2 ? 1 : 2; }

}  // namespace

// DOWN: the down projection (one matrix of a.I rows over a.H inputs; a tile is
// 32 rows, its first 16 taking the gate role and the next 16 the up role,
// each output rounded to bf16 on its own) instead of gate/up + SwiGLU.
// Q8: signed int8 weights, one byte per weight (else packed nibbles).
// XF: f32 activations and outputs (else bf16).
template <int NT, bool VEC, bool DOWN, bool Q8, bool XF>
__global__ __launch_bounds__(kResThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void resident_kernel(const GateUpParams a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kResLds];
  __shared__ int s_pairs[kResMaxPairs];
  __shared__ int s_ptok[kResMaxPairs];       // token of each pair, relative to the pass
  __shared__ int s_xmax[kResMaxTokens];
  __shared__ int s_xmin[kResMaxTokens];      // smallest non-zero exponent field of each token
  __shared__ int s_wcnt[kResWaves];
  __shared__ int s_fixcnt[kResFixSlots];
  __shared__ int s_bound[kResWaves + 1];     // unit ranges of the segment, by position
  __shared__ int s_invalid;
  __shared__ uint16_t s_sig[kSigTable];      // bf16 sigmoid of the tabulated gT

  constexpr int kResD = res_depth(NT, Q8);
  constexpr bool WIDE = res_wide(NT, Q8, XF);
  constexpr bool WL = Q8 || WIDE;            // 32 bytes per lane and step
  constexpr int NPL = WIDE ? 4 : 2;          // operand planes per step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, cc = lane & 15;
  const int H = a.H, I = a.I, M = a.M, K = a.K;
  const int P = M * K;
  const bool grouped = a.ids != nullptr;
  constexpr bool xf = XF;
  const int S = a.steps;                     // K-steps per tile, a multiple of D
  const int sbytes = res_step_bytes(NT, NPL);
  const int hw = H / 8;                      // 16-byte chunks of one token's x
  constexpr int RT = DOWN ? 32 : 16;         // rows per tile
  const int tps = (I + RT - 1) / RT;         // tiles per slot
  const int T = a.num_slots * tps;
  const int NB = gridDim.x;
  const int v0 = (int)((int64_t)blockIdx.x * T / NB), v1 = (int)((int64_t)(blockIdx.x + 1) * T / NB);
  const uint32_t rbytes = row_bytes<Q8>(H);  // bytes of one weight row
  const uint32_t wbytes = (uint32_t)((uint64_t)I * rbytes);
  const uint64_t below = (1ull << lane) - 1ull;
  unsigned long long* const s_fix = (unsigned long long*)(s_lds + S * sbytes);

  // routing ids of the first pairs, read once, before any weight load
  int idr[kResIdRegs];
#pragma unroll
  for (int j = 0; j < kResIdRegs; ++j) {
    const int p = tid + j * kResThreads;
    idr[j] = (grouped && p < P) ? a.ids[p] : -1;
  }

  if (tid < kResMaxTokens) {
    s_xmax[tid] = 0;
    s_xmin[tid] = 255;
  }
  if (tid == 0) s_invalid = 0;
  __syncthreads();

  // ---- invalid routing ids (grouped): zero-filled by work-group 0 ----
  if (grouped && blockIdx.x == 0) {
    int cnt = 0;
    for (int p = tid; p < P; p += kResThreads) {
      const int e = a.ids[p];
      if (e < 0 || e >= a.num_slots) {
        ++cnt;
        for (int r = 0; r < I; ++r) {
          const uint64_t o = (uint64_t)p * I + r;
          if (xf)
            ((float*)a.out)[o] = 0.0f;
          else
            a.out[o] = 0;
          if (a.gate_probe) a.gate_probe[o] = 0.0f;
          if (a.up_probe) a.up_probe[o] = 0.0f;
        }
      }
    }
    if (cnt) atomicAdd(&s_invalid, cnt);
    __syncthreads();
    if (tid == 0 && a.invalid_count) *a.invalid_count = s_invalid;
  }

  // ---- x of every token, loaded before any weight load ----
  uint4 xv[kResXRegs];
  const int nxc = M * hw;
#pragma unroll
  for (int j = 0; j < kResXRegs; ++j) {
    const int q = tid + j * kResThreads;
    xv[j] = (!xf && q < nxc) ? ((const uint4*)a.x)[q] : make_uint4(0, 0, 0, 0);
  }
  // chunk q (8 consecutive values) of f32 activations: two 16-byte loads
  auto xf_chunk = [&](int q, uint4& lo4, uint4& hi4) {
    const uint4* xp = (const uint4*)((const float*)a.x + 8 * (size_t)q);
    lo4 = xp[0];
    hi4 = xp[1];
  };

  // ---- the current slot segment: tiles [t0, t1) of slot e ----
  int v = v0;
  int e = 0, t0 = 0, t1 = 0, nunits = 0, ua = 0, ub = 0;
  __amdgpu_buffer_rsrc_t gsrc, usrc;
  const float* gscale = nullptr;
  const float* uscale = nullptr;
  // Unit range start of position k (0..8).  The units are cut into four equal
  // quarters, one per SIMD; quarter q goes to waves q (first on its SIMD,
  // which wins the SIMD's issue arbitration more often) and q + 4, the first
  // taking wave_share/1024.  Position k = 2*(wave % 4) + wave / 4 orders the
  // ranges by unit.
  auto bound = [&](int k) {
    if (k >= kResWaves) return nunits;
    const int q = k >> 1;
    const int qa = (int)(((int64_t)q * nunits / 4) / kResU * kResU);
    if (!(k & 1)) return qa;
    const int qb = q == 3 ? nunits : (int)(((int64_t)(q + 1) * nunits / 4) / kResU * kResU);
    return qa + (int)(((int64_t)(qb - qa) * a.wave_share / 1024) / kResU * kResU);
  };
  const int wpos = 2 * (wave & 3) + (wave >> 2);
  auto open_segment = [&]() {
    e = v / tps;
    t0 = v - e * tps;
    t1 = min(v1, (e + 1) * tps) - e * tps;
    v = e * tps + t1;
    const uint8_t* slot = a.slots + (uint64_t)e * a.slot_stride;
    gsrc = make_rsrc(slot + a.gate_w_off, wbytes);
    if constexpr (DOWN) {
      // rows 16..31 of each tile: the same matrix 16 rows further on (loads
      // past its end return zeros, for rows that are never stored)
      const uint32_t skip = 16u * rbytes;
      usrc = make_rsrc(slot + a.gate_w_off + skip, wbytes > skip ? wbytes - skip : 0u);
    } else {
      usrc = make_rsrc(slot + a.up_w_off, wbytes);
    }
    gscale = (const float*)(slot + a.gate_s_off);
    uscale = (const float*)(slot + a.up_s_off);
    nunits = (t1 - t0) * S;
    ua = bound(wpos);
    ub = bound(wpos + 1);
  };

  auto row_off = [&](int tile) {
    const int row = tile * RT + cc;
    return (uint32_t)(row < I ? row : I - 1) * rbytes + (uint32_t)g4 * group_bytes<WL>();
  };
  StepW<WL> rg[kResD], ru[kResD];
  int lt = 0, ls = 0;                        // load cursor (tile, step)
  uint32_t loff = 0;
  auto issue = [&](StepW<WL>& g, StepW<WL>& u_, bool live, uint32_t dep = 0u) {
    const uint32_t o = (live ? loff + (uint32_t)ls * step_row_bytes<WL>() : kOffNone) + dep;
    load_step<WL, VEC>(g, gsrc, o);
    load_step<WL, VEC>(u_, usrc, o);
    // cursor step without branches, so the loads stay unconditional
    const int nls = ls + (live ? 1 : 0);
    const bool wrap = nls == S;
    ls = wrap ? 0 : nls;
    lt += wrap ? 1 : 0;
    loff = wrap ? row_off(lt) : loff;
  };
  // The ring always holds D loads per array: slots past the wave's range
  // load nothing (kOffNone) and are never consumed.
  auto start_ring = [&]() {
    lt = t0 + ua / S;
    ls = ua % S;
    loff = row_off(lt);
#pragma unroll
    for (int d = 0; d < kResD; ++d) issue(rg[d], ru[d], ua + d < ub);
  };

  // digits per value and columns per token, fixed once x has been read
  int L = 6, W = 8;
  auto etop = [&](int m) { return xf ? max((s_xmax[m] >> 23) & 0xFF, 1) : max((s_xmax[m] >> 7) & 0xFF, 1); };
  // digits of chunk w8 (8 consecutive K values) of pass token tl
  auto stage_unit4 = [&](int tl, int w8, const uint4 xq, int etop1) {
    const int st = w8 >> 4, gg = (w8 >> 2) & 3, i = w8 & 3;
    {
      uint32_t d[2][4];
      x8_digits4(xq, etop1, d);
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        uint8_t* base = s_lds + st * sbytes + par * NT * 1024 + 4 * i;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int col = tl * 4 + s;
          *(uint32_t*)(base + (col >> 4) * 1024 + res_chunk(gg, col & 15, st) * 16) = d[par][s];
        }
      }
    }
  };
  auto stage_unit8 = [&](int tl, int w8, const uint4 xq, int etop1) {
    const int st = w8 >> 4, gg = (w8 >> 2) & 3, i = w8 & 3;
    uint32_t lo[8], hi[8];
    x8_digits(xq, etop1, lo, hi);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      uint32_t d[6];
      digit_words(lo, hi, par, d);
      uint8_t* base = s_lds + st * sbytes + par * NT * 1024 + 4 * i;
      auto put = [&](int col, uint32_t w) {
        *(uint32_t*)(base + (col >> 4) * 1024 + res_chunk(gg, col & 15, st) * 16) = w;
      };
      put(tl * 8 + 0, d[0]);
      put(tl * 8 + 1, d[1]);
      put(tl * 8 + 2, d[2]);
      put(tl * 8 + 3, 0u);
      put(tl * 8 + 4, d[3]);
      put(tl * 8 + 5, d[4]);
      put(tl * 8 + 6, d[5]);
      put(tl * 8 + 7, 0u);
    }
  };
  // eight digits of eight f32 activations: all eight columns of the token
  auto stage_unitf = [&](int tl, int w8, const uint4 xa, const uint4 xb, int etop1) {
    const int st = w8 >> 4, gg = (w8 >> 2) & 3, i = w8 & 3;
    uint32_t d[2][8];
    xf8_digits(xa, xb, etop1, d);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      uint8_t* base = s_lds + st * sbytes + par * NT * 1024 + 4 * i;
#pragma unroll
      for (int sd = 0; sd < 8; ++sd) {
        const int col = tl * 8 + sd;
        *(uint32_t*)(base + (col >> 4) * 1024 + res_chunk(gg, col & 15, st) * 16) = d[par][sd];
      }
    }
  };
  auto stage_unit = [&](int tl, int w8, const uint4 xq, int etop1) {
    if (W == 4)
      stage_unit4(tl, w8, xq, etop1);
    else
      stage_unit8(tl, w8, xq, etop1);
  };
  // wide steps: digits of unit pair r (units 2r, 2r+1: words 2i, 2i+1 of k-group
  // g of step st) of pass token tl, one dword per plane and digit column
  auto stage_pair = [&](int tl, int r, const uint4 xa, const uint4 xb, int etop1) {
    const int st = r >> 4, gg = (r >> 2) & 3, i = r & 3;
    uint8_t* base = s_lds + st * sbytes + 4 * i;
    auto put = [&](int j, int col, uint32_t v) {
      *(uint32_t*)(base + (j * NT + (col >> 4)) * 1024 + res_chunk(gg, col & 15, st) * 16) = v;
    };
    const uint32_t xs[2][8] = {{xa.x & 0xFFFFu, xa.x >> 16, xa.y & 0xFFFFu, xa.y >> 16, xa.z & 0xFFFFu, xa.z >> 16,
                                xa.w & 0xFFFFu, xa.w >> 16},
                               {xb.x & 0xFFFFu, xb.x >> 16, xb.y & 0xFFFFu, xb.y >> 16, xb.z & 0xFFFFu, xb.z >> 16,
                                xb.w & 0xFFFFu, xb.w >> 16}};
    uint32_t v0[8], v1[8], d[4][4];
    if (W == 4) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        v0[p] = x_digits4(xs[0][p], etop1);
        v1[p] = x_digits4(xs[1][p], etop1);
      }
      plane_words4(v0, v1, d);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int sd = 0; sd < 4; ++sd) put(j, tl * 4 + sd, d[j][sd]);
      return;
    }
    // six digits: columns [d0 d1 d2 0 d3 d4 d5 0]
    uint32_t h0[8], h1[8], e[4][4];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint64_t z0 = x_digits(xs[0][p], etop1), z1 = x_digits(xs[1][p], etop1);
      v0[p] = (uint32_t)z0;
      h0[p] = (uint32_t)(z0 >> 32);
      v1[p] = (uint32_t)z1;
      h1[p] = (uint32_t)(z1 >> 32);
    }
    plane_words4(v0, v1, d);
    plane_words4(h0, h1, e);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      put(j, tl * 8 + 0, d[j][0]);
      put(j, tl * 8 + 1, d[j][1]);
      put(j, tl * 8 + 2, d[j][2]);
      put(j, tl * 8 + 3, 0u);
      put(j, tl * 8 + 4, d[j][3]);
      put(j, tl * 8 + 5, e[j][0]);
      put(j, tl * 8 + 6, e[j][1]);
      put(j, tl * 8 + 7, 0u);
    }
  };

  // ---- the digits of the first pass, then the first segment's weights in flight ----
  // (x is split before any weight load is issued: a load issued after the ring,
  // such as a rematerialised x chunk, would wait for the whole ring to arrive)
  // largest |x| and smallest non-zero exponent of each token.  When a token's
  // chunks fill whole waves (hw % 64 == 0), each wave's 64 chunks of x
  // register j belong to one token: the sixteen wave reductions (DPP, no
  // branches, so the scheduler interleaves them) go to lane 0, which posts
  // them; otherwise every lane posts its own values.
  if (xf) {
    // f32: a rolled loop over the chunks, wave reductions when a wave's
    // chunks belong to one token
#pragma unroll 1
    for (int q = tid; q < (nxc + 63) / 64 * 64; q += kResThreads) {
      uint32_t mx = 0, mn = 255;
      if (q < nxc) {
        uint4 xa, xb;
        xf_chunk(q, xa, xb);
        f32_range8(xa, xb, mx, mn);
      }
      if (hw % 64 == 0) {
        mx = wave_extreme<true>(mx);
        mn = wave_extreme<false>(mn);
        if (lane == 0 && q < nxc) {
          const int m = q / hw;
          if (mx) atomicMax(&s_xmax[m], (int)mx);
          if (mn < 255) atomicMin(&s_xmin[m], (int)mn);
        }
      } else if (q < nxc) {
        const int m = q / hw;
        if (mx) atomicMax(&s_xmax[m], (int)mx);
        if (mn < 255) atomicMin(&s_xmin[m], (int)mn);
      }
    }
  } else {
    // registers past the last chunk in every lane (j * threads >= nxc, the
    // same for the whole work-group) are skipped; lanes past it hold zeros,
    // whose range (0, 255) posts nothing
#pragma unroll
    for (int j = 0; j < kResXRegs; ++j) {
      if (j * kResThreads < nxc) {
        uint32_t mx, mn;
        range8(xv[j], mx, mn);
        if (hw % 64 == 0) {
          mx = wave_extreme<true>(mx);
          mn = wave_extreme<false>(mn);
          const int q0 = j * kResThreads + (tid & ~63);
          if (lane == 0 && q0 < nxc) {
            const int m = q0 / hw;
            if (mx) atomicMax(&s_xmax[m], (int)mx);
            if (mn < 255) atomicMin(&s_xmin[m], (int)mn);
          }
        } else {
          const int q = tid + j * kResThreads;
          if (q < nxc) {
            const int m = q / hw;
            if (mx) atomicMax(&s_xmax[m], (int)mx);
            if (mn < 255) atomicMin(&s_xmin[m], (int)mn);
          }
        }
      }
    }
  }
  __syncthreads();
  {
    int l = 4;
    for (int m = 0; m < M; ++m) l = max(l, digits_for(s_xmax[m], s_xmin[m]));
    L = xf ? 8 : __builtin_amdgcn_readfirstlane(l);
  }
  W = L == 4 ? 4 : 8;
  const int tpp = 16 * NT / W;                              // tokens per pass
  const int npass = (M + tpp - 1) / tpp;
  if constexpr (WIDE) {
    // wide steps: unit pairs (16 values, one dword of every plane and digit
    // column) over the whole padded K range, so the padding gets zero digits
    const int ntok = min(M, tpp);
    const int npair = S * 16;
    // up to four pairs per thread and pass of this loop, their loads issued
    // together (one round trip instead of four)
    constexpr int kPairs = 4;
#pragma unroll 1
    for (int u0 = tid; u0 < ntok * npair; u0 += kPairs * kResThreads) {
      uint4 xa[kPairs], xb[kPairs];
#pragma unroll
      for (int k = 0; k < kPairs; ++k) {
        const int u = u0 + k * kResThreads;
        const int m = u / npair, w8 = 2 * (u - m * npair);
        const bool live = u < ntok * npair;
        xa[k] = (live && w8 < hw) ? ((const uint4*)a.x)[m * hw + w8] : make_uint4(0, 0, 0, 0);
        xb[k] = (live && w8 + 1 < hw) ? ((const uint4*)a.x)[m * hw + w8 + 1] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < kPairs; ++k) {
        const int u = u0 + k * kResThreads;
        if (u < ntok * npair) {
          const int m = u / npair;
          stage_pair(m, u - m * npair, xa[k], xb[k], etop(m));
        }
      }
    }
  } else {
    const int ntok = min(M, tpp);
    // a rolled loop that reads x again (cache hits: no weight load is in
    // flight yet), the next chunk's load in flight: the launch's setup runs
    // once per work-group, so its straight-line code is fetched cold
    const int nq = ntok * hw;
    int q = tid;
    uint4 xq = (!xf && q < nq) ? ((const uint4*)a.x)[q] : make_uint4(0, 0, 0, 0);
    if (xf) {
#pragma unroll 1
      for (; q < nq; q += kResThreads) {
        uint4 xa, xb;
        xf_chunk(q, xa, xb);
        const int m = q / hw;
        stage_unitf(m, q - m * hw, xa, xb, etop(m));
      }
    } else if (W == 4) {
#pragma unroll 1
      for (; q < nq; q += kResThreads) {
        const int qn = q + kResThreads;
        const uint4 xn = qn < nq ? ((const uint4*)a.x)[qn] : make_uint4(0, 0, 0, 0);
        const int m = q / hw;
        stage_unit4(m, q - m * hw, xq, etop(m));
        xq = xn;
      }
    } else {
#pragma unroll 1
      for (; q < nq; q += kResThreads) {
        const int qn = q + kResThreads;
        const uint4 xn = qn < nq ? ((const uint4*)a.x)[qn] : make_uint4(0, 0, 0, 0);
        const int m = q / hw;
        stage_unit8(m, q - m * hw, xq, etop(m));
        xq = xn;
      }
    }
    // zero digits for the padding steps
    const int padw = S * 16 - hw;
    for (int u = tid; u < ntok * padw; u += kResThreads) {
      if (xf)
        stage_unitf(u % ntok, hw + u / ntok, make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), 1);
      else
        stage_unit(u % ntok, hw + u / ntok, make_uint4(0, 0, 0, 0), 1);
    }
  }
  open_segment();
  start_ring();
  // the sigmoid table while the first weights are on their way
  if constexpr (!DOWN)
    for (int i = tid; i < kSigTable; i += kResThreads) s_sig[i] = sigmoid_bf16(sig_table_bits(i));

  // exact (row, token) sum of the four digit columns of a lane quad: lane j
  // of the quad receives row 4*g4 + j (transposing quad reduction)
  const int qj = cc & 3;
  auto quad_row_sum = [&](const v4i acc) {
    const int64_t w0 = (int64_t)acc[0] << (8 * qj), w1 = (int64_t)acc[1] << (8 * qj);
    const int64_t w2 = (int64_t)acc[2] << (8 * qj), w3 = (int64_t)acc[3] << (8 * qj);
    const bool up2 = (qj & 2) != 0;
    const int64_t r0 = quad_xor<2>(up2 ? w0 : w2), r1 = quad_xor<2>(up2 ? w1 : w3);
    const int64_t k0 = (up2 ? w2 : w0) + r0, k1 = (up2 ? w3 : w1) + r1;  // rows (qj&2), (qj&2)+1
    const int64_t r = quad_xor<1>((qj & 1) ? k0 : k1);
    return ((qj & 1) ? k1 : k0) + r;
  };
  // this lane's B-fragment chunk for steps 0..3 mod 4
  static_assert(kResU % kResD == 0, "the step loop's pass covers whole turns of the ring");
  int rdo[kResU];
#pragma unroll
  for (int j = 0; j < kResU; ++j) rdo[j] = res_chunk(g4, cc, j) * 16;

  for (int pass = 0;;) {
    const int tp0 = pass * tpp;                             // first token of the pass
    const int tp1 = min(M, tp0 + tpp);                      // end token
    const int pend = tp1 * K;                               // end pair
    int next_pair = tp0 * K;
    bool first_group = true;
    // the pass token of this lane's quad in each column tile, and its exponent
    int ltok[NT], lxm[NT];
    bool lok[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      ltok[n] = W == 4 ? 4 * n + (cc >> 2) : 2 * n + (cc >> 3);
      lok[n] = (W == 4 || (cc & 4) == 0) && ltok[n] < tp1 - tp0;
      lxm[n] = lok[n] ? s_xmax[tp0 + ltok[n]] : 0;
    }
    for (;;) {
      __syncthreads();  // previous group done with the fix-up slots, s_bound and s_pairs; digits visible
      if (tid < kResFixSlots) s_fixcnt[tid] = 0;
      if (tid <= kResWaves) s_bound[tid] = bound(tid);
      for (int i = tid; i < kResFixSlots * res_fix_words(NT); i += kResThreads) s_fix[i] = 0;

      // ---- next group of up to kResMaxPairs pairs of the pass routed to slot e ----
      int count, more;
      if (!grouped) {
        count = min(kResMaxPairs, pend - next_pair);
        more = next_pair + count < pend;
        if (tid < count) {
          s_pairs[tid] = next_pair + tid;
          s_ptok[tid] = next_pair + tid - tp0;               // K == 1
        }
        __syncthreads();  // s_pairs, s_bound and the cleared fix-up slots visible
      } else {
        // block-wide scan of ids[next_pair..pend) in aligned windows of
        // kResThreads (the first kResIdRegs from registers); stops once a
        // further match proves there is another group
        int found = 0;
        int base = next_pair & ~(kResThreads - 1);
        more = 0;
        for (;;) {
          const int p = base + tid;
          const int k = base / kResThreads;
          int id;
          if (k < kResIdRegs) {
            id = k == 0 ? idr[0] : k == 1 ? idr[1] : k == 2 ? idr[2] : idr[3];
          } else {
            id = p < P ? a.ids[p] : -1;
            // This load completes after the ring issued before it in any
            // case.  Waiting here, on this path alone, keeps the compiler
            // from placing a wait for every load in flight (the whole ring)
            // on the register path too, where the merged id is used.
            __builtin_amdgcn_s_waitcnt(kWaitVmem0);
          }
          const bool m = id == e && p >= next_pair && p < pend;
          const uint64_t bal = __ballot(m);
          if (lane == 0) s_wcnt[wave] = __popcll(bal);
          __syncthreads();
          int before = found, total = found;
#pragma unroll
          for (int w = 0; w < kResWaves; ++w) {
            const int c = s_wcnt[w];
            if (w < wave) before += c;
            total += c;
          }
          before += __popcll(bal & below);
          if (m && before < kResMaxPairs) {
            s_pairs[before] = p;
            s_ptok[before] = p / K - tp0;
          }
          found = total;
          base += kResThreads;
          if (found > kResMaxPairs) more = 1;
          __syncthreads();  // s_wcnt reused; s_pairs visible
          if (more || base >= pend) break;
        }
        count = min(found, kResMaxPairs);
      }
      if (count <= 0) break;
      next_pair = s_pairs[count - 1] + 1;
      // the group's pairs and their pass tokens, uniform: held in scalar registers
      int gpair[kResMaxPairs], gtok[kResMaxPairs];
#pragma unroll
      for (int q = 0; q < kResMaxPairs; ++q) {
        gpair[q] = __builtin_amdgcn_readfirstlane(q < count ? s_pairs[q] : 0);
        gtok[q] = __builtin_amdgcn_readfirstlane(q < count ? s_ptok[q] : -1);
      }
      // the pair of this lane's token in each column tile when it has exactly
      // one in the group (-1: none); several pairs of one token take the loop
      int mypair[NT];
      bool multi = false;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        int mp = -1;
        for (int q = 0; q < count; ++q)
          if (gtok[q] == ltok[n]) mp = mp == -1 ? gpair[q] : -2;   // -2: two or more
        mypair[n] = mp;
        multi = multi || __ballot(lok[n] && mp == -2) != 0;
      }
      if (!first_group) start_ring();
      first_group = false;

      int u = ua;
      while (u < ub) {
        // one portion: the rest of the current tile inside [u, ub)
        const int tile = t0 + u / S;
        const int sa = u % S;
        const int pe = min(ub, (u / S + 1) * S);              // portion end (unit)
        // the row scales this lane may finish with, loaded ahead of the
        // portion's weight loads: loads complete in order, so a scale load
        // issued at the finish would wait for every weight load in flight
        const int row = tile * RT + 4 * g4 + qj;
        const float gsc = gscale[min(row, I - 1)];
        const float usc = DOWN ? gscale[min(row + 16, I - 1)] : uscale[min(row, I - 1)];
        float gscr = 0.0f, uscr = 0.0f;
        v4i accg[NT], accu[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          accg[n] = v4i{0, 0, 0, 0};
          accu[n] = v4i{0, 0, 0, 0};
        }
        int s = sa;                                           // a multiple of 4: (s + j) % 4 == j
        for (; u < pe; u += kResU) {
#pragma unroll
          for (int j = 0; j < kResU; ++j) {
            const int d = j % kResD;                          // ring slot of step s + j
            v4i pg[NPL], pu[NPL];
            if constexpr (WIDE) {
              split_planes(rg[d].a, rg[d].b, pg);
              split_planes(ru[d].a, ru[d].b, pu);
            } else {
              split_step(rg[d], pg[0], pg[1]);
              split_step(ru[d], pu[0], pu[1]);
            }
            // The slot's registers are free once split: refill it before the
            // multiply.  The refill's offset passes through an empty asm that
            // takes the split planes, so the loads are issued after the split
            // has read the slot and can land in the slot's own registers.
            // Otherwise the compiler issues them early into other registers
            // and, at the loop's back edge, copies every slot back, waiting
            // for all loads in flight each pass.
            uint32_t dep = 0u;
            if constexpr (!XF) {
#pragma unroll
              for (int pl = 0; pl < NPL; ++pl) asm volatile("" : "+v"(dep) : "v"(pg[pl]), "v"(pu[pl]));
            }
            issue(rg[d], ru[d], u + j + kResD < ub, dep);
            const uint8_t* bp = s_lds + (s + j) * sbytes + rdo[j];
            v4i bq[NPL][NT];
#pragma unroll
            for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
              for (int n = 0; n < NT; ++n) bq[pl][n] = *(const v4i*)(bp + (pl * NT + n) * 1024);
#pragma unroll
            for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
              for (int n = 0; n < NT; ++n) {
                accg[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pg[pl], bq[pl][n], accg[n], 0, 0, 0);
                accu[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pu[pl], bq[pl][n], accu[n], 0, 0, 0);
              }
          }
          s += kResU;
          // take the row scales over here, where the compiler counts the
          // weight loads issued after them exactly (left to the finish, the
          // wait for them covers every load in flight)
          __asm__ volatile("v_mov_b32 %0, %2\n\tv_mov_b32 %1, %3" : "=v"(gscr), "=v"(uscr) : "v"(gsc), "v"(usc));
        }
        const int se = s;                                     // portion covers steps [sa, se)

        int64_t gq[NT], uq[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          gq[n] = quad_row_sum(accg[n]);
          uq[n] = quad_row_sum(accu[n]);
        }
        bool finish = (sa == 0 && se == S);
        if (!finish) {
          // contributors of this tile: ranges that meet its units, by position
          const int tu0 = (tile - t0) * S, tu1 = tu0 + S;
          int first = -1, ncontrib = 0;
          for (int k = 0; k < kResWaves; ++k) {
            const int qa = s_bound[k], qb = s_bound[k + 1];
            if (qa < qb && qa < tu1 && qb > tu0) {
              if (first < 0) first = k;
              ++ncontrib;
            }
          }
          // first < kResFixSlots: the last range ends on a tile end
          unsigned long long* fx = s_fix + first * res_fix_words(NT) + lane;
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            atomicAdd(&fx[(2 * n) * 64], (unsigned long long)gq[n]);
            atomicAdd(&fx[(2 * n + 1) * 64], (unsigned long long)uq[n]);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          int prev = 0;
          if (lane == 0) prev = atomicAdd(&s_fixcnt[first], 1);
          prev = __shfl(prev, 0);
          if (prev == ncontrib - 1) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              gq[n] = (int64_t)fx[(2 * n) * 64];
              uq[n] = (int64_t)fx[(2 * n + 1) * 64];
            }
            finish = true;
          }
        }
        if (finish) {
          // ---- (row, token) sums, F32 rounding, SwiGLU tail, routed stores ----
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const int tl = ltok[n];
            int64_t ghi, glo, uhi, ulo;
            int e2off;
            if (W == 4) {
              // the quad holds digits 0..3 of one token
              ghi = gq[n] >> 24;
              glo = gq[n] & 0xFFFFFF;
              uhi = uq[n] >> 24;
              ulo = uq[n] & 0xFFFFFF;
              e2off = 16;
            } else {
              // quads [d0 d1 d2 0] and [d3 d4 d5 0]: the low half of the
              // sum, and its high half from the next quad
              const int64_t gx = __shfl_xor(gq[n], 4), ux = __shfl_xor(uq[n], 4);
              glo = gq[n];
              ghi = gx;
              ulo = uq[n];
              uhi = ux;
              e2off = 0;
            }
            const bool ok = lok[n] && row < I;
            float gate = 0.0f, up = 0.0f, ovf = 0.0f;
            uint16_t ov = 0;
            if (ok) {
              const int xm = lxm[n];
              if (xf) {
                // eight digits: quads [d0..d3] and [d4..d7], V = hi * 2^32 + lo
                const int e2 = sum_exponent_f32((uint32_t)xm) + weight_exp_shift<Q8>();
                gate = round_scaled_wide(ghi, glo, e2, gscr);
                up = round_scaled_wide(uhi, ulo, e2, uscr);
                if ((uint32_t)xm >= 0x7F800000u) {
                  gate = __builtin_nanf("");
                  up = __builtin_nanf("");
                }
                if constexpr (!DOWN) ovf = swiglu_tail_f32(gate, up);
              } else {
                const int e2 = sum_exponent(xm) + e2off + weight_exp_shift<Q8>();
                if (W == 4) {
                  gate = round_scaled53(gq[n], e2, gscr);
                  up = round_scaled53(uq[n], e2, uscr);
                } else {
                  gate = round_scaled(ghi, glo, e2, gscr);
                  up = round_scaled(uhi, ulo, e2, uscr);
                }
                if (xm >= 0x7F80) {
                  gate = __builtin_nanf("");
                  up = __builtin_nanf("");
                }
                if constexpr (!DOWN) ov = swiglu_tail_tab(gate, up, s_sig);
              }
            }
            // results of this (row, token) for routed pair `pair`
            auto store = [&](int pair) {
              const uint64_t o = (uint64_t)pair * I + row;
              float* const outf = (float*)a.out;
              if constexpr (DOWN) {
                // rows `row` and `row + 16`, each its own output
                if (xf)
                  outf[o] = gate;
                else
                  a.out[o] = bf16_rne(gate);
                if (a.gate_probe) a.gate_probe[o] = gate;
                if (row + 16 < I) {
                  if (xf)
                    outf[o + 16] = up;
                  else
                    a.out[o + 16] = bf16_rne(up);
                  if (a.gate_probe) a.gate_probe[o + 16] = up;
                }
              } else {
                if (xf)
                  outf[o] = ovf;
                else
                  a.out[o] = ov;
                if (a.gate_probe) a.gate_probe[o] = gate;
                if (a.up_probe) a.up_probe[o] = up;
              }
            };
            if (!multi) {
              if (ok && mypair[n] >= 0) store(mypair[n]);
            } else {
              for (int q = 0; q < count; ++q)
                if (ok && gtok[q] == tl) store(gpair[q]);
            }
          }
        }
      }
      if (!more) break;
    }

    // ---- next segment, or the next pass from the first segment ----
    if (v < v1) {
      open_segment();
      start_ring();
      continue;
    }
    if (++pass >= npass) break;
    __syncthreads();  // every wave is done with the previous pass's digits
    if constexpr (WIDE) {
      const int p0 = pass * tpp;
      const int ntok = min(M, p0 + tpp) - p0;
      const int npair = S * 16;
#pragma unroll 1
      for (int u = tid; u < ntok * npair; u += kResThreads) {
        const int tl = u / npair, r = u - tl * npair;
        const int w8 = 2 * r;
        const uint64_t xr = (uint64_t)(p0 + tl) * hw;
        const uint4 xa = w8 < hw ? ((const uint4*)a.x)[xr + w8] : make_uint4(0, 0, 0, 0);
        const uint4 xb = w8 + 1 < hw ? ((const uint4*)a.x)[xr + w8 + 1] : make_uint4(0, 0, 0, 0);
        stage_pair(tl, r, xa, xb, etop(p0 + tl));
      }
    } else {
      const int p0 = pass * tpp;
      const int ntok = min(M, p0 + tpp) - p0;
      for (int u = tid; u < ntok * S * 16; u += kResThreads) {
        const int tl = u % ntok, w8 = u / ntok;
        if (xf) {
          uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
          if (w8 < hw) xf_chunk((p0 + tl) * hw + w8, xa, xb);
          stage_unitf(tl, w8, xa, xb, etop(p0 + tl));
        } else {
          const uint4 xq = w8 < hw ? ((const uint4*)a.x)[(uint64_t)(p0 + tl) * hw + w8] : make_uint4(0, 0, 0, 0);
          stage_unit(tl, w8, xq, etop(p0 + tl));
        }
      }
    }
    v = v0;
    open_segment();
    start_ring();
  }
}

// ---- host side ----

namespace {

// Share of a SIMD's units for its first wave, in 1/1024, by column tiles
// (measured on MI355X: the first wave of a SIMD streams ~29% faster than the
// second with one column tile and ~14% faster with two).
constexpr int kWaveShare1 = 577;
constexpr int kWaveShare2 = 547;

// Work-groups that fit the device at once (one per CU: the LDS arrays take
// most of a CU's 160 KiB).
template <int NT, bool VEC, bool DOWN, bool Q8, bool XF>
int resident_blocks(int device) {
  static int cached[64] = {0};
  if (device < 0 || device >= 64) device = 0;
  if (!cached[device]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&resident_kernel<NT, VEC, DOWN, Q8, XF>), kResThreads, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    cached[device] = cus * per_cu;
  }
  return cached[device];
}

template <int NT, bool VEC, bool DOWN, bool Q8, bool XF>
hipError_t launch_resident_t(GateUpParams& p, hipStream_t stream) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  const int rt = DOWN ? 32 : 16;
  const int tiles = p.num_slots * ((p.I + rt - 1) / rt);
  int nb = resident_blocks<NT, VEC, DOWN, Q8, XF>(device);
  if (nb > tiles) nb = tiles;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&resident_kernel<NT, VEC, DOWN, Q8, XF>), dim3((unsigned)nb),
                         dim3(kResThreads), args, 0, stream);
}

template <bool DOWN, bool Q8, bool XF>
hipError_t launch_resident_m(GateUpParams& p, hipStream_t stream) {
  const bool vec = row_bytes<Q8>(p.H) % 16 == 0;
  if (res_tiles(p.M) == 1)
    return vec ? launch_resident_t<1, true, DOWN, Q8, XF>(p, stream) : launch_resident_t<1, false, DOWN, Q8, XF>(p, stream);
  return vec ? launch_resident_t<2, true, DOWN, Q8, XF>(p, stream) : launch_resident_t<2, false, DOWN, Q8, XF>(p, stream);
}

template <bool XF>
hipError_t launch_resident_x(GateUpParams& p, hipStream_t stream) {
  if (p.q8) return p.down ? launch_resident_m<true, true, XF>(p, stream) : launch_resident_m<false, true, XF>(p, stream);
  return p.down ? launch_resident_m<true, false, XF>(p, stream) : launch_resident_m<false, false, XF>(p, stream);
}

}  // namespace

bool resident_fits(int M, int H, bool q8, bool xf) {
  if (M < 1 || M > kResMaxTokens) return false;
  const int nt = res_tiles(M);
  const bool wide = res_wide(nt, q8, xf);
  return (int64_t)M * (H / 8) <= (int64_t)kResXRegs * kResThreads &&
         (int64_t)res_steps(H, wide ? 256 : 128) * res_step_bytes(nt, wide ? 4 : 2) +
                 (int64_t)kResFixSlots * res_fix_words(nt) * 8 <=
             (int64_t)kResLds;
}

hipError_t launch_resident(GateUpParams p, hipStream_t stream) {
  const int nt = res_tiles(p.M);
  p.steps = res_steps(p.H, res_wide(nt, p.q8 != 0, p.xf32 != 0) ? 256 : 128);
  p.G = kResMaxPairs;
  p.wave_share = res_tiles(p.M) == 1 ? kWaveShare1 : kWaveShare2;
  return p.xf32 ? launch_resident_x<true>(p, stream) : launch_resident_x<false>(p, stream);
}

hipError_t launch_gate_up(const GateUpParams& p, int tokens_per_slot, hipStream_t stream) {
  return resident_fits(tokens_per_slot, p.H, p.q8 != 0, p.xf32 != 0) ? launch_resident(p, stream)
                                                         : launch_batch(p, tokens_per_slot, stream);
}

hipError_t launch_down(const GateUpParams& p, int pairs_per_slot, hipStream_t stream) {
  return resident_fits(p.M, p.H, p.q8 != 0, p.xf32 != 0) ? launch_resident(p, stream)
                                                          : launch_batch(p, pairs_per_slot, stream);
}

}  // namespace q4
