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
//  * Routing: a grouped call over at most kBitSlots slots first builds, in
//    every work-group, the bitmap of the slots its ids name; the tiles of
//    the routed slots only (T = routed slots x tiles per slot) are then cut
//    into whole-tile ranges, work-group b taking [bT/NB, (b+1)T/NB).  With
//    more slots every slot counts as routed.
//  * One persistent launch, one 8-wave work-group per CU.  The slots a
//    work-group's range touches (its segments, up to kMaxSeg at a time: a
//    round) are listed in LDS with, for each token, its first routed pair and
//    pair count there.  The (tile, K-step) units of a round are cut into
//    eight wave ranges (multiples of four steps; the first wave of each SIMD
//    takes a little more, see wave_share).  Each wave streams its range with
//    D K-steps of weights in flight in a register ring that runs on across
//    tile and slot boundaries; nothing synchronises the waves inside a round.
//  * The first weight loads go out as soon as the round's slots are known,
//    before x is split into digits; x is held in registers from the start.
//  * A tile cut by a wave boundary has several contributors; each adds its
//    exact quad sums into an LDS fix-up slot with LDS atomics and bumps the
//    slot's counter; the last one to arrive finishes the tile.
//  * K-steps per tile are padded to a multiple of four; the padding steps
//    meet zero digits, so they add nothing.
//  * Pairs with an id outside [0, num_slots) get zero outputs; each
//    work-group zero-fills its share of them once its tiles are done.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "q4moe_device.h"
#include "q4moe_launch.h"

namespace q4 {

namespace {

constexpr int kResWaves = 8;
constexpr int kResThreads = kResWaves * 64;
#ifndef Q4_RES_DEPTH
#define Q4_RES_DEPTH 2
#endif
// K-steps of weights in flight per wave (1, 2 or 4).  With whole-line loads
// a step leaves the ring as soon as it has arrived (take), so two steps in
// flight per wave keep the CU's reads going; four measured no faster at one
// column tile and ~1.5% slower at two (register pressure).
__host__ __device__ constexpr int res_depth(int nt, bool q8, bool xf) {
  return (void)nt, (void)q8, (void)xf, Q4_RES_DEPTH;
}
// K-steps per pass of the step loop: the B-fragment swizzle repeats every
// four steps, so four steps per pass keep its offsets fixed.
constexpr int kResU = 4;
constexpr int kResLds = 144 * 1024;        // digits, then the fix-up slots
constexpr int kResXRegs = 8;               // 16-byte chunks of x held per thread
constexpr int kResMaxTokens = 8;           // tokens per call
constexpr int kResFixSlots = kResWaves - 1;
constexpr int kResIdRegs = 4;              // routing ids held per thread (2048 pairs)
constexpr int kBitSlots = 2048;            // slots a routing bitmap covers
constexpr int kBitWords = kBitSlots / 32;
constexpr int kMaxSeg = 64;                // slots per round
constexpr int kInvBatch = 64;              // invalid pairs zero-filled per batch

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
// Wide K-steps (256 packed nibbles per row, four operand planes) for Q4
// weights and bf16 activations: rows are read 128 bytes per step (measured:
// the same bytes stream ~3-6% faster than 64 bytes per step).
__host__ __device__ constexpr bool res_wide(int nt, bool q8, bool xf) { return (void)nt, !q8 && !xf; }
// Column tiles for a call of M tokens: one up to two tokens, else two.
__host__ __device__ constexpr int res_tiles(int M) { return M <= 2 ? 1 : 2; }

// Inclusive sum of v over the lanes of a wave, up to lane `lane`.
__device__ __forceinline__ int wave_incl_sum(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// Bit position of the j-th (from 0) set bit of w; j < popcount(w).
__device__ __forceinline__ int nth_set_bit(uint32_t w, int j) {
  for (int i = 0; i < j; ++i) w &= w - 1u;
  return __builtin_ctz(w);
}

}  // namespace

// DOWN: the down projection (one matrix of a.I rows over a.H inputs; a tile is
// 32 rows, its first 16 taking the gate role and the next 16 the up role,
// each output rounded to bf16 on its own) instead of gate/up + SwiGLU.
// Q8: signed int8 weights, one byte per weight (else packed nibbles).
// XF: f32 activations and outputs (else bf16).
template <int NT, bool VEC, bool DOWN, bool Q8, bool XF>
__global__ __launch_bounds__(kResThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void resident_kernel(const GateUpParams a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kResLds];
  __shared__ __attribute__((aligned(16))) uint16_t s_sig[kSigTable];  // bf16 sigmoid of the tabulated gT
  __shared__ int s_xmax[kResMaxTokens];
  __shared__ int s_xmin[kResMaxTokens];      // smallest non-zero exponent field of each token
  __shared__ uint32_t s_bits[kBitWords];     // routed slots
  __shared__ int s_first[kMaxSeg][kResMaxTokens];  // first pair of token t on segment k
  __shared__ int s_cnt[kMaxSeg][kResMaxTokens];    // pairs of token t on segment k
  __shared__ int s_fixcnt[kResFixSlots];
  __shared__ int s_bound[kResWaves + 1];     // unit ranges of the round, by position
  __shared__ int s_inv;
  __shared__ int s_ninv;
  __shared__ int s_invl[kInvBatch];

  constexpr int kResD = res_depth(NT, Q8, XF);
  constexpr bool WIDE = res_wide(NT, Q8, XF);
  constexpr bool WL = Q8 || WIDE;            // 32 bytes per lane and step
  constexpr bool LINE = WL;                  // weights loaded in whole lines (load_line)
  constexpr int NPL = WIDE ? 4 : 2;          // operand planes per step
  constexpr bool xf = XF;
  // x held in registers from the start and the first weights in flight
  // before it is split (f32 activations: split first, then the weights)
  constexpr bool RING_FIRST = !XF;
  // Every argument is read here, in one batch of scalar loads: left to the
  // compiler, the fields arrive in several dependent round trips spread over
  // the prologue.
  asm volatile("" ::"s"(a.slots), "s"(a.slot_stride), "s"(a.gate_w_off), "s"(a.up_w_off), "s"(a.gate_s_off),
               "s"(a.up_s_off), "s"(a.x), "s"(a.ids), "s"(a.out), "s"(a.gate_probe), "s"(a.up_probe),
               "s"(a.invalid_count), "s"(a.M), "s"(a.K), "s"(a.H), "s"(a.I), "s"(a.num_slots), "s"(a.steps),
               "s"(a.wave_share), "s"(a.sig), "s"(gridDim.x));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, cc = lane & 15;
  const int H = a.H, I = a.I, M = a.M, K = a.K;
  const int P = M * K;
  const bool grouped = a.ids != nullptr;
  const int S = a.steps;                     // K-steps per tile, a multiple of 4
  const int sbytes = res_step_bytes(NT, NPL);
  const int hw = H / 8;                      // 16-byte chunks of one token's x
  const int npr = (hw + 1) / 2;              // chunk pairs of one token's x
  constexpr int RT = DOWN ? 32 : 16;         // rows per tile
  const int tps = (I + RT - 1) / RT;         // tiles per slot
  const int NB = gridDim.x;
  const uint32_t rbytes = row_bytes<Q8>(H);  // bytes of one weight row
  const uint32_t wbytes = (uint32_t)((uint64_t)I * rbytes);
  unsigned long long* const s_fix = (unsigned long long*)(s_lds + S * sbytes);
  // the routed outputs, [P][I] elements of esz bytes (under 2^31 bytes: the
  // launcher sends larger calls to the batch kernel)
  const uint32_t esz = xf ? 4u : 2u;
  const __amdgpu_buffer_rsrc_t osrc = make_rsrc(a.out, (uint32_t)P * (uint32_t)I * esz);
  auto out_store = [&](uint32_t v, uint32_t off) {
    if (xf)
      __builtin_amdgcn_raw_buffer_store_b32(v, osrc, (int)off, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, osrc, (int)off, 0, 0);
  };

  // ---- routing ids, the sigmoid table and x, loaded before anything waits ----
  // (unconditional buffer loads: lanes past the data read zeros without a
  // memory access, and the compiler's wait counts stay exact)
  const __amdgpu_buffer_rsrc_t idsrc = make_rsrc(a.ids, grouped ? (uint32_t)P * 4u : 0u);
  int idr[kResIdRegs];
#pragma unroll
  for (int j = 0; j < kResIdRegs; ++j) {
    const int p = tid + j * kResThreads;
    const int v = (int)__builtin_amdgcn_raw_buffer_load_b32(idsrc, p * 4, 0, 0);
    idr[j] = p < P ? v : -1;
  }
  // the device's sigmoid table, 16 bytes per thread
  static_assert(kSigTable * 2 == 16 * kResThreads, "one 16-byte piece of the sigmoid table per thread");
  const uint4 sigv = DOWN ? make_uint4(0, 0, 0, 0) : load_u4(make_rsrc(a.sig, kSigTable * 2), tid * 16u);
  // wide steps: chunk pairs u = m * npr + r (chunks 2r, 2r+1 of token m),
  // u = tid + k * kResThreads; else chunks q = m * hw + w8
  const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(a.x, xf ? 0u : (uint32_t)M * (uint32_t)H * 2u);
  uint4 xv[kResXRegs];
  if constexpr (WIDE) {
#pragma unroll
    for (int k = 0; k < kResXRegs / 2; ++k) {
      const int u = tid + k * kResThreads;
      const int m = u / npr, r = u - m * npr;
      const bool live = u < M * npr;
      const uint32_t o0 = live ? (uint32_t)(m * hw + 2 * r) * 16u : kOffNone;
      const uint32_t o1 = (live && 2 * r + 1 < hw) ? o0 + 16u : kOffNone;
      xv[2 * k] = load_u4(xsrc, o0);
      xv[2 * k + 1] = load_u4(xsrc, o1);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kResXRegs; ++j) {
      const int q = tid + j * kResThreads;
      xv[j] = load_u4(xsrc, q < M * hw ? (uint32_t)q * 16u : kOffNone);
    }
  }

  // ---- tiles of the routed slots: whole-tile ranges per work-group ----
  const bool compact = grouped && a.num_slots <= kBitSlots;
  int R = grouped ? a.num_slots : 1;         // routed slots
  int v0 = 0, v1 = 0;
  // the current round: tiles [vr0, vr1), routed slots ra .. ra+nseg-1
  int vr0 = 0, vr1 = 0, ra = 0, nseg = 0, N = 0;
  auto tile_split = [&]() {
    const uint32_t T = (uint32_t)R * (uint32_t)tps;
    auto at = [&](uint32_t b) {
      const uint64_t n = (uint64_t)b * T;
      return (int)(n < 0x100000000ull ? (uint32_t)n / (uint32_t)NB : n / (uint32_t)NB);
    };
    v0 = at(blockIdx.x);
    v1 = at(blockIdx.x + 1);
    vr0 = v0;                                // the first round starts the range
  };
  // routing bitmap held by every wave (see below); before it is known the
  // slots are taken as all routed
  uint32_t wbits = 0u;
  int wpre = 0;
  bool known = !compact;                     // slot mapping final
  // slot of routed index r (wave-uniform, r < R)
  auto select = [&](int r) {
    if (!grouped) return 0;
    if (!compact || !known) return r;
    const uint64_t bal = __ballot(wpre <= r && r < wpre + (int)__popc(wbits));
    const int l = (int)__builtin_ctzll(bal);
    const uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)wbits, l);
    return 32 * l + nth_set_bit(bits, r - __builtin_amdgcn_readlane(wpre, l));
  };
  // ---- the current round: tiles [vr0, vr1), routed slots ra .. ra+nseg-1 ----
  // Unit range start of position k (0..8).  The units are cut into four equal
  // quarters, one per SIMD; quarter q goes to waves q (first on its SIMD,
  // which wins the SIMD's issue arbitration more often) and q + 4, the first
  // taking wave_share/1024.  Position k = 2*(wave % 4) + wave / 4 orders the
  // ranges by unit.
  auto bound = [&](int k) {
    if (k >= kResWaves) return N;
    const int q = k >> 1;
    const int qa = (int)(((int64_t)q * N / 4) / kResU * kResU);
    if (!(k & 1)) return qa;
    const int qb = q == 3 ? N : (int)(((int64_t)(q + 1) * N / 4) / kResU * kResU);
    return qa + (int)(((int64_t)(qb - qa) * a.wave_share / 1024) / kResU * kResU);
  };
  const int wpos = 2 * (wave & 3) + (wave >> 2);
  int ua = 0, ub = 0;
  // the round's extent and this wave's unit range (no LDS)
  auto open_round = [&]() {
    ra = vr0 / tps;
    nseg = vr0 < v1 ? min(kMaxSeg, (v1 - 1) / tps - ra + 1) : 0;
    vr1 = min(v1, (ra + nseg) * tps);
    N = (vr1 - vr0) * S;
    ua = bound(wpos);
    ub = bound(wpos + 1);
  };
  // ---- weight load cursor: round tile lt, step ls, segment lk ----
  // 32-byte steps are loaded in whole 128-byte lines (load_line): lane L
  // reads rows L / 8 and 8 + L / 8 of the tile; else lane 16 g + r reads row r
  auto row_off = [&](int t, int part) {
    const int row = LINE ? t * RT + 8 * part + (lane >> 3) : t * RT + cc;
    const uint32_t col = LINE ? 16u * (uint32_t)(lane & 7) : (uint32_t)g4 * group_bytes<WL>();
    return (uint32_t)(row < I ? row : I - 1) * rbytes + col;
  };
  const LineLanes lines = line_lanes(lane);
  // (an empty resource until a slot is set: every load through it returns
  // zeros without a memory access)
  __amdgpu_buffer_rsrc_t gsrc = make_rsrc(a.slots, 0u), usrc = make_rsrc(a.slots, 0u);
  auto set_slot = [&](int k) {                // segment k of the round
    const int e = select(ra + k);
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
  };
  StepW<WL> rg[kResD], ru[kResD];
  int ls = 0, lt = 0, lk = 0;                // load cursor: step, tile in slot, segment
  uint32_t loff = 0, loff2 = 0;              // the lane's row offsets in the tile
  auto seek = [&](int w) {                   // cursor to round tile w
    const int r = (vr0 + w) / tps;
    lk = r - ra;
    lt = vr0 + w - r * tps;
    set_slot(lk);
    loff = row_off(lt, 0);
    loff2 = row_off(lt, 1);
  };
  auto issue = [&](StepW<WL>& g, StepW<WL>& u_, bool live, uint32_t dep = 0u) {
    const uint32_t so = (uint32_t)ls * step_row_bytes<WL>();
    const uint32_t o = (live ? loff + so : kOffNone) + dep;
    if constexpr (LINE) {
      const uint32_t o2 = (live ? loff2 + so : kOffNone) + dep;
      load_line<VEC>(g, gsrc, o, o2);
      load_line<VEC>(u_, usrc, o, o2);
    } else {
      load_step<WL, VEC>(g, gsrc, o);
      load_step<WL, VEC>(u_, usrc, o);
    }
    // cursor step after the loads: next tile every S steps, next slot every
    // tps tiles (its resources reloaded then)
    const int nls = ls + (live ? 1 : 0);
    if (nls == S) {
      ls = 0;
      if (++lt == tps) {
        lt = 0;
        if (++lk < nseg) set_slot(lk);
      }
      loff = row_off(lt, 0);
      loff2 = row_off(lt, 1);
    } else {
      ls = nls;
    }
  };
  // Whole-line loads: the next step's weights, moved out of their ring slot
  // into the tile layout (line_to_tile), and the slot refilled at once with
  // the step D further on (live: inside the wave's range), so that D steps
  // stay in flight while a step is split and multiplied.  The refill's
  // offset passes through an empty asm that takes the moved bytes, so the
  // loads are issued after the moves have read the slot and land in the
  // slot's own registers.
  StepW<WL> sg, su;
  auto take = [&](int slot, bool live) {
    if constexpr (LINE) {
      sg = rg[slot];
      su = ru[slot];
      line_to_tile(sg, lines);
      line_to_tile(su, lines);
      uint32_t dep = 0u;
      asm volatile("" : "+v"(dep) : "v"(sg.a), "v"(sg.b), "v"(su.a), "v"(su.b));
      issue(rg[slot], ru[slot], live, dep);
    }
  };
  // The ring always holds D loads per array: slots past the wave's range
  // load nothing (kOffNone) and are never consumed.
  auto start_ring = [&]() {
    const int w = ua / S;
    ls = ua - w * S;
    if (ua < ub) seek(w);
#pragma unroll
    for (int d = 0; d < kResD; ++d) issue(rg[d], ru[d], ua + d < ub);
  };

  // With the slot mapping known up front (a single expert, more slots than
  // one bitmap covers) or likely to be the identity (at least as many pairs
  // as slots), the first weights go out before the ids have arrived.
  const bool spec = compact && P >= a.num_slots;
  const bool early = blockIdx.y == 0 && (known || spec);
  if (early) {
    tile_split();
    open_round();
    if constexpr (RING_FIRST) start_ring();
  }

  if (tid < kResMaxTokens) {
    s_xmax[tid] = 0;
    s_xmin[tid] = 255;
  }
  if (tid == 0) s_inv = 0;
  const int nw = (a.num_slots + 31) >> 5;
  if (compact && tid < nw) s_bits[tid] = 0;
  // empty pair tables of the first round: one entry per thread
  static_assert(kMaxSeg * kResMaxTokens == kResThreads, "one pair-table entry per thread");
  auto clear_tables = [&]() {
    s_first[tid / kResMaxTokens][tid % kResMaxTokens] = 0x7FFFFFFF;
    s_cnt[tid / kResMaxTokens][tid % kResMaxTokens] = 0;
  };
  clear_tables();
  __syncthreads();

  // ---- routed slots: bitmap, routed count R, invalid-id count ----
  // Every wave then holds the bitmap (word l in lane l) and, per word, the
  // routed slots before it, so that it finds the slot of a routed index or
  // the routed index of a slot by itself, without LDS or barriers.
  if (grouped) {
    int inv = 0;
    auto post = [&](int id) {
      if (id >= 0 && id < a.num_slots) {
        if (compact) atomicOr(&s_bits[id >> 5], 1u << (id & 31));
      } else {
        ++inv;
      }
    };
#pragma unroll
    for (int j = 0; j < kResIdRegs; ++j)
      if (tid + j * kResThreads < P) post(idr[j]);
    for (int p = tid + kResIdRegs * kResThreads; p < P; p += kResThreads) post(a.ids[p]);
    if (inv) atomicAdd(&s_inv, inv);                 // every work-group: the call's invalid ids
    __syncthreads();
    if (compact) {
      wbits = lane < nw ? s_bits[lane] : 0u;
      const int c = (int)__popc(wbits);
      const int incl = wave_incl_sum(c, lane);
      wpre = incl - c;
      R = __builtin_amdgcn_readlane(incl, 63);
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0 && a.invalid_count) *a.invalid_count = s_inv;
  }
  known = true;
  // the routed index of a routed slot id (per lane; the shuffles read other
  // lanes: every lane of the wave must be active)
  auto rank = [&](int id) {
    if (!compact) return id;
    const int w = id >> 5;
    const uint32_t bits = (uint32_t)__shfl((int)wbits, w);
    return __shfl(wpre, w) + (int)__popc(bits & ((1u << (id & 31)) - 1u));
  };

  if (early && R != (grouped ? a.num_slots : 1)) {
    // some slot is not routed: the weights in flight belong to the identity
    // mapping; let them land, then start over on the routed slots
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    tile_split();
    open_round();
    if constexpr (RING_FIRST) start_ring();
  } else if (!early) {
    tile_split();
  }

  // pairs of the round's slots (into cleared tables), unit bounds, cleared
  // fix-up slots (visible after the next barrier)
  auto fill_round = [&]() {
    if (!grouped) {
      if (tid < M) {
        s_first[0][tid] = tid;
        s_cnt[0][tid] = 1;
      }
    } else {
      // called with every lane active (rank shuffles); only the table
      // updates depend on the lane's pair
      auto put = [&](int p, int id) {
        const bool valid = p < P && id >= 0 && id < a.num_slots;
        const int k = rank(valid ? id : 0) - ra;
        if (valid && k >= 0 && k < nseg) {
          const int t = p / K;
          atomicMin(&s_first[k][t], p);
          atomicAdd(&s_cnt[k][t], 1);
        }
      };
#pragma unroll
      for (int j = 0; j < kResIdRegs; ++j) put(tid + j * kResThreads, idr[j]);
      for (int base = kResIdRegs * kResThreads; base < P; base += kResThreads) {
        const int p = base + tid;
        put(p, p < P ? a.ids[p] : -1);
      }
    }
    if (tid <= kResWaves) s_bound[tid] = bound(tid);
    if (tid < kResFixSlots) s_fixcnt[tid] = 0;
    for (int i = tid; i < kResFixSlots * res_fix_words(NT); i += kResThreads) s_fix[i] = 0;
  };

  // digits per value and columns per token, fixed once x has been read
  int L = 6, W = 8;
  auto etop = [&](int m) { return xf ? max((s_xmax[m] >> 23) & 0xFF, 1) : max((s_xmax[m] >> 7) & 0xFF, 1); };
  // chunk q (8 consecutive values) of f32 activations: two 16-byte loads
  auto xf_chunk = [&](int q, uint4& lo4, uint4& hi4) {
    const uint4* xp = (const uint4*)((const float*)a.x + 8 * (size_t)q);
    lo4 = xp[0];
    hi4 = xp[1];
  };
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
  // g of step st) of pass token tl, in the operand order of split_planes:
  // word 2i + h goes to planes 2(i/2) (even positions) and 2(i/2) + 1 (odd),
  // dword 2(i%2) + h of each 16-byte chunk
  auto stage_pair = [&](int tl, int r, const uint4 xa, const uint4 xb, int etop1) {
    const int st = r >> 4, gg = (r >> 2) & 3, i = r & 3;
    const int pe = 2 * (i >> 1);
    uint8_t* base = s_lds + st * sbytes + 8 * (i & 1);
    auto put = [&](int j, int h, int col, uint32_t v) {
      *(uint32_t*)(base + 4 * h + (j * NT + (col >> 4)) * 1024 + res_chunk(gg, col & 15, st) * 16) = v;
    };
    auto word = [&](int h, const uint4 xq) {
      const uint32_t xs[8] = {xq.x & 0xFFFFu, xq.x >> 16, xq.y & 0xFFFFu, xq.y >> 16,
                              xq.z & 0xFFFFu, xq.z >> 16, xq.w & 0xFFFFu, xq.w >> 16};
      uint32_t v[8], ev[4], od[4];
      if (W == 4) {
#pragma unroll
        for (int p = 0; p < 8; ++p) v[p] = x_digits4(xs[p], etop1);
        plane_digits4(v, ev, od);
#pragma unroll
        for (int sd = 0; sd < 4; ++sd) {
          put(pe, h, tl * 4 + sd, ev[sd]);
          put(pe + 1, h, tl * 4 + sd, od[sd]);
        }
      } else {
        // six digits: columns [d0 d1 d2 0 d3 d4 d5 0]
        uint32_t hv[8], eh[4], oh[4];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const uint64_t z = x_digits(xs[p], etop1);
          v[p] = (uint32_t)z;
          hv[p] = (uint32_t)(z >> 32);
        }
        plane_digits4(v, ev, od);
        plane_digits4(hv, eh, oh);
        put(pe, h, tl * 8 + 0, ev[0]);
        put(pe, h, tl * 8 + 1, ev[1]);
        put(pe, h, tl * 8 + 2, ev[2]);
        put(pe, h, tl * 8 + 3, 0u);
        put(pe, h, tl * 8 + 4, ev[3]);
        put(pe, h, tl * 8 + 5, eh[0]);
        put(pe, h, tl * 8 + 6, eh[1]);
        put(pe, h, tl * 8 + 7, 0u);
        put(pe + 1, h, tl * 8 + 0, od[0]);
        put(pe + 1, h, tl * 8 + 1, od[1]);
        put(pe + 1, h, tl * 8 + 2, od[2]);
        put(pe + 1, h, tl * 8 + 3, 0u);
        put(pe + 1, h, tl * 8 + 4, od[3]);
        put(pe + 1, h, tl * 8 + 5, oh[0]);
        put(pe + 1, h, tl * 8 + 6, oh[1]);
        put(pe + 1, h, tl * 8 + 7, 0u);
      }
    };
    word(0, xa);
    word(1, xb);
  };

  // ---- range of every token's x: largest |x| and smallest non-zero exponent ----
  // (register j or pair k of a lane belongs to one token for the whole wave
  // when a token's units fill whole waves: sixteen DPP wave reductions go to
  // lane 0, which posts them; otherwise every lane posts its own values)
  auto post_range = [&](int m, uint32_t mx, uint32_t mn) {
    if (mx) atomicMax(&s_xmax[m], (int)mx);
    if (mn < 255) atomicMin(&s_xmin[m], (int)mn);
  };
  auto x_range = [&]() {
    if constexpr (XF) {
#pragma unroll 1
      for (int q = tid; q < (M * hw + 63) / 64 * 64; q += kResThreads) {
        uint32_t mx = 0, mn = 255;
        if (q < M * hw) {
          uint4 xa, xb;
          xf_chunk(q, xa, xb);
          f32_range8(xa, xb, mx, mn);
        }
        if (hw % 64 == 0) {
          mx = wave_extreme<true>(mx);
          mn = wave_extreme<false>(mn);
          if (lane == 0 && q < M * hw) post_range(q / hw, mx, mn);
        } else if (q < M * hw) {
          post_range(q / hw, mx, mn);
        }
      }
    } else if constexpr (WIDE) {
#pragma unroll
      for (int k = 0; k < kResXRegs / 2; ++k) {
        if (k * kResThreads < M * npr) {
          uint32_t mx, mn, mx2, mn2;
          range8(xv[2 * k], mx, mn);
          range8(xv[2 * k + 1], mx2, mn2);
          mx = max(mx, mx2);
          mn = min(mn, mn2);
          if (npr % 64 == 0) {
            mx = wave_extreme<true>(mx);
            mn = wave_extreme<false>(mn);
            const int u0 = k * kResThreads + (tid & ~63);
            if (lane == 0 && u0 < M * npr) post_range(u0 / npr, mx, mn);
          } else {
            const int u = tid + k * kResThreads;
            if (u < M * npr) post_range(u / npr, mx, mn);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kResXRegs; ++j) {
        if (j * kResThreads < M * hw) {
          uint32_t mx, mn;
          range8(xv[j], mx, mn);
          if (hw % 64 == 0) {
            mx = wave_extreme<true>(mx);
            mn = wave_extreme<false>(mn);
            const int q0 = j * kResThreads + (tid & ~63);
            if (lane == 0 && q0 < M * hw) post_range(q0 / hw, mx, mn);
          } else {
            const int q = tid + j * kResThreads;
            if (q < M * hw) post_range(q / hw, mx, mn);
          }
        }
      }
    }
  };

  // ---- digits of the pass's tokens [p0, p0 + ntok) ----
  // from the registers (f32: from memory); the padding K-steps get zero digits
  auto stage_pass = [&](int p0, int ntok) {
    if constexpr (WIDE) {
      // a rolled loop over the held pairs, picked by a uniform branch (one
      // unit's temporaries at a time while x and the weight ring hold their
      // registers); units of token m are [m * npr, (m + 1) * npr)
#pragma unroll 1
      for (int k = 0; k < kResXRegs / 2 && k * kResThreads < (p0 + ntok) * npr; ++k) {
        // (an empty asm in each branch keeps the branches: merged into an
        // indexed load, x would move to scratch memory)
        uint4 xa = xv[0], xb = xv[1];
        if (k == 1) {
          xa = xv[2];
          xb = xv[3];
          opaque4(xa);
          opaque4(xb);
        } else if (k == 2) {
          xa = xv[4];
          xb = xv[5];
          opaque4(xa);
          opaque4(xb);
        } else if (k == 3) {
          xa = xv[6];
          xb = xv[7];
          opaque4(xa);
          opaque4(xb);
        }
        const int u = tid + k * kResThreads;
        const int m = u / npr;
        if (m >= p0 && m < p0 + ntok) stage_pair(m - p0, u - m * npr, xa, xb, etop(m));
      }
      const int padp = S * 16 - npr;
#pragma unroll 1
      for (int u = tid; u < ntok * padp; u += kResThreads)
        stage_pair(u % ntok, npr + u / ntok, make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), 1);
    } else {
      if (xf) {
#pragma unroll 1
        for (int q = tid; q < ntok * hw; q += kResThreads) {
          const int tl = q / hw;
          uint4 xa, xb;
          xf_chunk((p0 + tl) * hw + q - tl * hw, xa, xb);
          stage_unitf(tl, q - tl * hw, xa, xb, etop(p0 + tl));
        }
      } else {
#pragma unroll 1
        for (int j = 0; j < kResXRegs && j * kResThreads < (p0 + ntok) * hw; ++j) {
          uint4 xq = xv[0];
          if (j == 1) xq = xv[1];
          else if (j == 2) xq = xv[2];
          else if (j == 3) xq = xv[3];
          else if (j == 4) xq = xv[4];
          else if (j == 5) xq = xv[5];
          else if (j == 6) xq = xv[6];
          else if (j == 7) xq = xv[7];
          const int q = tid + j * kResThreads;
          const int m = q / hw;
          if (m >= p0 && m < p0 + ntok) stage_unit(m - p0, q - m * hw, xq, etop(m));
        }
      }
      const int padw = S * 16 - hw;
#pragma unroll 1
      for (int u = tid; u < ntok * padw; u += kResThreads) {
        if (xf)
          stage_unitf(u % ntok, hw + u / ntok, make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), 1);
        else
          stage_unit(u % ntok, hw + u / ntok, make_uint4(0, 0, 0, 0), 1);
      }
    }
  };

  // ---- prologue: first round's slots, its weights in flight, digits ----
  // pass = blockIdx.y: the tokens [pass * tpp, (pass + 1) * tpp) of a call
  // with more tokens than one pass holds (launched with as many y slices as
  // six-digit tokens would need; a slice with nothing to do exits here)
  const int pass = blockIdx.y;
  if (pass == 0 && !early) {
    open_round();
    if constexpr (RING_FIRST) start_ring();
  }
  x_range();
  __syncthreads();
  {
    int l = 4;
    for (int m = 0; m < M; ++m) l = max(l, digits_for(s_xmax[m], s_xmin[m]));
    L = xf ? 8 : __builtin_amdgcn_readfirstlane(l);
  }
  W = L == 4 ? 4 : 8;
  const int tpp = 16 * NT / W;                              // tokens per pass
  const int tp0 = pass * tpp;                               // first token of the pass
  if (tp0 >= M) return;
  const int tp1 = min(M, tp0 + tpp);                        // end token
  if (pass > 0) {
    open_round();
    if constexpr (RING_FIRST) start_ring();
  }
  stage_pass(tp0, tp1 - tp0);
  if constexpr (!RING_FIRST) start_ring();
  fill_round();
  if constexpr (!DOWN) *(uint4*)(s_sig + 8 * tid) = sigv;
  __syncthreads();
  // whole-line loads: the first step's weights out of the ring (each later
  // step is taken one step ahead, in the step loop)
  if constexpr (LINE) take(0, ua + kResD < ub);

  // exact (row, token) sums of the four digit columns of each lane quad:
  // lane j of the quad receives row 4*g4 + j
  const int qj = cc & 3;
  auto quad_row_sum = [&](const v4i acc) { return quad_digit_sum(acc, qj); };
  // this lane's B-fragment chunk for steps 0..3 mod 4
  static_assert(kResU % kResD == 0, "the step loop's pass covers whole turns of the ring");
  int rdo[kResU];
#pragma unroll
  for (int j = 0; j < kResU; ++j) rdo[j] = res_chunk(g4, cc, j) * 16;

  {
    // the pass token of this lane's quad in each column tile, and its exponent
    int ltok[NT], lxm[NT];
    bool lok[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      ltok[n] = W == 4 ? 4 * n + (cc >> 2) : 2 * n + (cc >> 3);
      lok[n] = (W == 4 || (cc & 4) == 0) && ltok[n] < tp1 - tp0;
      lxm[n] = lok[n] ? s_xmax[tp0 + ltok[n]] : 0;
    }

    // Output buffer: the outputs of this wave's last finished tiles, written
    // together once the tiles cover whole 128-byte lines of the output rows
    // (kOB tiles), at the end of the wave's range, or at a slot's last tile.
    // Written one tile at a time, the 32-byte pieces of a line reach the
    // cache tens of microseconds apart and go to HBM as partial lines, which
    // costs the weight stream ~5% at eight tokens.
    constexpr int kOB = (int)(128 / (XF ? 4 : 2)) / RT > 0 ? (int)(128 / (XF ? 4 : 2)) / RT : 1;
    uint32_t obv[kOB][NT], obo[kOB][NT], obv2[kOB][NT], obo2[kOB][NT];
#pragma unroll
    for (int q = 0; q < kOB; ++q)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        obv[q][n] = obv2[q][n] = 0u;
        obo[q][n] = obo2[q][n] = kOffNone;
      }
    for (;;) {                               // rounds
      int u = ua;
      while (u < ub) {
        // one portion: the rest of the current tile inside [u, ub)
        const int w = u / S;                                  // round tile
        const int sa = u - w * S;
        const int pe = min(ub, (w + 1) * S);                  // portion end (unit)
        const int v = vr0 + w;
        const int rr = v / tps;
        const int k = rr - ra;                                // segment
        const int e = select(rr);
        const uint8_t* slot = a.slots + (uint64_t)e * a.slot_stride;
        const float* gscale = (const float*)(slot + a.gate_s_off);
        const float* uscale = (const float*)(slot + a.up_s_off);
        // the row scales this lane may finish with, loaded ahead of the
        // portion's weight loads: loads complete in order, so a scale load
        // issued at the finish would wait for every weight load in flight
        const int row = (v - rr * tps) * RT + 4 * g4 + qj;
        const float gsc = gscale[min(row, I - 1)];
        const float usc = DOWN ? gscale[min(row + 16, I - 1)] : uscale[min(row, I - 1)];
        // the routed pairs of this lane's (slot, token) items, read before the
        // steps (LDS latency off the finish)
        int pcnt[NT], pfirst[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int tg = min(tp0 + ltok[n], kResMaxTokens - 1);
          pcnt[n] = s_cnt[k][tg];
          pfirst[n] = s_first[k][tg];
        }
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
            if constexpr (LINE) {
              // this step's weights were moved out of the ring one step ago
              if constexpr (WIDE) {
                split_planes(sg.a, sg.b, pg);
                split_planes(su.a, su.b, pu);
              } else {
                split_step(sg, pg[0], pg[1]);
                split_step(su, pu[0], pu[1]);
              }
              // the next step's slot: moved out and refilled at once
              take((j + 1) % kResD, u + j + 1 + kResD < ub);
            } else {
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
            }
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
          const int tu0 = w * S, tu1 = tu0 + S;
          int first = -1, ncontrib = 0;
          for (int kk = 0; kk < kResWaves; ++kk) {
            const int qa = s_bound[kk], qb = s_bound[kk + 1];
            if (qa < qb && qa < tu1 && qb > tu0) {
              if (first < 0) first = kk;
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
        // Outputs go out as buffer stores, the same stores on every portion:
        // an item with nothing to store (a portion that does not finish its
        // tile, a lane without a routed pair) stores at an offset past the
        // buffer, which drops the write.  The portion's memory operations are
        // then the same on every path and the wait counts of the weight loads
        // stay exact.  Optional stores (probes, duplicate ids) wait for every
        // memory operation before going on.
        uint32_t st_off[NT], st_off2[NT], st_val[NT], st_val2[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          st_off[n] = st_off2[n] = kOffNone;
          st_val[n] = st_val2[n] = 0u;
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
            // probes and duplicate pairs: global stores (optional path)
            auto store = [&](int pair, bool out_too) {
              const uint64_t o = (uint64_t)pair * I + row;
              float* const outf = (float*)a.out;
              if constexpr (DOWN) {
                // rows `row` and `row + 16`, each its own output
                if (out_too) {
                  if (xf)
                    outf[o] = gate;
                  else
                    a.out[o] = bf16_rne(gate);
                }
                if (a.gate_probe) a.gate_probe[o] = gate;
                if (row + 16 < I) {
                  if (out_too) {
                    if (xf)
                      outf[o + 16] = up;
                    else
                      a.out[o + 16] = bf16_rne(up);
                  }
                  if (a.gate_probe) a.gate_probe[o + 16] = up;
                }
              } else {
                if (out_too) {
                  if (xf)
                    outf[o] = ovf;
                  else
                    a.out[o] = ov;
                }
                if (a.gate_probe) a.gate_probe[o] = gate;
                if (a.up_probe) a.up_probe[o] = up;
              }
            };
            if (ok) {
              const int tg = tp0 + tl;                        // token of the call
              const int cnt = pcnt[n];
              const int p1 = pfirst[n];
              if (cnt > 0) {
                const uint32_t o = (uint32_t)p1 * (uint32_t)I + (uint32_t)row;
                if constexpr (DOWN) {
                  st_off[n] = o * esz;
                  st_val[n] = xf ? __float_as_uint(gate) : (uint32_t)bf16_rne(gate);
                  if (row + 16 < I) {
                    st_off2[n] = (o + 16u) * esz;
                    st_val2[n] = xf ? __float_as_uint(up) : (uint32_t)bf16_rne(up);
                  }
                } else {
                  st_off[n] = o * esz;
                  st_val[n] = xf ? __float_as_uint(ovf) : (uint32_t)ov;
                }
              }
              if ((cnt > 0 && (a.gate_probe || a.up_probe)) || cnt > 1) {
                if (cnt > 0) store(p1, false);
                // a token routed to this slot more than once (duplicate ids)
                if (cnt > 1)
                  for (int jj = 0; jj < K; ++jj) {
                    const int p = tg * K + jj;
                    if (p != p1 && a.ids[p] == e) store(p, true);
                  }
                __builtin_amdgcn_s_waitcnt(kWaitVmem0);
              }
            }
          }
        }
        if (finish) {
#pragma unroll
          for (int q = kOB - 1; q > 0; --q)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              obv[q][n] = obv[q - 1][n];
              obo[q][n] = obo[q - 1][n];
              obv2[q][n] = obv2[q - 1][n];
              obo2[q][n] = obo2[q - 1][n];
            }
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            obv[0][n] = st_val[n];
            obo[0][n] = st_off[n];
            obv2[0][n] = st_val2[n];
            obo2[0][n] = st_off2[n];
          }
        }
        // wave-uniform: the tile ends a line group or a slot, or the wave's
        // range ends here
        const int tis = v - rr * tps;                         // tile in its slot
        if (pe >= ub || (finish && (((tis + 1) * RT) % (RT * kOB) == 0 || tis + 1 == tps))) {
#pragma unroll
          for (int q = 0; q < kOB; ++q)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              out_store(obv[q][n], obo[q][n]);
              if constexpr (DOWN) out_store(obv2[q][n], obo2[q][n]);
              obo[q][n] = obo2[q][n] = kOffNone;
            }
        }
      }
      // ---- next round of this pass ----
      if (vr1 >= v1) break;
      __syncthreads();                       // every wave done with the round's tables
      vr0 = vr1;
      open_round();
      clear_tables();
      __syncthreads();
      start_ring();
      fill_round();
      __syncthreads();
      if constexpr (LINE) take(0, ua + kResD < ub);
    }

  }

  // ---- pairs with invalid ids get zero outputs: pairs b, b + NB, ... here
  // (skipped, with its barriers and id reloads, when the call has none) ----
  if (grouped && pass == 0 && s_inv > 0) {
    const int nmine = P > (int)blockIdx.x ? (P - (int)blockIdx.x + NB - 1) / NB : 0;
    for (int base = 0; base < nmine; base += kResThreads) {
      __syncthreads();
      if (tid == 0) s_ninv = 0;
      __syncthreads();
      const int i = base + tid;
      const int p = (int)blockIdx.x + i * NB;
      const bool bad = i < nmine && (a.ids[p] < 0 || a.ids[p] >= a.num_slots);
      int at = -1;
      if (bad) at = atomicAdd(&s_ninv, 1);
      if (bad && at < kInvBatch) s_invl[at] = p;
      __syncthreads();
      const int nl = min(s_ninv, kInvBatch);
      for (int q = 0; q < nl; ++q) {
        const int pq = s_invl[q];
        for (int r = tid; r < I; r += kResThreads) {
          const uint64_t o = (uint64_t)pq * I + r;
          if (xf)
            ((float*)a.out)[o] = 0.0f;
          else
            a.out[o] = 0;
          if (a.gate_probe) a.gate_probe[o] = 0.0f;
          if (a.up_probe) a.up_probe[o] = 0.0f;
        }
      }
      // past the batch: each finder fills its own pair
      if (bad && at >= kInvBatch)
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
  // per-device cache; concurrent first calls compute the same value
  static std::atomic<int> cached[64];
  if (device < 0 || device >= 64) device = 0;
  if (!cached[device].load(std::memory_order_relaxed)) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&resident_kernel<NT, VEC, DOWN, Q8, XF>), kResThreads, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    cached[device].store(cus * per_cu, std::memory_order_relaxed);
  }
  return cached[device].load(std::memory_order_relaxed);
}

template <int NT, bool VEC, bool DOWN, bool Q8, bool XF>
hipError_t launch_resident_t(GateUpParams& p, hipStream_t stream) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  const int rt = DOWN ? 32 : 16;
  const int tiles = p.num_slots * ((p.I + rt - 1) / rt);
  int nb = resident_blocks<NT, VEC, DOWN, Q8, XF>(device);
  if (nb > tiles) nb = tiles;
  // y slices: the passes six-digit tokens would need (2 * NT per pass)
  const int slices = (p.M + 2 * NT - 1) / (2 * NT);
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&resident_kernel<NT, VEC, DOWN, Q8, XF>), dim3((unsigned)nb, (unsigned)slices),
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
  // x of every token in registers: chunks, or chunk pairs with wide steps
  const int64_t xunits = wide ? (int64_t)M * ((H / 8 + 1) / 2) * 2 : (int64_t)M * (H / 8);
  return xunits <= (int64_t)kResXRegs * kResThreads &&
         (int64_t)res_steps(H, wide ? 256 : 128) * res_step_bytes(nt, wide ? 4 : 2) +
                 (int64_t)kResFixSlots * res_fix_words(nt) * 8 <=
             (int64_t)kResLds;
}

hipError_t launch_resident(GateUpParams p, hipStream_t stream) {
  const int nt = res_tiles(p.M);
  p.steps = res_steps(p.H, res_wide(nt, p.q8 != 0, p.xf32 != 0) ? 256 : 128);
  p.wave_share = res_tiles(p.M) == 1 ? kWaveShare1 : kWaveShare2;
  return p.xf32 ? launch_resident_x<true>(p, stream) : launch_resident_x<false>(p, stream);
}

// The resident kernel addresses its outputs with 32-bit buffer offsets.
static bool resident_out_fits(const GateUpParams& p) {
  return (uint64_t)p.M * (uint64_t)p.K * (uint64_t)p.I * (p.xf32 ? 4u : 2u) < 0x80000000ull;
}

hipError_t launch_gate_up(const GateUpParams& p, int tokens_per_slot, hipStream_t stream) {
  GateUpParams q = p;
  const hipError_t e = sigmoid_table(&q.sig);
  if (e != hipSuccess) return e;
  if (resident_fits(tokens_per_slot, q.H, q.q8 != 0, q.xf32 != 0) && resident_out_fits(q)) return launch_resident(q, stream);
  const int nt = chunked_tiles(q);
  return nt ? launch_chunked(q, nt, stream) : launch_batch(q, tokens_per_slot, stream);
}

hipError_t launch_down(const GateUpParams& p, int pairs_per_slot, hipStream_t stream) {
  if (resident_fits(p.M, p.H, p.q8 != 0, p.xf32 != 0) && resident_out_fits(p)) return launch_resident(p, stream);
  const int nt = chunked_tiles(p);
  return nt ? launch_chunked(p, nt, stream) : launch_batch(p, pairs_per_slot, stream);
}

}  // namespace q4
