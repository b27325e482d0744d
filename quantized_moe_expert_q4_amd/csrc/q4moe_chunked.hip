// Q4 gate/up + SwiGLU (and the down projection) for routed calls with a few
// tokens per slot whose digits do not all fit LDS for the launch: the routed
// step of a mixture-of-experts layer, the down projection of one routed row
// per slot, one GPU's share of expert-parallel routing.
//
// Arithmetic: GATE_UP_SOURCE and DOWN_SOURCE of the @mlx-bun/inference 1.0.0
// diff, page 52 (kernels/glm52/streamed-experts.ts), made exact as in
// q4moe_device.h.
//
// The weight stream is the resident kernel's: 16-row tiles, wide K-steps of
// 256 packed nibbles per row loaded in whole 128-byte lines with the
// non-temporal hint and moved to the operand layout by a lane shuffle, D steps
// in flight per wave in a register ring that takes each step one step ahead.
// What differs is where the activation digits come from:
//  * One persistent 8-wave work-group per CU takes an even share of the cost
//    of the (slot, pass, tile) units: a slot with c routed pairs takes
//    ceil(c/G) passes over its tiles (G = 7 pairs at two column tiles, 4 at
//    one); a tile counts for more in a pass of more pairs, and each pass adds
//    a segment set-up.  A work-group walks its share in segments (one pass
//    over at most 48 tiles of one slot, 64 for a down projection whose K
//    fits LDS), each in token groups: as
//    many of the pass's pairs as fit 16*NT digit columns, four per row or
//    eight for a row whose values need six digits.
//  * A group's digits are split from x into LDS per K-chunk, double buffered
//    (once for the whole K when it fits both buffers).
//  * A segment's tiles are cut into rounds of at most kChRoundTiles tiles.
//    The (round, chunk) elements of a group form one stream that every wave
//    walks in the same order; in each element a wave takes the same fraction
//    of the round's tiles (its (tile, K-step) units, in whole passes of the
//    step loop: a SIMD's quarter, the first wave of the SIMD a little more
//    than half of it), so it meets at most kChMaxT tiles of a round and keeps
//    their sums in registers from chunk to chunk.  A tile met by several waves
//    collects their exact quad sums in an LDS fix-up slot (LDS atomics); the
//    last contributor finishes it.
//  * The digits of element k+1 are staged while element k is multiplied: a
//    wave's share is cut into quads (32 values of one row, 64 bytes of x),
//    or half quads when there are too few quads for every lane, at one per
//    lane per pass of the step loop, loaded at a pass's last step and split
//    into LDS chunks one pass later, so the waits for x never cover the
//    weight loads in flight.  One barrier per element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "q4moe_device.h"
#include "q4moe_launch.h"

namespace q4 {

namespace {

constexpr int kChWaves = 8;
constexpr int kChThreads = kChWaves * 64;
constexpr int kChBuf = 64 * 1024;          // one of the two digit buffers
constexpr int kChU = 2;                    // K-steps per pass of the step loop
constexpr int kChD = 2;                    // K-steps in flight per wave
constexpr int kChRoundTiles = 14;          // tiles per round
constexpr int kChMaxT = 3;                 // tiles one wave meets in a round
constexpr int kChSegTiles = 48;            // tiles per segment (row scales held in LDS)
constexpr int kChSegTilesDown = 64;        // the same for the down projection with the whole K in LDS
constexpr int kChFixSlots = kChWaves - 1;
constexpr int kChCntSlots = 2048;          // slots whose passes are held in LDS
constexpr int kChIdRegs = 4;               // routing ids held per thread (2048 pairs)
constexpr int kChCntWords = kChCntSlots / 32;
constexpr int kChInvBatch = 64;            // invalid pairs zero-filled per batch
constexpr int kChTileBase = 16;            // a tile of n pairs costs (kChTileBase + n) / (kChTileBase + 1) one-pair tiles

// A wave's share of a round's units: the first wave of SIMD q takes the
// fraction [q/4, q/4 + share/4096) of the round's tiles, the second wave the
// rest of the quarter, share in [kChShareMin, kChShareMax] (the first wave of a
// SIMD wins its issue arbitration more often).  With at most kChRoundTiles
// tiles a share spans under two tiles, so it meets at most kChMaxT tiles.
constexpr int kChShareMin = 439, kChShareMax = 585;
static_assert(kChShareMax * kChRoundTiles < 2 * 4096 && (1024 - kChShareMin) * kChRoundTiles < 2 * 4096,
              "a wave's share of a round meets at most kChMaxT tiles");

// One wide K-step of digits: [plane 4][column tile n][k-group g 4][16 x 16
// bytes]; the 16-byte chunk of column c sits at position c ^ 4g of its
// k-group row (the sixteen lanes of a k-group read sixteen distinct chunks).
__host__ __device__ constexpr int ch_step_bytes(int nt) { return 4 * nt * 1024; }
__host__ __device__ constexpr int ch_chunk(int g, int c) { return g * 16 + (c ^ (4 * g)); }
// One fix-up slot: int64 [tile][gate, up][lane] (quad sums).
__host__ __device__ constexpr int ch_fix_words(int nt) { return nt * 2 * 64; }
// Wide K-steps per tile, padded to whole passes of the step loop (a padding
// step meets zero digits).
__host__ __device__ constexpr int ch_steps(int H) { return ((H + 255) / 256 + kChU - 1) / kChU * kChU; }
// K-steps per chunk: the whole K when it fits both buffers, else what fits one.
__host__ __device__ constexpr int ch_chunk_steps(int nt, int S) {
  return S * ch_step_bytes(nt) <= 2 * kChBuf ? S : kChBuf / ch_step_bytes(nt) / kChU * kChU;
}

}  // namespace

// DOWN: the down projection (one matrix of a.I rows over a.H inputs; a tile is
// 32 rows, its first 16 taking the gate role and the next 16 the up role,
// each output rounded to bf16 on its own) instead of gate/up + SwiGLU.
// WHOLE: the whole K's digits fit both buffers (one chunk), as the launcher
// decides from H and NT.
template <int NT, bool VEC, bool DOWN, bool WHOLE>
__global__ __launch_bounds__(kChThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunked_kernel(const GateUpParams a) {
  // pairs per pass: what fits 16*NT digit columns at four per row, with room
  // for one row of eight at two column tiles (a pass then needs a second
  // group only when two of its rows need six digits)
  constexpr int G = NT == 2 ? 7 : 4;
  constexpr int RT = DOWN ? 32 : 16;         // rows per tile
  constexpr int sbytes = ch_step_bytes(NT);
  __shared__ __attribute__((aligned(16))) uint8_t s_dig[2 * kChBuf];
  __shared__ unsigned long long s_fix[kChFixSlots * ch_fix_words(NT)];
  __shared__ int s_fixcnt[kChFixSlots];
  __shared__ __attribute__((aligned(16))) uint16_t s_sig[DOWN ? 8 : kSigTable];
  // tiles per segment: a down projection whose K fits LDS has no rounds and
  // one matrix of scales, and takes longer segments (fewer set-ups)
  constexpr int SEGT = DOWN && WHOLE ? kChSegTilesDown : kChSegTiles;
  __shared__ float s_gsc[SEGT * RT];          // row scales of the segment (DOWN: the down scales)
  __shared__ float s_usc[DOWN ? 1 : SEGT * RT];
  __shared__ uint8_t s_pass[kChCntSlots];     // passes of each slot
  __shared__ int s_ppre[kChCntWords + 1];     // passes of the slots before each 32-slot word, and in all
  __shared__ long long s_cpre[kChCntWords + 1];  // cost of the slots before each word, and in all
  __shared__ int s_pairs[G];
  __shared__ int s_tok[G];                   // x row of each pair of the group
  __shared__ int s_xmax[G];
  __shared__ int s_xmin[G];                  // smallest non-zero exponent field of each row
  __shared__ int s_col[G];                   // first digit column of each row
  __shared__ int s_wid[G];                   // digit columns of each row: 4, or 8 for six digits
  __shared__ int s_quad[4 * NT];             // row of each 4-column quad; + 64 for the high quad of an 8-column row
  __shared__ int s_wcnt[kChWaves];
  __shared__ int s_inv;
  __shared__ int s_ninv;
  __shared__ int s_invl[kChInvBatch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, cc = lane & 15;
  const int qj = cc & 3;
  const int H = a.H, I = a.I, K = a.K;
  const int P = a.M * K;
  const bool grouped = a.ids != nullptr;
  const int S = a.steps;                     // wide K-steps per tile, a multiple of kChU
  const int Sc = WHOLE ? S : ch_chunk_steps(NT, S);
  const int nch = WHOLE ? 1 : (S + Sc - 1) / Sc;
  const int tps = (I + RT - 1) / RT;         // tiles per slot
  const int NB = gridDim.x;
  const uint32_t rbytes = (uint32_t)(H / 2);
  const uint32_t wbytes = (uint32_t)((uint64_t)I * rbytes);
  const int hw = H / 8;                      // 8-value units of one row of x

  // ---- the sigmoid table, fix-up slots, routed slots, invalid ids ----
  if constexpr (!DOWN) {
    static_assert(kSigTable * 2 == 16 * kChThreads, "one 16-byte piece of the sigmoid table per thread");
    *(uint4*)(s_sig + 8 * tid) = load_u4(make_rsrc(a.sig, kSigTable * 2), tid * 16u);
  }
  if (tid == 0) s_inv = 0;
  if (tid < kChFixSlots) s_fixcnt[tid] = 0;
  for (int i = tid; i < kChFixSlots * ch_fix_words(NT); i += kChThreads) s_fix[i] = 0;
  // Work is cut by cost: a slot with c routed pairs takes ceil(c / G) passes
  // over its tiles (pass g: its pairs g*G .. g*G + G - 1 in id order), and
  // the cost of the (slot, pass, tile) units is split evenly over the
  // work-groups, so a slot that many tokens chose spreads over more
  // work-groups instead of lengthening the launch.  The passes are held for
  // up to kChCntSlots slots, fewer than 65536 pairs and at most 255 passes a
  // slot; otherwise every slot takes one pass, its pairs in as many groups as
  // they need.
  // The ids of the first kChIdRegs * kChThreads pairs stay in registers for
  // the group scans.
  const __amdgpu_buffer_rsrc_t idsrc = make_rsrc(a.ids, grouped ? (uint32_t)P * 4u : 0u);
  int idr[kChIdRegs];
#pragma unroll
  for (int j = 0; j < kChIdRegs; ++j) {
    const int p = tid + j * kChThreads;
    const int id = (int)__builtin_amdgcn_raw_buffer_load_b32(idsrc, p * 4, 0, 0);
    idr[j] = p < P ? id : -1;
  }
  // id of pair p = tid + j * kChThreads (a select over the held registers:
  // indexed, they would move to scratch memory)
  static_assert(kChIdRegs == 4, "id_at selects among four registers");
  auto id_at = [&](int j, int p) {
    if (j >= kChIdRegs) return p < P ? a.ids[p] : -1;
    const int lo = j & 1 ? idr[1] : idr[0], hi = j & 1 ? idr[3] : idr[2];
    return j & 2 ? hi : lo;
  };
  // pair counts per slot, in the digit buffer (free until the first group)
  uint32_t* const cnt = (uint32_t*)s_dig;
  const bool counting = grouped && a.num_slots <= kChCntSlots && P < 65536;
  if (counting)
    for (int i = tid; i < kChCntSlots; i += kChThreads) cnt[i] = 0u;
  __syncthreads();
  if (grouped) {
    int inv = 0;
    for (int j = 0; j * kChThreads < P; ++j) {
      const int p = tid + j * kChThreads;
      const int id = id_at(j, p);
      if (p >= P) continue;
      if (id >= 0 && id < a.num_slots) {
        if (counting) atomicAdd(&cnt[id], 1u);
      } else {
        ++inv;
      }
    }
    if (inv) atomicAdd(&s_inv, inv);               // every work-group: the call's invalid ids
  }
  __syncthreads();
  auto passes = [&](int c) { return (c + G - 1) / G; };
  // Cost units: a tile of a pass of n pairs costs S * (kChTileBase + n)
  // (staging and finishing grow with the pairs), a segment's set-up
  // segu; a slot with c pairs in ps passes costs ps * segu + ts * (ps *
  // kChTileBase + c).
  const int64_t ts = (int64_t)tps * S;
  const int64_t segu = (int64_t)a.seg_cost * (kChTileBase + 1);
  auto slot_cost = [&](int ps, int n) { return ps * segu + ts * ((int64_t)ps * kChTileBase + n); };
  if (counting && wave == 0) {
    // passes (one byte each) and cost of every slot, two 32-slot words per
    // step (lane j: slot 64 i + j), each word's totals parked in s_ppre and
    // s_cpre; then their prefixes over words.  A slot with more than 255
    // passes turns the counts off.
    const int nw = (a.num_slots + 31) >> 5;
    int big = 0;
    for (int i = 0; 2 * i < nw; ++i) {
      const int sl = 64 * i + lane;
      const int n = sl < a.num_slots ? (int)cnt[sl] : 0;
      const int ps = passes(n);
      big |= ps > 255;
      s_pass[sl] = (uint8_t)ps;
      int pw = ps;
      long long cw = slot_cost(ps, n);
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) {
        pw += __shfl_xor(pw, d);
        cw += __shfl_xor(cw, d);
      }
      if ((lane & 31) == 0 && 2 * i + (lane >> 5) < nw) {
        s_ppre[2 * i + (lane >> 5)] = pw;
        s_cpre[2 * i + (lane >> 5)] = cw;
      }
    }
    const int c = lane < nw ? s_ppre[lane] : 0;
    const long long cw = lane < nw ? s_cpre[lane] : 0;
    int incl = c;
    long long cincl = cw;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      const long long co = __shfl_up(cincl, d);
      if (lane >= d) {
        incl += o;
        cincl += co;
      }
    }
    s_ppre[lane] = incl - c;
    s_cpre[lane] = cincl - cw;
    const bool anybig = __any(big);                // (a vote of every lane of the wave)
    if (lane == 63) {
      s_ppre[64] = anybig ? -1 : incl;
      s_cpre[64] = cincl;
    }
  }
  if (grouped && blockIdx.x == 0 && tid == 0 && a.invalid_count) *a.invalid_count = s_inv;
  __syncthreads();
  const bool counted = counting && s_ppre[64] >= 0;
  // passes in all: counted slots, one per slot, or the single slot's tokens
  const int npass = counted ? s_ppre[64] : (grouped ? a.num_slots : passes(a.M));
  // slot and pass of pass index pv (wave-uniform)
  auto decode = [&](int pv, int& e, int& g) {
    if (!grouped) {
      e = 0;
      g = pv;
      return;
    }
    if (!counted) {
      e = pv;
      g = 0;
      return;
    }
    // the last word starting at or before pv (word prefixes one per lane)
    const int lo = __popcll(__ballot(s_ppre[lane] <= pv)) - 1;
    // the word's slots one per lane (both half-waves alike): the first whose
    // inclusive pass count exceeds pv's place in the word
    const int rem = pv - s_ppre[lo];
    const int ps = s_pass[32 * lo + (lane & 31)];
    int incl = ps;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const int o = __shfl_up(incl, d, 32);
      if ((lane & 31) >= d) incl += o;
    }
    const int k = __builtin_ctzll(__ballot(incl > rem) & 0xFFFFFFFFull);
    e = 32 * lo + k;
    g = __builtin_amdgcn_readfirstlane(rem - (__shfl(incl, k) - __shfl(ps, k)));
  };
  // Work-groups take even shares of a cost axis on which each pass is a
  // set-up block (segu) followed by its tiles: a share that reaches into
  // another pass (one more segment set-up) takes fewer tiles, and tiles of
  // passes with more pairs count for more.  Tile j of a pass goes to the
  // work-group whose share holds its start.  Without counts every pass is
  // costed as one of G pairs.
  // ceil(x / d) and floor(x / d) for 0 <= x < 2^50, 0 < d < 2^31: a double
  // quotient corrected by one step either way (no 64-bit division)
  auto ceil_div = [&](int64_t x, int64_t d) {
    int64_t q = (int64_t)((double)x / (double)d);
    if (q * d < x) ++q;
    if (q > 0 && (q - 1) * d >= x) --q;
    return q;
  };
  auto floor_div = [&](int64_t x, int64_t d) {
    int64_t q = (int64_t)((double)x / (double)d);
    if (q * d > x) --q;
    if ((q + 1) * d <= x) ++q;
    return q;
  };
  auto tile_at = [&](int64_t rem, int pv, int n) {   // rem: cost into pass pv of n pairs
    const int64_t r = rem - segu, tc = (int64_t)S * (kChTileBase + n);
    return pv * tps + (r > 0 ? (int)ceil_div(r, tc) : 0);
  };
  // Both boundaries of this work-group's share at once: lanes 0..31 locate
  // cut c0 and lanes 32..63 cut c1, each half-wave scanning its own word (the
  // second locate no longer waits for the first).  A cut at or past the
  // total cost is the end; it is located as the last cost unit first, so
  // that every lane's scan and pass loop see a slot that holds its cut.
  auto locate2 = [&](int64_t c0, int64_t c1) {
    const bool hi = lane >= 32;
    const int64_t cut = hi ? c1 : c0;
    if (!counted) {
      const int64_t pc = segu + ts * (kChTileBase + G);
      const int64_t p = floor_div(cut, pc);
      return tile_at(cut - p * pc, (int)p, G);
    }
    const int64_t total = s_cpre[64];
    if (total == 0) return npass * tps;
    const int64_t d0 = min(c0, total - 1), d1 = min(c1, total - 1);
    const int64_t c = hi ? d1 : d0;
    // the last word starting at or before each cut (word prefixes one per lane)
    const long long wp = s_cpre[lane];
    const uint64_t b0 = __ballot(wp <= d0), b1 = __ballot(wp <= d1);
    const int lo = (int)__popcll(hi ? b1 : b0) - 1;
    // the word's slots one per lane of the half-wave: the first whose
    // inclusive cost exceeds the cut's place in the word
    int64_t rem = c - s_cpre[lo];
    const int sl = 32 * lo + (lane & 31);
    const int ps = s_pass[sl], n = (int)cnt[sl];
    int pincl = ps;
    long long cincl = slot_cost(ps, n);
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const int po = __shfl_up(pincl, d, 32);
      const long long co = __shfl_up(cincl, d, 32);
      if ((lane & 31) >= d) {
        pincl += po;
        cincl += co;
      }
    }
    const uint64_t m = __ballot(cincl > rem);
    const int k = hi ? 32 + __builtin_ctzll(m >> 32) : __builtin_ctzll(m & 0xFFFFFFFFull);
    const int psk = __shfl(ps, k), nk = __shfl(n, k);
    rem -= __shfl(cincl, k) - slot_cost(psk, nk);
    const int pv = s_ppre[lo] + __shfl(pincl, k) - psk;
    int g = 0, cg = min(G, nk);
    for (;; ++g) {                                 // the slot's pass that holds the cut
      cg = min(G, nk - g * G);
      const int64_t pcost = segu + ts * (kChTileBase + cg);
      if (rem < pcost || g == psk - 1) break;
      rem -= pcost;
    }
    return cut >= total ? npass * tps : tile_at(rem, pv + g, cg);
  };
  const int64_t C = counted ? s_cpre[64] : (int64_t)npass * (segu + ts * (kChTileBase + G));
  const int vv = locate2(floor_div((int64_t)blockIdx.x * C, NB), floor_div((int64_t)(blockIdx.x + 1) * C, NB));
  const int v1 = min(__builtin_amdgcn_readlane(vv, 32), npass * tps);
  const int v0 = min(__builtin_amdgcn_readlane(vv, 0), v1);

  // ---- per-lane constants ----
  const LineLanes lines = line_lanes(lane);
  const int rdo = ch_chunk(g4, cc) * 16;               // this lane's B-fragment chunk
  // this wave's position in unit order (pos = 2 * SIMD + second wave) and the
  // start of its share, in 1/4096 of a round's tiles
  const int pos = 2 * (wave & 3) + (wave >> 2);
  const int share = min(max(a.wave_share, kChShareMin), kChShareMax);
  auto xfrac = [&](int k) { return k >= kChWaves ? 4096 : (k >> 1) * 1024 + ((k & 1) ? share : 0); };
  // first and last tile that position k's share meets in a round of nt tiles
  auto tile_lo = [&](int k, int nt) { return xfrac(k) * nt / 4096; };
  auto tile_hi = [&](int k, int nt) { return min(xfrac(k + 1) * nt / 4096, nt - 1); };
  // where position k's share starts in an element of nt tiles and scc
  // steps: tile t, step s (the same tile fraction in every chunk, whole
  // passes), and as a unit index; shifts only, no division (the cursor runs
  // between weight loads, where a division's scratch registers would have to
  // wait for loads in flight)
  auto unit_pos = [&](int k, int nt, int scc, int& t, int& s) {
    const int num = xfrac(k) * nt;
    t = num >> 12;
    s = (((num & 4095) * scc) >> 12) & ~(kChU - 1);
  };
  static_assert(kChU == 2, "passes of two steps: unit_pos rounds down to even steps");
  auto unit_at = [&](int k, int nt, int scc) {
    int t, s;
    unit_pos(k, nt, scc, t, s);
    return t * scc + s;
  };
  // whole-line loads: lane L reads rows L / 8 and 8 + L / 8 of the tile
  auto row_off = [&](int t, int part) {
    const int row = t * RT + 8 * part + (lane >> 3);
    return (uint32_t)(row < I ? row : I - 1) * rbytes + 16u * (uint32_t)(lane & 7);
  };

  // Digits of one quad of x: 32 consecutive values of a group row (its 8-
  // value words j = 0..3, starting at value 32 qg of chunk step st, qg =
  // 2 k-group + q) in the operand order of split_planes.  Word j is dword j
  // of the 16-byte chunks of planes 2q (its even positions) and 2q + 1 (odd)
  // in the row's digit columns, so the quad fills whole chunks: one 16-byte
  // store per (column, plane), at fixed offsets from the row's first chunk
  // (columns col0 .. col0 + 3 of a four-column row lie in one 4-aligned
  // group, which the k-group's swizzle keeps together; an eight-column row
  // has two such groups).  A piece of NWD = 2 words is half h of a quad
  // (words 2h, 2h + 1): the same stores, 8 bytes each, at byte 8h of every
  // chunk.
  auto stage_piece = [&](auto nwd, uint8_t* buf, int W, int col0, int st, int qg, int h, const uint4 (&xq)[4],
                         int etop1) {
    constexpr int NWD = decltype(nwd)::value;
    const int gg = qg >> 1, q = qg & 1;
    const int bp = (col0 & 15) ^ (4 * gg);           // chunk position of column col0
    uint8_t* const b0 = buf + st * sbytes + (2 * q * NT + (col0 >> 4)) * 1024 + gg * 256 + bp * 16 + 8 * h;
    // one piece's digit sd of every word: a 16-byte (or 8-byte) store
    auto put = [&](uint8_t* at, uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3) {
      if constexpr (NWD == 4)
        *(uint4*)at = make_uint4(d0, d1, d2, d3);
      else
        *(uint2*)at = make_uint2(d0, d1);
    };
    auto vals = [&](const uint4 w, int par, uint32_t (&xs)[4]) {
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[e] = par ? u[e] >> 16 : u[e] & 0xFFFFu;
    };
    if (W == 4) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        uint32_t d[4][4] = {};                         // [word][digit]
#pragma unroll
        for (int wj = 0; wj < NWD; ++wj) {
          uint32_t xs[4], v[4];
          vals(xq[wj], par, xs);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = x_digits4(xs[e], etop1);
          transpose4(v[0], v[1], v[2], v[3], d[wj]);
        }
#pragma unroll
        for (int sd = 0; sd < 4; ++sd) put(b0 + par * NT * 1024 + 16 * sd, d[0][sd], d[1][sd], d[2][sd], d[3][sd]);
      }
    } else {
      // six digits: columns [d0 d1 d2 0 d3 d4 d5 0], the second group of
      // four at chunk position bp ^ 4
      uint8_t* const b1 = b0 + ((bp ^ 4) - bp) * 16;
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        uint32_t dl[4][4] = {}, dh[4][4] = {};
#pragma unroll
        for (int wj = 0; wj < NWD; ++wj) {
          uint32_t xs[4], lo[4], hi[4];
          vals(xq[wj], par, xs);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint64_t z = x_digits_nb(xs[e], etop1);
            lo[e] = (uint32_t)z;
            hi[e] = (uint32_t)(z >> 32);
          }
          transpose4(lo[0], lo[1], lo[2], lo[3], dl[wj]);
          transpose4(hi[0], hi[1], hi[2], hi[3], dh[wj]);
        }
        uint8_t* const p0 = b0 + par * NT * 1024;
        uint8_t* const p1 = b1 + par * NT * 1024;
#pragma unroll
        for (int sd = 0; sd < 3; ++sd) put(p0 + 16 * sd, dl[0][sd], dl[1][sd], dl[2][sd], dl[3][sd]);
        put(p0 + 48, 0, 0, 0, 0);
        put(p1, dl[0][3], dl[1][3], dl[2][3], dl[3][3]);
#pragma unroll
        for (int sd = 0; sd < 2; ++sd) put(p1 + 16 + 16 * sd, dh[0][sd], dh[1][sd], dh[2][sd], dh[3][sd]);
        put(p1 + 48, 0, 0, 0, 0);
      }
    }
  };

  // ---- segments: one pass over at most SEGT tiles of one slot ----
  int v = v0;
  while (v < v1) {
    const int pv = v / tps;                            // pass index
    const int t0 = v - pv * tps;
    const int t1 = min(min(v1 - pv * tps, tps), t0 + SEGT);
    v = pv * tps + t1;
    int e, g;
    decode(pv, e, g);
    const uint8_t* slot = a.slots + (uint64_t)e * a.slot_stride;
    const __amdgpu_buffer_rsrc_t gsrc = make_rsrc(slot + a.gate_w_off, wbytes);
    // DOWN: rows 16..31 of each tile are the same matrix 16 rows further on
    // (loads past its end return zeros, for rows that are never stored)
    const uint32_t skip = 16u * rbytes;
    const __amdgpu_buffer_rsrc_t usrc =
        DOWN ? make_rsrc(slot + a.gate_w_off + skip, wbytes > skip ? wbytes - skip : 0u)
             : make_rsrc(slot + a.up_w_off, wbytes);
    const float* gscale = (const float*)(slot + a.gate_s_off);
    const float* uscale = (const float*)(slot + a.up_s_off);
    const int nseg = t1 - t0;
    // the pass's pairs: indices [ilo, ihi) of the slot's pairs in id order
    const int ilo = counted || !grouped ? g * G : 0;
    const int ihi = counted || !grouped ? ilo + G : 0x7FFFFFFF;

    // ---- the segment's stream of (round, chunk) elements ----
    // With the whole K in LDS (one chunk) the segment is one round whose
    // tiles each wave finishes as it completes them; else rounds of at most
    // kChRoundTiles tiles whose sums stay in registers from chunk to chunk.
    const int nr = WHOLE ? 1 : (nseg + kChRoundTiles - 1) / kChRoundTiles;
    // first tile of round r (in the slot): rounds of near-equal size
    static_assert(WHOLE || SEGT <= 4 * kChRoundTiles, "at most four rounds per segment");
    auto round_at = [&](int r) {
      const int q = r * nseg;
      return t0 + (nr == 1 ? q : nr == 2 ? q >> 1 : nr == 3 ? q / 3 : q >> 2);
    };
    // element (r, c): round r's first tile and tile count, chunk c's steps,
    // and this wave's unit range [ua, ub) in (tile, step) order
    auto elem = [&](int r, int c, int& ta, int& nt, int& scc, int& s0, int& ua, int& ub) {
      ta = round_at(r);
      nt = round_at(r + 1) - ta;
      s0 = c * Sc;
      scc = min(Sc, S - s0);
      ua = unit_at(pos, nt, scc);
      ub = unit_at(pos + 1, nt, scc);
    };

    // ---- weight load cursor: element (cr, cch), unit cu of [.., cub) ----
    int cr = 0, cch = 0, cu = 0, cub = 0, cscc = 1, cs0 = 0, lt = 0, lsc = 0;
    uint32_t loff = 0, loff2 = 0;
    auto next_elem = [&]() {
      if (++cch == nch) {
        cch = 0;
        ++cr;
      }
    };
    auto seek = [&]() {                                // to the first unit of element (cr, cch) or later
      while (cr < nr) {
        int ta, nt, ua, ub;
        elem(cr, cch, ta, nt, cscc, cs0, ua, ub);
        if (ua < ub) {
          int t, st;
          unit_pos(pos, nt, cscc, t, st);
          cu = ua;
          cub = ub;
          lt = ta + t;
          lsc = st;
          loff = row_off(lt, 0);
          loff2 = row_off(lt, 1);
          return;
        }
        next_elem();
      }
    };
    // always four loads per call (offsets past the weights once this wave's
    // units are all issued: the cursor is past the last element), so that the
    // compiler's wait counts stay exact
    auto issue = [&](StepW<true>& gw, StepW<true>& uw, uint32_t dep) {
      const bool live = cr < nr;
      const uint32_t so = (uint32_t)(cs0 + lsc) * 128u;
      const uint32_t o = (live ? loff + so : kOffNone) + dep;
      const uint32_t o2 = (live ? loff2 + so : kOffNone) + dep;
      load_line<VEC>(gw, gsrc, o, o2);
      load_line<VEC>(uw, usrc, o, o2);
      if (live) {
        if (++cu == cub) {
          next_elem();
          seek();
        } else if (++lsc == cscc) {
          lsc = 0;
          ++lt;
          loff = row_off(lt, 0);
          loff2 = row_off(lt, 1);
        }
      }
    };
    StepW<true> rg[kChD], ru[kChD], sg, su;
    // the next unit's weights, moved out of their ring slot into the tile
    // layout, and the slot refilled at once (see the resident kernel)
    auto take = [&](int sl) {
      sg = rg[sl];
      su = ru[sl];
      line_to_tile(sg, lines);
      line_to_tile(su, lines);
      uint32_t dep = 0u;
      asm volatile("" : "+v"(dep) : "v"(sg.a), "v"(sg.b), "v"(su.a), "v"(su.b));
      issue(rg[sl], ru[sl], dep);
    };
    // the stream from its start: the first weights go out before the group's
    // pairs, ranges and digits are known (the addresses depend on none of them)
    auto stream_start = [&]() {
      cr = 0;
      cch = 0;
      seek();
#pragma unroll
      for (int d = 0; d < kChD; ++d) issue(rg[d], ru[d], 0u);
    };
    stream_start();

    int done = 0;                                      // pairs of the pass already processed
    for (;;) {
      __syncthreads();  // the previous group is done with the group tables and digits
      // ---- next group: the pass's pairs [start, start + G) ----
      const int start = ilo + done;
      const int stop = min(ihi, start + G);
      int count, more;
      if (!grouped) {
        count = max(0, min(stop, P) - start);
        more = start + count < min(ihi, P);
        if (tid < count) s_pairs[tid] = start + tid;
        __syncthreads();
      } else {
        // block-wide scan of the ids in windows of kChThreads, counting the
        // slot's pairs in id order; stops once it has seen past `stop`.  Ids
        // held in registers and ids read from memory take separate loops (one
        // merged loop would wait for every load in flight at each compare).
        int found = 0;
        auto window = [&](int base, bool m) {
          const uint64_t bal = __ballot(m);
          if (lane == 0) s_wcnt[wave] = __popcll(bal);
          __syncthreads();
          int before = found;
#pragma unroll 1
          for (int w = 0; w < wave; ++w) before += s_wcnt[w];
          int total = found;
#pragma unroll 1
          for (int w = 0; w < kChWaves; ++w) total += s_wcnt[w];
          before += __popcll(bal & ((1ull << lane) - 1ull));
          if (m && before >= start && before < stop) s_pairs[before - start] = base + tid;
          found = total;
          __syncthreads();  // s_wcnt reused; s_pairs visible
          return found > stop;
        };
#pragma unroll
        for (int j = 0; j < kChIdRegs; ++j)
          if (j * kChThreads < P && !(j > 0 && found > stop))
            if (window(j * kChThreads, idr[j] == e)) break;
        if (found <= stop)
          for (int base = kChIdRegs * kChThreads; base < P; base += kChThreads)
            if (window(base, base + tid < P && a.ids[base + tid] == e)) break;
        count = max(0, min(found, stop) - start);
        more = start + count < min(ihi, found);
      }
      if (count <= 0) break;

      // ---- range of each row of the group (row `wave`, G < kChWaves):
      // largest |x|, smallest exponent; four loads in flight per lane ----
      static_assert(G <= kChWaves, "one wave per row of a group");
      if (wave < count) {
        const int tok = __builtin_amdgcn_readfirstlane(s_pairs[wave] / K);
        const uint4* row = (const uint4*)(a.x + (uint64_t)tok * H);
        uint32_t mx = 0, mn = 255;
        auto acc = [&](const uint4 xq) {
          uint32_t m1, n1;
          range8(xq, m1, n1);
          mx = max(mx, m1);
          mn = min(mn, n1);
        };
        int u = lane;
        for (; u + 192 < hw; u += 256) {
          const uint4 q0 = row[u], q1 = row[u + 64], q2 = row[u + 128], q3 = row[u + 192];
          acc(q0);
          acc(q1);
          acc(q2);
          acc(q3);
        }
        for (; u < hw; u += 64) acc(row[u]);
        mx = wave_extreme<true>(mx);
        mn = wave_extreme<false>(mn);
        if (lane == 0) {
          s_tok[wave] = tok;
          s_xmax[wave] = (int)mx;
          s_xmin[wave] = (int)mn;
        }
      }
      // row scales of the segment
      for (int i = tid; i < nseg * RT; i += kChThreads) {
        const int row = t0 * RT + i;
        s_gsc[i] = row < I ? gscale[row] : 0.0f;
        if constexpr (!DOWN) s_usc[i] = row < I ? uscale[row] : 0.0f;
      }
      __syncthreads();
      // Digit columns: four per row when all its values lie within 22
      // binades of its largest, else eight ([d0 d1 d2 0 d3 d4 d5 0]).  Eight-
      // column rows take the first 8-aligned columns, four-column rows the
      // rest; the group is the longest run of its pairs that fits 16*NT
      // columns (the rest go to the next group).  Lane ti of every wave reads
      // row ti's range, a ballot gives the eight-column rows, and row ti's
      // thread and quad q's thread store the layout.
      const bool w8l = lane < count && digits_for(s_xmax[lane], s_xmin[lane]) != 4;
      const uint32_t wall = (uint32_t)__ballot(w8l);   // rows of eight columns (G <= 32)
      // rows 0..ti take 4 (ti + 1) + 4 (eight-column rows among them) columns
      const bool okl = lane < count && 4 * (lane + 1) + 4 * __popc(wall & ((2u << lane) - 1u)) <= 16 * NT;
      const int fit = __builtin_amdgcn_readfirstlane(__popcll(__ballot(okl)));  // a prefix of the rows
      const uint32_t wmask = __builtin_amdgcn_readfirstlane(wall & ((1u << fit) - 1u));
      const int n8 = __builtin_amdgcn_readfirstlane(__popc(wmask));
      if (fit < count) {
        count = fit;
        more = 1;
      }
      auto nth_row = [&](uint32_t w, int j) {          // the j-th set bit of w
        for (int k = 0; k < j; ++k) w &= w - 1u;
        return (int)__builtin_ctz(w);
      };
      if (tid < count) {
        const bool wide = (wmask >> tid) & 1u;
        const int b8 = __popc(wmask & ((1u << tid) - 1u));
        const int q0 = wide ? 2 * b8 : 2 * n8 + (tid - b8);  // first quad of the row
        s_col[tid] = 4 * q0;
        s_wid[tid] = wide ? 8 : 4;
      }
      if (tid < 4 * NT) {
        int myq = -1;
        if (tid < 2 * n8)
          myq = nth_row(wmask, tid >> 1) + ((tid & 1) ? 64 : 0);
        else if (tid - 2 * n8 < count - n8)
          myq = nth_row(~wmask & ((1u << count) - 1u), tid - 2 * n8);
        s_quad[tid] = myq;
      }
      __syncthreads();

      // Piece xs of chunk c: pieces in row-major order (xs = tl * np + p for
      // np pieces per row in the chunk), so that a wave's pieces mostly share
      // a row (and its digit width).  A piece is a quad (hs = 0: p = r = 8 st
      // + qg) or, when a chunk has too few quads for every lane of the work-
      // group, half a quad (hs = 1: p = 2 r + h), which halves each lane's
      // split.  Words past the row's end (padding steps) are loaded from its
      // start and replaced by zeros when they are split, not here (a write to
      // the loads' registers would have to wait for them at once).
      auto piece_k = [&](int c, int p, int hs) { return c * Sc * 256 + (p << (5 - hs)); };
      auto load_piece = [&](int c, int p, int hs, int tl, uint4 (&xq)[4]) {
        const int k0 = piece_k(c, p, hs);
        const uint16_t* row = a.x + (uint64_t)s_tok[tl] * H;
#pragma unroll
        for (int wj = 0; wj < 4; ++wj)
          if (wj < (4 >> hs)) xq[wj] = *(const uint4*)(row + (k0 + 8 * wj < H ? k0 + 8 * wj : 0));
      };
      auto put_piece = [&](uint8_t* buf, int c, int p, int hs, int tl, uint4 (&xq)[4]) {
        const int k0 = piece_k(c, p, hs);
#pragma unroll
        for (int wj = 0; wj < 4; ++wj)
          if (k0 + 8 * wj >= H) xq[wj] = make_uint4(0, 0, 0, 0);
        const int r = p >> hs, etop1 = max((s_xmax[tl] >> 7) & 0xFF, 1);
        if (hs)
          stage_piece(std::integral_constant<int, 2>(), buf, s_wid[tl], s_col[tl], r >> 3, r & 7, p & 1, xq, etop1);
        else
          stage_piece(std::integral_constant<int, 4>(), buf, s_wid[tl], s_col[tl], r >> 3, r & 7, 0, xq, etop1);
      };
      // half-quad pieces when a chunk of nq quads per row has at most one
      // quad for every two threads
      auto piece_shift = [&](int nq) { return count * nq * 2 <= kChThreads ? 1 : 0; };
      // chunk 0 of the group, by every thread
      {
        const int hs0 = piece_shift(min(Sc, S) * 8);
        const int np0 = (min(Sc, S) * 8) << hs0;
        for (int xs = tid; xs < count * np0; xs += kChThreads) {
          const int tl = xs / np0, pc = xs - tl * np0;
          uint4 xq[4];
          load_piece(0, pc, hs0, tl, xq);
          put_piece(s_dig, 0, pc, hs0, tl, xq);
        }
      }
      __syncthreads();
      take(0);

      // ---- a finished tile (tseg of the segment) with its sums in ag/au:
      // fix-up with the other `ncon` contributors (slot `first`), then the
      // (row, pair) sums, F32 rounding, SwiGLU tail and stores ----
      auto finish_tile = [&](int tseg, int first, int ncon, const v4i* ag, const v4i* au) {
        int64_t gq[NT], uq[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          gq[n] = quad_digit_sum(ag[n], qj);
          uq[n] = quad_digit_sum(au[n], qj);
        }
        if (ncon > 1) {
          // first < kChFixSlots: a shared tile is the last one its first
          // contributor meets, and a later position meets it too
          unsigned long long* fx = s_fix + first * ch_fix_words(NT) + lane;
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            atomicAdd(&fx[(2 * n) * 64], (unsigned long long)gq[n]);
            atomicAdd(&fx[(2 * n + 1) * 64], (unsigned long long)uq[n]);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          int prev = 0;
          if (lane == 0) prev = atomicAdd(&s_fixcnt[first], 1);
          prev = __shfl(prev, 0);
          if (prev != ncon - 1) return;
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            gq[n] = (int64_t)fx[(2 * n) * 64];
            uq[n] = (int64_t)fx[(2 * n + 1) * 64];
            fx[(2 * n) * 64] = 0;
            fx[(2 * n + 1) * 64] = 0;
          }
          if (lane == 0) s_fixcnt[first] = 0;
        }
        const int row = (t0 + tseg) * RT + 4 * g4 + qj;
        const int si = tseg * RT + 4 * g4 + qj;        // scale index in the segment
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          // the row of this lane's quad; an 8-column row's quads are [d0 d1
          // d2 0] and [d3 d4 d5 0], the high half of the sum from the next quad
          const int qv = s_quad[4 * n + (cc >> 2)];
          const int64_t gx = __shfl_xor(gq[n], 4), ux = __shfl_xor(uq[n], 4);
          if (qv < 0 || qv >= 64 || row >= I) continue;
          const int tq = qv;
          const bool w8 = s_wid[tq] == 8;
          const int xm = s_xmax[tq];
          const float gs = s_gsc[si];
          const float us = DOWN ? s_gsc[si + 16] : s_usc[si];
          float gate, up;
          if (!w8) {
            const int e2 = sum_exponent(xm) + 16;
            gate = round_scaled53(gq[n], e2, gs);
            up = round_scaled53(uq[n], e2, us);
          } else {
            const int e2 = sum_exponent(xm);
            gate = round_scaled(gx, gq[n], e2, gs);
            up = round_scaled(ux, uq[n], e2, us);
          }
          if (xm >= 0x7F80) {
            gate = __builtin_nanf("");
            up = __builtin_nanf("");
          }
          const uint64_t o = (uint64_t)s_pairs[tq] * I + row;
          if constexpr (DOWN) {
            a.out[o] = bf16_rne(gate);
            if (a.gate_probe) a.gate_probe[o] = gate;
            if (row + 16 < I) {
              a.out[o + 16] = bf16_rne(up);
              if (a.gate_probe) a.gate_probe[o + 16] = up;
            }
          } else {
            a.out[o] = swiglu_tail_tab(gate, up, s_sig);
            if (a.gate_probe) a.gate_probe[o] = gate;
            if (a.up_probe) a.up_probe[o] = up;
          }
        }
      };
      // one pass of the step loop (kChU steps) into ag/au, B fragments of
      // chunk steps sl.. of digit buffer buf; `slice` runs after the take of
      // the pass's last step
      auto steps = [&](const uint8_t* buf, int sl, v4i* ag, v4i* au, auto&& slice) {
#pragma unroll
        for (int jj = 0; jj < kChU; ++jj) {
          v4i pg[4], pu[4];
          split_planes(sg.a, sg.b, pg);
          split_planes(su.a, su.b, pu);
          take((jj + 1) % kChD);
          if (jj == kChU - 1) slice();
          const uint8_t* bp = buf + (sl + jj) * sbytes + rdo;
          v4i bq[4][NT];
#pragma unroll
          for (int pl = 0; pl < 4; ++pl)
#pragma unroll
            for (int n = 0; n < NT; ++n) bq[pl][n] = *(const v4i*)(bp + (pl * NT + n) * 1024);
#pragma unroll
          for (int pl = 0; pl < 4; ++pl)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              ag[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pg[pl], bq[pl][n], ag[n], 0, 0, 0);
              au[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pu[pl], bq[pl][n], au[n], 0, 0, 0);
            }
        }
      };

      if constexpr (WHOLE) {
        // ---- the whole K in LDS: portions (the rest of a tile inside this
        // wave's range), each tile finished as its last step is done ----
        int ta, nt, scc, s0, ua, ub;
        elem(0, 0, ta, nt, scc, s0, ua, ub);
        int w, st0;                                    // tile of the segment, and the step the range starts at
        unit_pos(pos, nseg, S, w, st0);
        for (int u = ua; u < ub; ++w) {
          const int pe = min(ub, (w + 1) * S);
          const bool full = u == w * S && pe == (w + 1) * S;
          v4i ag[NT], au[NT];
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            ag[n] = v4i{0, 0, 0, 0};
            au[n] = v4i{0, 0, 0, 0};
          }
          for (; u < pe; u += kChU) steps(s_dig, u - w * S, ag, au, [] {});
          // contributors: the positions whose ranges meet the tile
          int first = pos, ncon = 1;
          if (!full) {
            first = -1;
            ncon = 0;
            for (int k = 0; k < kChWaves; ++k) {
              const int b0 = unit_at(k, nseg, S), b1 = unit_at(k + 1, nseg, S);
              if (b0 < b1 && b0 < (w + 1) * S && b1 > w * S) {
                if (first < 0) first = k;
                ++ncon;
              }
            }
          }
          finish_tile(w, first, ncon, ag, au);
        }
      } else {
        v4i accg[kChMaxT][NT], accu[kChMaxT][NT];
        for (int r = 0; r < nr; ++r)
        for (int c = 0; c < nch; ++c) {
          const int k = r * nch + c;                   // element index: digit buffer k % 2
          int ta, nt, scc, s0, ua, ub;
          elem(r, c, ta, nt, scc, s0, ua, ub);
          const int tf = tile_lo(pos, nt);            // first tile this wave meets in the round
          if (c == 0) {
#pragma unroll
            for (int j = 0; j < kChMaxT; ++j)
#pragma unroll
              for (int n = 0; n < NT; ++n) {
                accg[j][n] = v4i{0, 0, 0, 0};
                accu[j][n] = v4i{0, 0, 0, 0};
              }
          }
          const uint8_t* buf = s_dig + (k & 1) * kChBuf;
          // this wave's share of element k+1's digits: pieces [xs, xe) of
          // chunk c1, one slice (64 pieces, one per lane) per pass of the step
          // loop
          const bool stg = k + 1 < nr * nch;
          const int c1 = c + 1 == nch ? 0 : c + 1;
          uint8_t* sbuf = s_dig + ((k + 1) & 1) * kChBuf;
          const int hs1 = piece_shift(min(Sc, S - c1 * Sc) * 8);
          const int nq1 = (min(Sc, S - c1 * Sc) * 8) << hs1;  // pieces per row in chunk c1
          const int xpn = stg ? count * nq1 : 0;
          int xs = wave * xpn / kChWaves + lane;
          const int xe = (wave + 1) * xpn / kChWaves;
          // A slice's x is loaded after the take at a pass's last step and
          // split into LDS at the same point of the next pass: the take there
          // has waited for every weight load issued before the x loads, so the
          // wait for x covers nothing still in flight for the ring.
          uint4 xq[4] = {};
          int rp = 0, tlp = 0;                         // the pending slice's piece
          bool pend = false;
          auto slice = [&]() {
            if (pend) put_piece(sbuf, c1, rp, hs1, tlp, xq);
            pend = xs < xe;
            if (pend) {
              tlp = xs / nq1;
              rp = xs - tlp * nq1;
              load_piece(c1, rp, hs1, tlp, xq);
              xs += 64;
            }
          };
#pragma unroll
          for (int j = 0; j < kChMaxT; ++j) {
            const int tile = tf + j;                   // tile of the round
            const int pa = max(ua, tile * scc), pb = min(ub, (tile + 1) * scc);
            for (int u = pa; u < pb; u += kChU) steps(buf, u - tile * scc, accg[j], accu[j], slice);
          }
          if (pend) put_piece(sbuf, c1, rp, hs1, tlp, xq);
          // the rest of this wave's share (rounds too short for all its slices)
          while (xs < xe) {
            tlp = xs / nq1;
            rp = xs - tlp * nq1;
            load_piece(c1, rp, hs1, tlp, xq);
            put_piece(sbuf, c1, rp, hs1, tlp, xq);
            xs += 64;
          }
          __syncthreads();  // element k's digits read, element k+1's staged
          if (c != nch - 1) continue;
          // ---- the round's tiles this wave met ----
          const int tl_last = tile_hi(pos, nt);
#pragma unroll
          for (int j = 0; j < kChMaxT; ++j) {
            const int tile = tf + j;
            if (tile > tl_last) continue;
            int first = -1, ncon = 0;
            for (int kk = 0; kk < kChWaves; ++kk) {
              if (tile_lo(kk, nt) <= tile && tile <= tile_hi(kk, nt)) {
                if (first < 0) first = kk;
                ++ncon;
              }
            }
            finish_tile(ta - t0 + tile, first, ncon, accg[j], accu[j]);
          }
        }
      }
      done += count;
      if (!more) break;
      stream_start();                                  // the next group streams the segment again
    }
  }

  // ---- pairs with invalid ids get zero outputs: pairs b, b + NB, ... here
  // (skipped, with its barriers and id reloads, when the call has none) ----
  if (grouped && s_inv > 0) {
    const int nmine = P > (int)blockIdx.x ? (P - (int)blockIdx.x + NB - 1) / NB : 0;
    for (int base = 0; base < nmine; base += kChThreads) {
      __syncthreads();
      if (tid == 0) s_ninv = 0;
      __syncthreads();
      const int i = base + tid;
      const int p = (int)blockIdx.x + i * NB;
      const bool bad = i < nmine && (a.ids[p] < 0 || a.ids[p] >= a.num_slots);
      int at = -1;
      if (bad) at = atomicAdd(&s_ninv, 1);
      if (bad && at < kChInvBatch) s_invl[at] = p;
      __syncthreads();
      const int nl = min(s_ninv, kChInvBatch);
      for (int q = 0; q < nl; ++q) {
        const int pq = s_invl[q];
        for (int r = tid; r < I; r += kChThreads) {
          const uint64_t o = (uint64_t)pq * I + r;
          a.out[o] = 0;
          if (a.gate_probe) a.gate_probe[o] = 0.0f;
          if (a.up_probe) a.up_probe[o] = 0.0f;
        }
      }
      // past the batch: each finder fills its own pair
      if (bad && at >= kChInvBatch)
        for (int r = 0; r < I; ++r) {
          const uint64_t o = (uint64_t)p * I + r;
          a.out[o] = 0;
          if (a.gate_probe) a.gate_probe[o] = 0.0f;
          if (a.up_probe) a.up_probe[o] = 0.0f;
        }
    }
  }
}

// ---- host side ----

namespace {

template <int NT, bool VEC, bool DOWN, bool WHOLE>
int chunked_blocks(int device) {
  // per-device cache; concurrent first calls compute the same value
  static std::atomic<int> cached[64];
  if (device < 0 || device >= 64) device = 0;
  if (!cached[device].load(std::memory_order_relaxed)) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&chunked_kernel<NT, VEC, DOWN, WHOLE>), kChThreads, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    cached[device].store(cus * per_cu, std::memory_order_relaxed);
  }
  return cached[device].load(std::memory_order_relaxed);
}

template <int NT, bool VEC, bool DOWN, bool WHOLE>
hipError_t launch_chunked_t(GateUpParams& p, hipStream_t stream) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  const int rt = DOWN ? 32 : 16;
  const int tiles = p.num_slots * ((p.I + rt - 1) / rt);
  int nb = chunked_blocks<NT, VEC, DOWN, WHOLE>(device);
  if (nb > tiles) nb = tiles;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&chunked_kernel<NT, VEC, DOWN, WHOLE>), dim3((unsigned)nb),
                         dim3(kChThreads), args, 0, stream);
}

template <int NT, bool DOWN>
hipError_t launch_chunked_n(GateUpParams& p, hipStream_t stream) {
  const bool vec = (p.H / 2) % 16 == 0;
  const bool whole = ch_chunk_steps(NT, p.steps) == p.steps;
  if (whole)
    return vec ? launch_chunked_t<NT, true, DOWN, true>(p, stream) : launch_chunked_t<NT, false, DOWN, true>(p, stream);
  return vec ? launch_chunked_t<NT, true, DOWN, false>(p, stream) : launch_chunked_t<NT, false, DOWN, false>(p, stream);
}

template <bool DOWN>
hipError_t launch_chunked_d(GateUpParams& p, int nt, hipStream_t stream) {
  return nt == 1 ? launch_chunked_n<1, DOWN>(p, stream) : launch_chunked_n<2, DOWN>(p, stream);
}

}  // namespace

int chunked_tiles(const GateUpParams& p) {
  if (p.q8 || p.xf32) return 0;
  // single expert: its tokens; grouped: the routed pairs per slot on average
  // (over all slots: routing often touches a few), two column tiles except
  // for a down projection of one row per slot
  if (!p.ids) return p.M <= 2 ? 1 : (p.M <= 8 ? 2 : 0);
  const int64_t pairs = (int64_t)p.M * p.K;
  const int64_t per_slot = (pairs + p.num_slots - 1) / p.num_slots;
  if (per_slot > 6) return 0;
  return p.down && per_slot <= 1 ? 1 : 2;
}

hipError_t launch_chunked(GateUpParams p, int nt, hipStream_t stream) {
  p.steps = ch_steps(p.H);
  // a SIMD's first-wave share, 1/1024 of the SIMD's quarter, as measured on
  // this kernel: one column tile 550 (490, 520, 577 and 585 slower on the down
  // projection), two 580 (512 and 547 slower on the routed step)
  p.wave_share = nt == 1 ? 550 : 580;
  // a segment's set-up (id scan, row ranges, first digits, the first weights'
  // latency), in K-steps of a one-pair tile: a fixed part and one that grows
  // with the row length (the range pass reads whole rows); fitted to interleaved
  // runs of the down projection (6 steps: 64 best of 0..128), the routed step
  // (24: 128 of 96..192) and the large shape at four tokens (28: 192 of 96..192)
  p.seg_cost = 40 + 4 * p.steps;
  return p.down ? launch_chunked_d<true>(p, nt, stream) : launch_chunked_d<false>(p, nt, stream);
}

}  // namespace q4
