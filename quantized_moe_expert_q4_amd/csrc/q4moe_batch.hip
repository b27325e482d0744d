// Q4 gate/up + SwiGLU for wide token groups (verify / prefill widths).
//
// Arithmetic: GATE_UP_SOURCE of the @mlx-bun/inference 1.0.0 diff, page 52
// (kernels/glm52/streamed-experts.ts), made exact as in q4moe_device.h.
//
// A group of up to G = 16*NT/6 tokens has C = L*count digit columns, with
// L = 4 digits per value when every value of the group's tokens lies within
// 22 binades of its token's largest (exact, see digits_for) and L = 6
// otherwise.  For the whole K the digits do not fit LDS in general, so the
// sixteen waves of a work-group move through K together, one K-chunk at a
// time:
//  * One persistent launch, one 1024-thread work-group per CU: work-group b
//    takes the whole 16-row tiles [bT/NB, (b+1)T/NB); it walks them in
//    batches of sixteen (one tile per wave), so the per-CU weight bytes
//    differ by at most one tile.
//  * Per batch the K-steps are cut into chunks; chunk c+1's digits are split
//    from x into one half of a double-buffered LDS area while the waves
//    multiply chunk c out of the other half (one barrier per chunk).  When
//    one chunk covers K, the digits are staged once per token group.
//  * Each wave keeps two K-steps of weights in flight in a register ring that
//    runs on across chunk barriers and into its next batch's tile.
//  * Each wave's 16 x C digit matrix goes through the LDS buffer left idle
//    after the batch's last chunk, and its lanes recombine (row, token) sums
//    exactly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "q4moe_device.h"
#include "q4moe_launch.h"

namespace q4 {

namespace {

constexpr int kBatWaves = 16;
constexpr int kBatThreads = kBatWaves * 64;
constexpr int kBatBuf = 72 * 1024;        // one of two digit buffers
constexpr int kEpStride = 52;             // int32 row stride of a wave's 16 x C epilogue matrix
constexpr int kBatBitSlots = 2048;        // slots a routing bitmap covers
constexpr int kBatBitWords = kBatBitSlots / 32;
constexpr int kBatInvBatch = 64;          // invalid pairs zero-filled per batch

static_assert(kBatWaves * 16 * kEpStride * 4 <= kBatBuf, "epilogue matrices fit one digit buffer");

// Digits of one K-step: [parity 2][column tile n][lane 64][16 bytes], lane =
// 16*k-group + column in tile: every B fragment is one lane-linear 1 KiB read.
__host__ __device__ constexpr int bat_step_bytes(int ntiles) { return 2 * ntiles * 1024; }

// K-steps per chunk for `ntiles` column tiles and S (even) steps: chunks of
// equal even length.
__host__ __device__ inline int bat_chunk_steps(int ntiles, int S) {
  int mx = kBatBuf / bat_step_bytes(ntiles);
  mx -= mx & 1;
  if (mx < 2) mx = 2;
  const int n = (S + mx - 1) / mx;
  int spc = (S + n - 1) / n;
  spc += spc & 1;
  return spc;
}

}  // namespace

// DOWN: the down projection (one matrix of a.I rows over a.H inputs; a tile is
// 32 rows, its first 16 taking the gate role and the next 16 the up role,
// each output rounded to bf16 on its own) instead of gate/up + SwiGLU.
// Q8: signed int8 weights, one byte per weight (else packed nibbles).
// XF: f32 activations and outputs (else bf16).
template <int NT, bool VEC, bool DOWN, bool Q8, bool XF>
__global__ __launch_bounds__(kBatThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void batch_kernel(const GateUpParams a) {
  // pairs per token group: up to 16*NT/4 (four digits), trimmed to 16*NT/6
  // once the group's tokens turn out to need six
  constexpr int G = (16 * NT) / 4;
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[2 * kBatBuf];  // two digit buffers, or one spanning both
  __shared__ int s_pairs[G];
  __shared__ int s_tok[G];                   // token (x row) of each pair of the group
  __shared__ int s_xmax[G];
  __shared__ int s_xmin[G];                  // smallest non-zero exponent field of each token
  __shared__ int s_wcnt[kBatWaves];
  __shared__ int s_invalid;
  __shared__ int s_ninv;
  __shared__ int s_invl[kBatInvBatch];
  __shared__ uint32_t s_bits[kBatBitWords];  // routed slots
  __shared__ int s_bpre[kBatBitWords + 1];   // routed slots before each word, and in all
  __shared__ __attribute__((aligned(16))) uint16_t s_sig[kSigTable];  // bf16 sigmoid of the tabulated gT

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, cc = lane & 15;
  const int H = a.H, I = a.I;
  const int P = a.M * a.K;
  const bool grouped = a.ids != nullptr;
  constexpr bool xf = XF;
  const int S = a.steps;                     // K-steps per tile, even
  constexpr int RT = DOWN ? 32 : 16;         // rows per tile
  const int tps = (I + RT - 1) / RT;
  const int NB = gridDim.x;
  const uint32_t rbytes = row_bytes<Q8>(H);  // bytes of one weight row
  const uint32_t wbytes = (uint32_t)((uint64_t)I * rbytes);

  // the device's sigmoid table, 16 bytes per thread of the first half
  if constexpr (!DOWN)
    if (tid < kSigTable / 8) *(uint4*)(s_sig + 8 * tid) = ((const uint4*)a.sig)[tid];

  // ---- invalid routing ids (grouped): counted and zero-filled by work-group
  // 0, a batch of them at a time with every thread on a row range ----
  if (grouped && blockIdx.x == 0) {
    auto zero = [&](uint64_t o) {
      if (xf)
        ((float*)a.out)[o] = 0.0f;
      else
        a.out[o] = 0;
      if (a.gate_probe) a.gate_probe[o] = 0.0f;
      if (a.up_probe) a.up_probe[o] = 0.0f;
    };
    if (tid == 0) s_invalid = 0;
    for (int base = 0; base < P; base += kBatThreads) {
      __syncthreads();
      if (tid == 0) s_ninv = 0;
      __syncthreads();
      const int p = base + tid;
      const bool bad = p < P && (a.ids[p] < 0 || a.ids[p] >= a.num_slots);
      int at = -1;
      if (bad) at = atomicAdd(&s_ninv, 1);
      if (bad && at < kBatInvBatch) s_invl[at] = p;
      __syncthreads();
      const int nl = min(s_ninv, kBatInvBatch);
      if (tid == 0) s_invalid += s_ninv;
      for (int q = 0; q < nl; ++q)
        for (int r = tid; r < I; r += kBatThreads) zero((uint64_t)s_invl[q] * I + r);
      // past the batch: each finder fills its own pair
      if (bad && at >= kBatInvBatch)
        for (int r = 0; r < I; ++r) zero((uint64_t)p * I + r);
    }
    __syncthreads();
    if (tid == 0 && a.invalid_count) *a.invalid_count = s_invalid;
  }

  // ---- routed slots: a grouped call over at most kBatBitSlots slots cuts
  // only the tiles of the slots its ids name (T = routed slots x tiles per
  // slot) into whole-tile ranges; the bitmap of routed slots and its word
  // prefix counts stay in LDS ----
  const bool compact = grouped && a.num_slots <= kBatBitSlots;
  int R = grouped ? a.num_slots : 1;
  if (compact) {
    const int nw = (a.num_slots + 31) >> 5;
    if (tid < kBatBitWords) s_bits[tid] = 0u;
    __syncthreads();
    for (int p = tid; p < P; p += kBatThreads) {
      const int id = a.ids[p];
      if (id >= 0 && id < a.num_slots) atomicOr(&s_bits[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
    // routed slots before word l, by wave 0
    if (wave == 0) {
      const int c = lane < nw ? (int)__popc(s_bits[lane]) : 0;
      int incl = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      s_bpre[lane] = incl - c;
      if (lane == 63) s_bpre[64] = incl;
    }
    __syncthreads();
    R = s_bpre[64];
  }
  // slot of routed index r (wave-uniform): the word whose prefix brackets r,
  // then the bit within it (LDS reads only, once per slot segment)
  auto select = [&](int r) {
    if (!compact) return r;
    int lo = 0;
#pragma unroll
    for (int step = 32; step > 0; step >>= 1)
      if (s_bpre[lo + step] <= r) lo += step;
    uint32_t bits = s_bits[lo];
    for (int j = r - s_bpre[lo]; j > 0; --j) bits &= bits - 1u;
    return 32 * lo + (int)__builtin_ctz(bits);
  };
  const int T = R * tps;
  const int v0 = (int)((int64_t)blockIdx.x * T / NB), v1 = (int)((int64_t)(blockIdx.x + 1) * T / NB);

  int v = v0;
  while (v < v1) {
    const int ri = v / tps;                            // routed index of the slot
    const int t0 = v - ri * tps;
    const int t1 = min(v1, (ri + 1) * tps) - ri * tps;
    v = ri * tps + t1;
    const int e = select(ri);
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

    int next_pair = 0;
    int idv = -1;                                      // ids of the scan window at next_pair
    if (grouped && tid < P) idv = a.ids[tid];
    for (;;) {
      __syncthreads();  // previous group done with s_b and s_pairs
      if (tid < G) {
        s_xmax[tid] = 0;
        s_xmin[tid] = 255;
      }
      // ---- next group of up to G pairs routed to slot e ----
      int count, more;
      if (!grouped) {
        count = min(G, P - next_pair);
        more = next_pair + count < P;
        if (tid < count) s_pairs[tid] = next_pair + tid;
        __syncthreads();
      } else {
        // block-wide scan of ids[next_pair..P) in windows of kBatThreads;
        // stops once a further match proves there is another group
        int found = 0;
        int base = next_pair;
        more = 0;
        for (;;) {
          const bool m = idv == e;
          const uint64_t bal = __ballot(m);
          if (lane == 0) s_wcnt[wave] = __popcll(bal);
          __syncthreads();
          int before = found;
#pragma unroll 1
          for (int w = 0; w < wave; ++w) before += s_wcnt[w];
          int total = before;
#pragma unroll 1
          for (int w = wave; w < kBatWaves; ++w) total += s_wcnt[w];
          before += __popcll(bal & ((1ull << lane) - 1ull));
          if (m && before < G) s_pairs[before] = base + tid;
          found = total;
          base += kBatThreads;
          if (found > G) more = 1;
          __syncthreads();  // s_wcnt reused; s_pairs visible
          if (more || base >= P) break;
          idv = (base + tid < P) ? a.ids[base + tid] : -1;
        }
        count = min(found, G);
      }
      if (count <= 0) break;
      if (tid < count) s_tok[tid] = s_pairs[tid] / a.K;
      __syncthreads();
      const int nbatch = (t1 - t0 + kBatWaves - 1) / kBatWaves;

      const int nxu = count * (H / 8);                 // 16-byte units of x, token-major

      // ---- load cursor over this wave's tiles ----
      int lt = t0 + wave;                              // load cursor: tile, step
      int ls = 0;
      int left = 0;                                    // K-steps this wave still has to load
      for (int t = lt; t < t1; t += kBatWaves) left += S;
      auto row_off = [&](int tile) {
        const int row = tile * RT + cc;
        return (uint32_t)(row < I ? row : I - 1) * rbytes + (uint32_t)g4 * group_bytes<Q8>();
      };
      uint32_t loff = row_off(lt);
      // always two loads per call (kOffNone once the wave's tiles are all
      // issued), so that the compiler's wait counts stay exact
      auto issue = [&](StepW<Q8>& g, StepW<Q8>& u_) {
        const bool live = left > 0;
        const uint32_t o = live ? loff + (uint32_t)ls * step_row_bytes<Q8>() : kOffNone;
        load_step<Q8, VEC>(g, gsrc, o);
        load_step<Q8, VEC>(u_, usrc, o);
        // cursor step without branches, so the loads stay unconditional
        left -= live ? 1 : 0;
        const int nls = ls + (live ? 1 : 0);
        const bool wrap = nls == S;
        ls = wrap ? 0 : nls;
        lt += wrap ? kBatWaves : 0;
        loff = wrap ? row_off(lt) : loff;
      };
      // ---- largest |x| of each token (one LDS atomic per wave when its 64
      // units belong to one token) ----
      for (int u0 = 0; u0 < nxu; u0 += kBatThreads) {
        const int u = u0 + tid;
        const int ti = min(u, nxu - 1) / (H / 8);
        uint32_t mx = 0, mn = 255;
        if (u < nxu) {
          const int w8 = u - ti * (H / 8);
          if (xf) {
            const uint4* xp = (const uint4*)((const float*)a.x + (uint64_t)s_tok[ti] * H + 8 * w8);
            f32_range8(xp[0], xp[1], mx, mn);
          } else {
            const uint4 xq = *(const uint4*)(a.x + (uint64_t)s_tok[ti] * H + 8 * w8);
            range8(xq, mx, mn);
          }
        }
        if (__shfl(ti, 0) == __shfl(ti, 63)) {
          mx = wave_extreme<true>(mx);
          mn = wave_extreme<false>(mn);
          if (lane == 0 && mx) atomicMax(&s_xmax[ti], (int)mx);
          if (lane == 0 && mn < 255) atomicMin(&s_xmin[ti], (int)mn);
        } else {
          if (mx) atomicMax(&s_xmax[ti], (int)mx);
          if (mn < 255) atomicMin(&s_xmin[ti], (int)mn);
        }
      }
      __syncthreads();
      // digits per value for the whole group: four when every token allows it
      int L = 4;
      for (int ti = 0; ti < count; ++ti) L = max(L, digits_for(s_xmax[ti], s_xmin[ti]));
      L = xf ? 8 : __builtin_amdgcn_readfirstlane(L);   // f32: eight digits per value
      if (L > 4 && count > (16 * NT) / L) {
        count = (16 * NT) / L;                         // the rest go to the next group
        more = 1;
      }
      next_pair = s_pairs[count - 1] + 1;
      if (grouped && more) idv = (next_pair + tid < P) ? a.ids[next_pair + tid] : -1;
      const int C = L * count;
      const int ntiles = (C + 15) >> 4;
      const int sb = bat_step_bytes(ntiles);
      // Four-digit groups whose digits for the whole K fit both buffers keep
      // them resident for the group: no chunk barriers, no restaging per
      // batch, and the epilogue recombines digits across lanes (no LDS).
      const bool whole = L == 4 && S * sb <= 2 * kBatBuf;
      const int spc = whole ? S : bat_chunk_steps(ntiles, S);
      const int nch = (S + spc - 1) / spc;
      auto half = [&](int h) { return s_buf + (h & 1) * kBatBuf; };

      // digits of 8 consecutive K values (unit w8 of a chunk) of token ti
      auto stage_unit = [&](uint8_t* buf, int ti, int w8, const uint4 xq) {
        const int etop1 = max((s_xmax[ti] >> 7) & 0xFF, 1);
        const int tl = w8 >> 4, gg = (w8 >> 2) & 3, i = w8 & 3;
        if (L == 4) {
          uint32_t d[2][4];
          x8_digits4(xq, etop1, d);
#pragma unroll
          for (int par = 0; par < 2; ++par) {
            uint8_t* base = buf + tl * sb + par * ntiles * 1024 + gg * 256 + 4 * i;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int col = ti * 4 + s;
              *(uint32_t*)(base + (col >> 4) * 1024 + (col & 15) * 16) = d[par][s];
            }
          }
          return;
        }
        uint32_t lo[8], hi[8];
        x8_digits(xq, etop1, lo, hi);
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          uint32_t d[6];
          digit_words(lo, hi, par, d);
          uint8_t* base = buf + tl * sb + par * ntiles * 1024 + gg * 256 + 4 * i;
#pragma unroll
          for (int s = 0; s < 6; ++s) {
            const int col = ti * 6 + s;
            *(uint32_t*)(base + (col >> 4) * 1024 + (col & 15) * 16) = d[s];
          }
        }
      };
      // eight digits of eight f32 activations: columns 8*ti .. 8*ti+7
      auto stage_unitf = [&](uint8_t* buf, int ti, int w8, const uint4 xa, const uint4 xb) {
        const int etop1 = max((int)(((uint32_t)s_xmax[ti] >> 23) & 0xFFu), 1);
        const int tl = w8 >> 4, gg = (w8 >> 2) & 3, i = w8 & 3;
        uint32_t d[2][8];
        xf8_digits(xa, xb, etop1, d);
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          uint8_t* base = buf + tl * sb + par * ntiles * 1024 + gg * 256 + 4 * i;
#pragma unroll
          for (int sd = 0; sd < 8; ++sd) {
            const int col = ti * 8 + sd;
            *(uint32_t*)(base + (col >> 4) * 1024 + (col & 15) * 16) = d[par][sd];
          }
        }
      };
      auto stage = [&](int c, uint8_t* buf) {
        const int k0c = c * spc * 128;
        const int n8 = min(spc, S - c * spc) * 16;
        // unit u = w8 * count + ti, stepped by kBatThreads without dividing
        const int qd = kBatThreads / count, rd = kBatThreads - qd * count;
        int ti = tid % count, w8 = tid / count;
        for (int u = tid; u < count * n8; u += kBatThreads) {
          const int k0 = k0c + 8 * w8;
          if (xf) {
            uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
            if (k0 < H) {
              const uint4* xp = (const uint4*)((const float*)a.x + (uint64_t)s_tok[ti] * H + k0);
              xa = xp[0];
              xb = xp[1];
            }
            stage_unitf(buf, ti, w8, xa, xb);
          } else {
            uint4 xq = make_uint4(0, 0, 0, 0);
            if (k0 < H) xq = *(const uint4*)(a.x + (uint64_t)s_tok[ti] * H + k0);
            stage_unit(buf, ti, w8, xq);
          }
          ti += rd;
          w8 += qd;
          if (ti >= count) {
            ti -= count;
            ++w8;
          }
        }
        // x was loaded after the weights in flight and is used up here, so
        // none of them is pending any more: said explicitly, the compiler's
        // wait counts at the head of the step loop stay exact (otherwise a
        // register the x loads once held makes it wait for every load there)
        __builtin_amdgcn_s_waitcnt(kWaitVmem0);
      };

      // columns past C in the last tile hold stale bytes; their results are never read

      stage(0, s_buf);
      __syncthreads();
      // the weights of this wave's first tile go out now
      StepW<Q8> rg0, ru0, rg1, ru1;
      issue(rg0, ru0);
      issue(rg1, ru1);
      int gch = 0;                                     // chunks done in this group (buffer parity)
      for (int bb = 0; bb < nbatch; ++bb) {
        const int tile = t0 + bb * kBatWaves + wave;
        const bool active = tile < t1;
        v4i accg[NT], accu[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          accg[n] = v4i{0, 0, 0, 0};
          accu[n] = v4i{0, 0, 0, 0};
        }
        for (int c = 0; c < nch; ++c, ++gch) {
          const uint8_t* buf = nch == 1 ? s_buf : half(gch);
          const bool more = (c + 1 < nch) || (bb + 1 < nbatch);
          if (nch > 1 && more) stage((c + 1) % nch, half(gch + 1));
          if (active) {
            const int sa = c * spc, se = min(S, sa + spc);
            auto compute = [&](const StepW<Q8>& g, const StepW<Q8>& u_, int s) {
              v4i ge, go, ue, uo;
              split_step(g, ge, go);
              split_step(u_, ue, uo);
              const uint8_t* bp = buf + (s - sa) * sb + lane * 16;
              v4i be[NT], bo[NT];
#pragma unroll
              for (int n = 0; n < NT; ++n) {
                be[n] = *(const v4i*)(bp + n * 1024);
                bo[n] = *(const v4i*)(bp + (ntiles + n) * 1024);
              }
#pragma unroll
              for (int n = 0; n < NT; ++n) {
                if (n < ntiles) {
                  accg[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ge, be[n], accg[n], 0, 0, 0);
                  accu[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ue, be[n], accu[n], 0, 0, 0);
                  accg[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(go, bo[n], accg[n], 0, 0, 0);
                  accu[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(uo, bo[n], accu[n], 0, 0, 0);
                }
              }
            };
            for (int s = sa; s < se; s += 2) {
              compute(rg0, ru0, s);
              issue(rg0, ru0);
              compute(rg1, ru1, s + 1);
              issue(rg1, ru1);
            }
          }
          if (!whole) __syncthreads();
        }

        if (whole) {
          // ---- epilogue across lanes: with four digits per token, the digits of
          // a (row, token) sum sit in the four lanes of a quad (columns 4t..4t+3);
          // a transposing quad reduction leaves lane j of the quad with row j ----
          if (active) {
            const int j = cc & 3;
            const int row = tile * RT + 4 * g4 + j;
            auto quad_row_sum = [&](const v4i acc) { return quad_digit_sum(acc, j); };
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              if (n < ntiles) {
                const int ti = 4 * n + (cc >> 2);
                const int64_t vg = quad_row_sum(accg[n]);
                const int64_t vu = quad_row_sum(accu[n]);
                if (ti < count && row < I) {
                  const int e2 = sum_exponent(s_xmax[ti]) + 16 + weight_exp_shift<Q8>();
                  const float gate = round_scaled53(vg, e2, gscale[row]);
                  const uint64_t o = (uint64_t)s_pairs[ti] * I + row;
                  if constexpr (DOWN) {
                    a.out[o] = bf16_rne(gate);
                    if (a.gate_probe) a.gate_probe[o] = gate;
                    if (row + 16 < I) {
                      const float r16 = round_scaled53(vu, e2, gscale[row + 16]);
                      a.out[o + 16] = bf16_rne(r16);
                      if (a.gate_probe) a.gate_probe[o + 16] = r16;
                    }
                  } else {
                    const float up = round_scaled53(vu, e2, uscale[row]);
                    a.out[o] = swiglu_tail_tab(gate, up, s_sig);
                    if (a.gate_probe) a.gate_probe[o] = gate;
                    if (a.up_probe) a.up_probe[o] = up;
                  }
                }
              }
            }
          }
          continue;
        }

        // ---- epilogue: digit matrix through the free LDS buffer ----
        // After the batch's last chunk barrier one buffer is idle: the single
        // buffer's twin when one chunk covers K, else the last chunk's buffer
        // (the other one already holds the next batch's first chunk).
        {
          int32_t* ep = (int32_t*)half(nch == 1 ? 1 : gch - 1) + wave * (16 * kEpStride);
          if (active) {
            // gate first, then up, through the same 16 x C matrix
            constexpr int kItemRounds = (16 * G + 63) / 64;   // (row, token) items per lane
            float gv[kItemRounds];
#pragma unroll
            for (int part = 0; part < 2; ++part) {
#pragma unroll
              for (int n = 0; n < NT; ++n) {
                const int col = 16 * n + cc;
                if (n < ntiles && col < C) {
#pragma unroll
                  for (int i = 0; i < 4; ++i) ep[(4 * g4 + i) * kEpStride + col] = part ? accu[n][i] : accg[n][i];
                }
              }
              wave_sync();
#pragma unroll
              for (int j = 0; j < kItemRounds; ++j) {
                const int item = lane + 64 * j;
                const int rr = item & 15, ti = item >> 4;
                const int row = tile * RT + rr + (DOWN ? 16 * part : 0);
                if (ti < count && row < I) {
                  const int32_t* d = ep + rr * kEpStride + ti * L;
                  const int xm = s_xmax[ti];
                  const float sc = (part && !DOWN) ? uscale[row] : gscale[row];
                  float r;
                  if (xf) {
                    // eight digits: V = hi * 2^32 + lo
                    const int64_t lo = (int64_t)d[0] + ((int64_t)d[1] << 8) + ((int64_t)d[2] << 16) +
                                       ((int64_t)d[3] << 24);
                    const int64_t hi = (int64_t)d[4] + ((int64_t)d[5] << 8) + ((int64_t)d[6] << 16) +
                                       ((int64_t)d[7] << 24);
                    r = round_scaled_wide(hi, lo, sum_exponent_f32((uint32_t)xm) + weight_exp_shift<Q8>(), sc);
                    if ((uint32_t)xm >= 0x7F800000u) r = __builtin_nanf("");
                  } else {
                    const int64_t lo = (int64_t)d[0] + ((int64_t)d[1] << 8) + ((int64_t)d[2] << 16);
                    const int64_t hi = L == 6 ? (int64_t)d[3] + ((int64_t)d[4] << 8) + ((int64_t)d[5] << 16)
                                              : (int64_t)d[3];
                    r = round_scaled(hi, lo, sum_exponent(xm) + 8 * (6 - L) + weight_exp_shift<Q8>(), sc);
                    if (xm >= 0x7F80) r = __builtin_nanf("");
                  }
                  if constexpr (DOWN) {
                    const uint64_t o = (uint64_t)s_pairs[ti] * I + row;
                    if (xf)
                      ((float*)a.out)[o] = r;
                    else
                      a.out[o] = bf16_rne(r);
                    if (a.gate_probe) a.gate_probe[o] = r;
                  } else if (!part) {
                    gv[j] = r;
                  } else {
                    const uint64_t o = (uint64_t)s_pairs[ti] * I + row;
                    if (xf)
                      ((float*)a.out)[o] = swiglu_tail_f32(gv[j], r);
                    else
                      a.out[o] = swiglu_tail_tab(gv[j], r, s_sig);
                    if (a.gate_probe) a.gate_probe[o] = gv[j];
                    if (a.up_probe) a.up_probe[o] = r;
                  }
                }
              }
              wave_sync();
            }
          }
          __syncthreads();  // the epilogue buffer is staged into by the next batch
        }
      }
      if (!more) break;
    }
  }
}

// ---- host side ----

namespace {

template <int NT, bool VEC, bool DOWN, bool Q8, bool XF>
int batch_blocks(int device) {
  // per-device cache; concurrent first calls compute the same value
  static std::atomic<int> cached[64];
  if (device < 0 || device >= 64) device = 0;
  if (!cached[device].load(std::memory_order_relaxed)) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&batch_kernel<NT, VEC, DOWN, Q8, XF>), kBatThreads, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    cached[device].store(cus * per_cu, std::memory_order_relaxed);
  }
  return cached[device].load(std::memory_order_relaxed);
}

template <int NT, bool VEC, bool DOWN, bool Q8, bool XF>
hipError_t launch_batch_t(GateUpParams& p, hipStream_t stream) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  const int rt = DOWN ? 32 : 16;
  const int tiles = p.num_slots * ((p.I + rt - 1) / rt);
  int nb = batch_blocks<NT, VEC, DOWN, Q8, XF>(device);
  if (nb > tiles) nb = tiles;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&batch_kernel<NT, VEC, DOWN, Q8, XF>), dim3((unsigned)nb),
                         dim3(kBatThreads), args, 0, stream);
}

template <bool DOWN, bool Q8, bool XF>
hipError_t launch_batch_m(GateUpParams& p, int nt, hipStream_t stream) {
  const bool vec = row_bytes<Q8>(p.H) % 16 == 0;
  if (nt == 1)
    return vec ? launch_batch_t<1, true, DOWN, Q8, XF>(p, stream) : launch_batch_t<1, false, DOWN, Q8, XF>(p, stream);
  if (nt == 2)
    return vec ? launch_batch_t<2, true, DOWN, Q8, XF>(p, stream) : launch_batch_t<2, false, DOWN, Q8, XF>(p, stream);
  return vec ? launch_batch_t<3, true, DOWN, Q8, XF>(p, stream) : launch_batch_t<3, false, DOWN, Q8, XF>(p, stream);
}

template <bool XF>
hipError_t launch_batch_x(GateUpParams& p, int nt, hipStream_t stream) {
  if (p.q8) return p.down ? launch_batch_m<true, true, XF>(p, nt, stream) : launch_batch_m<false, true, XF>(p, nt, stream);
  return p.down ? launch_batch_m<true, false, XF>(p, nt, stream) : launch_batch_m<false, false, XF>(p, nt, stream);
}

}  // namespace

hipError_t launch_batch(GateUpParams p, int tokens_per_slot, hipStream_t stream) {
  p.steps = (p.H + 127) / 128;
  p.steps += p.steps & 1;
  const int nt = tokens_per_slot <= 2 ? 1 : (tokens_per_slot <= 5 ? 2 : 3);
  p.G = (16 * nt) / 4;
  return p.xf32 ? launch_batch_x<true>(p, nt, stream) : launch_batch_x<false>(p, nt, stream);
}

}  // namespace q4
