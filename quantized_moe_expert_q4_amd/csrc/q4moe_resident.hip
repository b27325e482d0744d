// Q4 gate/up + SwiGLU for narrow token sets (decode): digits resident in LDS.
//
// Arithmetic: GATE_UP_SOURCE of the @mlx-bun/inference 1.0.0 diff, page 52
// (kernels/glm52/streamed-experts.ts), made exact as in q4moe_device.h.
//
// With at most two tokens in the call, the digit-split activations of every
// token (C = 6*M columns) for the whole K fit one LDS buffer.  A work-group
// splits them once, from a single read of x, and keeps them for the whole
// launch: every slot's group of routed pairs reads the columns of its own
// tokens, so nothing is staged again when the slot changes.
//  * One persistent launch: work-group b takes the whole tiles
//    [bT/NB, (b+1)T/NB) of the T = slots x tiles-per-slot tiles, so the
//    weight bytes per work-group differ by at most one tile.
//  * Inside a work-group the unit range of a slot segment is cut into eight
//    equal wave ranges (multiples of D steps).  Each wave streams its own
//    (16-row tile, K-step) units, keeping D K-steps of weights in flight in a
//    register ring; the first loads of a segment go out before the routing
//    scan and (first segment) before x is read.
//  * A tile cut by a wave boundary has several contributors; each adds its
//    exact int64 partial sums into an LDS slot with LDS atomics and bumps the
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
constexpr int kResBBytes = 56 * 1024;     // digits of all tokens over the whole K
constexpr int kResMaxCols = 12;           // two tokens of six digits
constexpr int kResGroup = 2;              // routed pairs finished per pass over a slot
constexpr int kResItems = 16 * kResGroup; // (row, pair) results of one tile
constexpr int kResXRegs = 3;              // 16-byte chunks of x held per thread while splitting

__host__ __device__ constexpr int block_stride(int C) { return C * 16 + 16; }  // one padded (step, parity, g) block

}  // namespace

template <int D, bool VEC>
__global__ __launch_bounds__(kResThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void resident_kernel(const GateUpParams a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_b[kResBBytes];
  __shared__ int32_t s_acc[kResWaves][2][16 * kResMaxCols];   // per-wave digit matrix of a tile
  __shared__ unsigned long long s_fix[kResWaves][kResItems * 4];
  __shared__ int s_fixcnt[kResWaves];
  __shared__ int s_pairs[kResGroup];
  __shared__ int s_wcnt[kResWaves];
  __shared__ int s_xmax[2];
  __shared__ int s_invalid;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, cc = lane & 15;
  const int H = a.H, I = a.I;
  const int P = a.M * a.K;
  const bool grouped = a.ids != nullptr;
  const int S = a.steps;                     // K-steps per tile, a multiple of D
  const int C = 6 * a.M;                     // digit columns: every token of the call
  const int bs = block_stride(C);
  const int tps = (I + 15) / 16;             // tiles per slot
  const int T = a.num_slots * tps;
  const int NB = gridDim.x;
  // Tile range of this work-group.  With two work-groups per CU (pair_share
  // > 0) the grid is split into CU pairs (b, b + NB/2): the one dispatched
  // first wins the CU's memory-issue arbitration more often, so it takes
  // pair_share/1024 of the pair's tiles and both finish together.
  int v0, v1;
  if (a.pair_share > 0) {
    const int P2 = NB / 2;
    const int pair = (int)blockIdx.x % P2;
    const int pa = (int)((int64_t)pair * T / P2), pb = (int)((int64_t)(pair + 1) * T / P2);
    const int mid = pa + (int)(((int64_t)(pb - pa) * a.pair_share + 512) / 1024);
    v0 = (int)blockIdx.x < P2 ? pa : mid;
    v1 = (int)blockIdx.x < P2 ? mid : pb;
  } else {
    v0 = (int)((int64_t)blockIdx.x * T / NB);
    v1 = (int)((int64_t)(blockIdx.x + 1) * T / NB);
  }
  const uint32_t wbytes = (uint32_t)((uint64_t)I * (uint32_t)(H / 2));
  const uint64_t below = (1ull << lane) - 1ull;

  if (tid < 2) s_xmax[tid] = 0;
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

  auto row_off = [&](int tile) {
    const int row = tile * 16 + cc;
    return (uint32_t)(row < I ? row : I - 1) * (uint32_t)(H / 2) + (uint32_t)(g4 * 16);
  };
  const int col = min(cc, C - 1);
  const uint8_t* bl = s_b + g4 * bs + col * 16;                // + (step*2 + par)*4*bs

  bool staged = false;
  int v = v0;
  while (v < v1) {
    const int e = v / tps;
    const int t0 = v - e * tps;                               // first tile of the segment in slot e
    const int t1 = min(v1, (e + 1) * tps) - e * tps;          // end tile
    v = e * tps + t1;
    const uint8_t* slot = a.slots + (uint64_t)e * a.slot_stride;
    const __amdgpu_buffer_rsrc_t gsrc = make_rsrc(slot + a.gate_w_off, wbytes);
    const __amdgpu_buffer_rsrc_t usrc = make_rsrc(slot + a.up_w_off, wbytes);
    const float* gscale = (const float*)(slot + a.gate_s_off);
    const float* uscale = (const float*)(slot + a.up_s_off);

    // ---- this wave's unit range of the segment ----
    const int nunits = (t1 - t0) * S;
    auto bound = [&](int q) { return (int)(((int64_t)q * nunits / kResWaves) / D * D); };
    const int ua = bound(wave), ub = (wave + 1 == kResWaves) ? nunits : bound(wave + 1);

    v4u rg[D], ru[D];
    int lt, ls;                                              // load cursor (tile, step)
    uint32_t loff;
    auto issue = [&](v4u& g, v4u& u_, bool live) {
      const uint32_t o = live ? loff + (uint32_t)ls * 64u : kOffNone;
      g = load16<VEC>(gsrc, o);
      u_ = load16<VEC>(usrc, o);
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
      for (int d = 0; d < D; ++d) issue(rg[d], ru[d], ua + d < ub);
    };

    // first routing-scan window, loaded before the ring so that its wait
    // does not include the weight loads
    int next_pair = 0;
    int idv = -1;
    if (grouped && tid < P) idv = a.ids[tid];

    // ---- first segment: x of every token, loaded before the ring ----
    uint4 xv[kResXRegs];
    const int nxc = a.M * (H / 8);                            // 16-byte chunks of x
    if (!staged) {
#pragma unroll
      for (int j = 0; j < kResXRegs; ++j) {
        const int q = tid + j * kResThreads;
        xv[j] = q < nxc ? ((const uint4*)a.x)[q] : make_uint4(0, 0, 0, 0);
      }
    }
    start_ring();

    if (!staged) {
      // largest |x| of each token
      uint32_t m0 = 0, m1 = 0;
#pragma unroll
      for (int j = 0; j < kResXRegs; ++j) {
        const int q = tid + j * kResThreads;
        const uint32_t mx = max_mag8(xv[j]);
        if (q < nxc) {
          if (q < H / 8) m0 = max(m0, mx);
          else m1 = max(m1, mx);
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        m0 = max(m0, (uint32_t)__shfl_xor((int)m0, off));
        m1 = max(m1, (uint32_t)__shfl_xor((int)m1, off));
      }
      if (lane == 0) {
        if (m0) atomicMax(&s_xmax[0], (int)m0);
        if (m1) atomicMax(&s_xmax[1], (int)m1);
      }
      __syncthreads();
      // the digits of every token, and zero digits for the padding steps
#pragma unroll
      for (int j = 0; j < kResXRegs; ++j) {
        const int q = tid + j * kResThreads;
        if (q < nxc) {
          const int m = q / (H / 8), w8 = q - m * (H / 8);
          uint32_t lo[8], hi[8];
          x8_digits(xv[j], max((s_xmax[m] >> 7) & 0xFF, 1), lo, hi);
          const int tl = w8 >> 4, gg = (w8 >> 2) & 3, i = w8 & 3;
#pragma unroll
          for (int par = 0; par < 2; ++par) {
            uint32_t d[6];
            digit_words(lo, hi, par, d);
            uint8_t* base = s_b + ((tl * 2 + par) * 4 + gg) * bs + m * 96 + 4 * i;
#pragma unroll
            for (int s = 0; s < 6; ++s) *(uint32_t*)(base + s * 16) = d[s];
          }
        }
      }
      const int padw = S * 16 - H / 8;
      for (int u = tid; u < a.M * padw; u += kResThreads) {
        const int m = u % a.M, w8 = H / 8 + u / a.M;
        const int tl = w8 >> 4, gg = (w8 >> 2) & 3, i = w8 & 3;
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          uint8_t* base = s_b + ((tl * 2 + par) * 4 + gg) * bs + m * 96 + 4 * i;
#pragma unroll
          for (int s = 0; s < 6; ++s) *(uint32_t*)(base + s * 16) = 0u;
        }
      }
      staged = true;
    }

    bool first_group = true;
    for (;;) {
      __syncthreads();  // previous group done with s_fix and s_pairs; digits visible
      if (tid < kResWaves) s_fixcnt[tid] = 0;
      for (int i = tid; i < kResWaves * kResItems * 4; i += kResThreads) (&s_fix[0][0])[i] = 0ull;

      // ---- next group of up to kResGroup pairs routed to slot e ----
      int count, more;
      if (!grouped) {
        count = min(kResGroup, P - next_pair);
        more = next_pair + count < P;
        if (tid < count) s_pairs[tid] = next_pair + tid;
        __syncthreads();  // s_pairs and the cleared fix-up slots visible
      } else {
        // block-wide scan of ids[next_pair..P) in windows of kResThreads;
        // stops once a further match proves there is another group
        int found = 0;
        int base = next_pair;
        more = 0;
        for (;;) {
          const bool m = idv == e;
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
          if (m && before < kResGroup) s_pairs[before] = base + tid;
          found = total;
          base += kResThreads;
          if (found > kResGroup) more = 1;
          __syncthreads();  // s_wcnt reused; s_pairs visible
          if (more || base >= P) break;
          idv = (base + tid < P) ? a.ids[base + tid] : -1;
        }
        count = min(found, kResGroup);
      }
      if (count <= 0) break;
      next_pair = s_pairs[count - 1] + 1;
      if (grouped && more) idv = (next_pair + tid < P) ? a.ids[next_pair + tid] : -1;
      if (!first_group) start_ring();
      first_group = false;

      int u = ua;
      while (u < ub) {
        // one portion: the rest of the current tile inside [u, ub)
        const int tile = t0 + u / S;
        const int sa = u % S;
        const int pe = min(ub, (u / S + 1) * S);             // portion end (unit)
        v4i accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
        int s = sa;
        for (; u < pe; u += D) {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            v4i ge, go, ue, uo;
            split_weights(rg[d], ge, go);
            split_weights(ru[d], ue, uo);
            const uint8_t* bp = bl + (s + d) * 8 * bs;
            const v4i be = *(const v4i*)bp;
            const v4i bo = *(const v4i*)(bp + 4 * bs);
            accg = __builtin_amdgcn_mfma_i32_16x16x64_i8(ge, be, accg, 0, 0, 0);
            accu = __builtin_amdgcn_mfma_i32_16x16x64_i8(ue, be, accu, 0, 0, 0);
            accg = __builtin_amdgcn_mfma_i32_16x16x64_i8(go, bo, accg, 0, 0, 0);
            accu = __builtin_amdgcn_mfma_i32_16x16x64_i8(uo, bo, accu, 0, 0, 0);
            issue(rg[d], ru[d], u + d + D < ub);
          }
          s += D;
        }
        const int se = s;                                    // portion covers steps [sa, se)

        // ---- digit matrix -> (row, pair) exact int64 sums ----
        int32_t* eg = s_acc[wave][0];
        int32_t* eu = s_acc[wave][1];
        if (cc < C) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            eg[(4 * g4 + i) * C + cc] = accg[i];
            eu[(4 * g4 + i) * C + cc] = accu[i];
          }
        }
        wave_sync();
        const int rr = lane & 15, ti = lane >> 4;            // item = (row rr, pair ti), ti < kResGroup
        int64_t sm[4] = {0, 0, 0, 0};
        int tok = 0;
        if (ti < count) {
          tok = s_pairs[ti] / a.K;
          const int32_t* gd = eg + rr * C + tok * 6;
          const int32_t* ud = eu + rr * C + tok * 6;
          sm[0] = (int64_t)gd[0] + ((int64_t)gd[1] << 8) + ((int64_t)gd[2] << 16);
          sm[1] = (int64_t)gd[3] + ((int64_t)gd[4] << 8) + ((int64_t)gd[5] << 16);
          sm[2] = (int64_t)ud[0] + ((int64_t)ud[1] << 8) + ((int64_t)ud[2] << 16);
          sm[3] = (int64_t)ud[3] + ((int64_t)ud[4] << 8) + ((int64_t)ud[5] << 16);
        }
        wave_sync();

        bool finish = (sa == 0 && se == S);
        if (!finish) {
          // contributors of this tile: waves whose ranges meet its units
          const int tu0 = (tile - t0) * S, tu1 = tu0 + S;
          int first = -1, ncontrib = 0;
          for (int q = 0; q < kResWaves; ++q) {
            const int qa = bound(q), qb = (q + 1 == kResWaves) ? nunits : bound(q + 1);
            if (qa < qb && qa < tu1 && qb > tu0) {
              if (first < 0) first = q;
              ++ncontrib;
            }
          }
          unsigned long long* slotp = s_fix[first];
          if (lane < kResItems && ti < count) {
#pragma unroll
            for (int j = 0; j < 4; ++j) atomicAdd(&slotp[lane * 4 + j], (unsigned long long)sm[j]);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          int prev = 0;
          if (lane == 0) prev = atomicAdd(&s_fixcnt[first], 1);
          prev = __shfl(prev, 0);
          if (prev == ncontrib - 1) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            if (lane < kResItems && ti < count) {
#pragma unroll
              for (int j = 0; j < 4; ++j) sm[j] = (int64_t)atomicAdd(&slotp[lane * 4 + j], 0ull);
            }
            finish = true;
          }
        }
        if (finish && ti < count) {
          const int row = tile * 16 + rr;
          if (row < I) {
            const int p = s_pairs[ti];
            const int xm = s_xmax[tok];
            const int e2 = sum_exponent(xm);
            float gate = round_scaled(sm[1], sm[0], e2, gscale[row]);
            float up = round_scaled(sm[3], sm[2], e2, uscale[row]);
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
      if (!more) break;
    }
  }
}

// ---- host side ----

namespace {

// Work-groups that fit the device at once, and how many share a CU.
template <int D, bool VEC>
int resident_blocks(int device, int* per_cu_out) {
  static int cached[64] = {0}, cached_per_cu[64] = {0};
  if (device < 0 || device >= 64) device = 0;
  if (!cached[device]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&resident_kernel<D, VEC>), kResThreads, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    cached_per_cu[device] = per_cu;
    cached[device] = cus * per_cu;
  }
  *per_cu_out = cached_per_cu[device];
  return cached[device];
}

// Share of a CU pair's tiles for the first-dispatched work-group, in 1/1024
// (measured on MI355X: with equal shares the first-dispatched work-groups
// finish at about 0.86 of the time of the second ones).
constexpr int kPairShare = 650;

constexpr int kResD = 2;

}  // namespace

bool resident_fits(int M, int H) {
  const int steps = ((H + 127) / 128 + kResD - 1) / kResD * kResD;
  return M >= 1 && M <= 2 && (size_t)block_stride(6 * M) * 8 * steps <= (size_t)kResBBytes &&
         (int64_t)M * (H / 8) <= (int64_t)kResXRegs * kResThreads;
}

hipError_t launch_resident(GateUpParams p, hipStream_t stream) {
  p.steps = ((p.H + 127) / 128 + kResD - 1) / kResD * kResD;
  p.G = kResGroup;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  const bool vec = (p.H % 32) == 0;
  const int tiles = p.num_slots * ((p.I + 15) / 16);
  int per_cu = 1;
  int nb = vec ? resident_blocks<kResD, true>(device, &per_cu) : resident_blocks<kResD, false>(device, &per_cu);
  // uneven CU-pair shares only for a full grid of two work-groups per CU,
  // each with several tiles
  p.pair_share = (per_cu == 2 && tiles >= 8 * nb) ? kPairShare : 0;
  if (nb > tiles) nb = tiles;
  void* args[] = {&p};
  const void* fn = vec ? reinterpret_cast<const void*>(&resident_kernel<kResD, true>)
                       : reinterpret_cast<const void*>(&resident_kernel<kResD, false>);
  return hipLaunchKernel(fn, dim3((unsigned)nb), dim3(kResThreads), args, 0, stream);
}

hipError_t launch_gate_up(const GateUpParams& p, int tokens_per_slot, hipStream_t stream) {
  return resident_fits(tokens_per_slot, p.H) ? launch_resident(p, stream) : launch_batch(p, tokens_per_slot, stream);
}

}  // namespace q4
