// Q4 gate/up + SwiGLU for narrow token groups (decode): digits resident in LDS.
//
// Arithmetic: GATE_UP_SOURCE of the @mlx-bun/inference 1.0.0 diff, page 52
// (kernels/glm52/streamed-experts.ts), made exact as in q4moe_device.h.
//
// When the digit-split activations of a token group (C = 6*count columns)
// for the whole K fit one LDS buffer, the waves of a work-group need not move
// through K together: each wave streams its own contiguous range of
// (16-row tile, K-step) units, reading its B fragments from the resident
// digits, and keeps D K-steps of weights in flight in a register ring.
//  * One persistent launch: work-group b takes the whole tiles
//    [bT/NB, (b+1)T/NB) of the T = slots x tiles-per-slot tiles, so the
//    weight bytes per work-group differ by at most one tile.
//  * Inside a work-group the unit range of a slot segment is cut into eight
//    equal wave ranges (multiples of D steps).  A tile cut by a wave boundary
//    has several contributors; each adds its exact int64 partial sums into an
//    LDS slot with LDS atomics and bumps the slot's counter; the last one to
//    arrive finishes the tile.  No wave waits on another.
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
constexpr int kResBBytes = 56 * 1024;     // digits of one token group over the whole K
constexpr int kResMaxCols = 12;           // two tokens of six digits
constexpr int kResItems = 16 * 2;         // (row, token) results of one tile (<= 2 tokens)

__host__ __device__ constexpr int block_stride(int C) { return C * 16 + 16; }  // one padded (step, parity, g) block

}  // namespace

template <int D, bool VEC>
__global__ __launch_bounds__(kResThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void resident_kernel(const GateUpParams a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_b[kResBBytes];
  __shared__ int32_t s_acc[kResWaves][2][16 * kResMaxCols];   // per-wave digit matrix of a tile
  __shared__ unsigned long long s_fix[kResWaves][kResItems * 4];
  __shared__ int s_fixcnt[kResWaves];
  __shared__ int s_pairs[2];
  __shared__ int s_xmax[2];
  __shared__ int s_count;
  __shared__ int s_invalid;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4, cc = lane & 15;
  const int H = a.H, I = a.I;
  const int P = a.M * a.K;
  const bool grouped = a.ids != nullptr;
  const int S = a.steps;                     // K-steps per tile, a multiple of D
  const int tps = (I + 15) / 16;             // tiles per slot
  const int T = a.num_slots * tps;
  const int NB = gridDim.x;
  const int v0 = (int)((int64_t)blockIdx.x * T / NB), v1 = (int)((int64_t)(blockIdx.x + 1) * T / NB);
  const uint32_t wbytes = (uint32_t)((uint64_t)I * (uint32_t)(H / 2));

  // ---- invalid routing ids (grouped): zero-filled by work-group 0 ----
  if (grouped && blockIdx.x == 0) {
    if (tid == 0) s_invalid = 0;
    __syncthreads();
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

    int next_pair = 0;
    for (;;) {
      __syncthreads();  // previous group done with s_b, s_fix, s_pairs
      // ---- next group of up to G pairs routed to slot e ----
      if (!grouped) {
        if (tid < a.G) s_pairs[tid] = next_pair + tid;
        if (tid == 0) s_count = min(a.G, P - next_pair);
      } else if (wave == 0) {
        int found = 0;
        int p = next_pair;
        while (found < a.G && p < P) {
          const int q = p + lane;
          const bool m = q < P && a.ids[q] == e;
          const uint64_t bal = __ballot(m);
          const int before = __popcll(bal & ((1ull << lane) - 1ull));
          if (m && found + before < a.G) s_pairs[found + before] = q;
          found += __popcll(bal);
          p += 64;
        }
        if (lane == 0) s_count = min(found, a.G);
      }
      if (tid < 2) s_xmax[tid] = 0;
      if (tid < kResWaves) s_fixcnt[tid] = 0;
      for (int i = tid; i < kResWaves * kResItems * 4; i += kResThreads) (&s_fix[0][0])[i] = 0ull;
      __syncthreads();
      const int count = s_count;
      if (count <= 0) break;
      next_pair = grouped ? s_pairs[count - 1] + 1 : next_pair + count;
      const int C = 6 * count;
      const int bs = block_stride(C);

      // ---- largest |x| of each token, then the resident digits ----
      for (int ti = 0; ti < count; ++ti) {
        const uint4* xr = (const uint4*)(a.x + (uint64_t)(s_pairs[ti] / a.K) * H);
        uint32_t mx = 0;
        for (int w8 = tid; w8 < H / 8; w8 += kResThreads) mx = max(mx, max_mag8(xr[w8]));
        if (mx) atomicMax(&s_xmax[ti], (int)mx);
      }
      __syncthreads();
      for (int u = tid; u < count * S * 16; u += kResThreads) {
        const int ti = u % count;
        const int w8 = u / count;
        const int k0 = 8 * w8;
        uint4 xv = make_uint4(0, 0, 0, 0);
        if (k0 < H) xv = *(const uint4*)(a.x + (uint64_t)(s_pairs[ti] / a.K) * H + k0);
        uint32_t lo[8], hi[8];
        x8_digits(xv, max((s_xmax[ti] >> 7) & 0xFF, 1), lo, hi);
        const int tl = w8 >> 4, gg = (w8 >> 2) & 3, i = w8 & 3;
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          uint32_t d[6];
          digit_words(lo, hi, par, d);
          uint8_t* base = s_b + ((tl * 2 + par) * 4 + gg) * bs + ti * 96 + 4 * i;
#pragma unroll
          for (int s = 0; s < 6; ++s) *(uint32_t*)(base + s * 16) = d[s];
        }
      }
      __syncthreads();

      // ---- this wave's unit range of the segment ----
      const int nunits = (t1 - t0) * S;
      auto bound = [&](int q) { return (int)(((int64_t)q * nunits / kResWaves) / D * D); };
      const int ua = bound(wave), ub = (wave + 1 == kResWaves) ? nunits : bound(wave + 1);
      const int col = min(cc, C - 1);
      const uint8_t* bl = s_b + g4 * bs + col * 16;           // + (step*2 + par)*4*bs

      v4u rg[D], ru[D];
      int lt = t0 + ua / S, ls = ua % S;                      // load cursor (tile, step)
      auto row_off = [&](int tile) {
        const int row = tile * 16 + cc;
        return (uint32_t)(row < I ? row : I - 1) * (uint32_t)(H / 2) + (uint32_t)(g4 * 16);
      };
      uint32_t loff = row_off(lt);
      auto issue = [&](v4u& g, v4u& u_) {
        const uint32_t o = loff + (uint32_t)ls * 64u;
        g = load16<VEC>(gsrc, o);
        u_ = load16<VEC>(usrc, o);
        if (++ls == S) {
          ls = 0;
          loff = row_off(++lt);
        }
      };
#pragma unroll
      for (int d = 0; d < D; ++d)
        if (ua + d < ub) issue(rg[d], ru[d]);

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
            if (u + d + D < ub) issue(rg[d], ru[d]);
          }
          s += D;
        }
        const int se = s;                                    // portion covers steps [sa, se)

        // ---- digit matrix -> (row, token) exact int64 sums ----
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
        const int rr = lane & 15, ti = lane >> 4;            // item = (row rr, token ti), ti < 2
        int64_t sm[4] = {0, 0, 0, 0};
        if (ti < count) {
          const int32_t* gd = eg + rr * C + ti * 6;
          const int32_t* ud = eu + rr * C + ti * 6;
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
            const int xm = s_xmax[ti];
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
      if (count < a.G) break;
      if (!grouped && next_pair >= P) break;
    }
  }
}

// ---- host side ----

namespace {

template <int D, bool VEC>
int resident_blocks(int device) {
  static int cached[64] = {0};
  if (device < 0 || device >= 64) device = 0;
  if (!cached[device]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&resident_kernel<D, VEC>), kResThreads, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    cached[device] = cus * per_cu;
  }
  return cached[device];
}

constexpr int kResD = 2;

}  // namespace

bool resident_fits(int M_per_slot, int H) {
  const int steps = ((H + 127) / 128 + kResD - 1) / kResD * kResD;
  return M_per_slot >= 1 && M_per_slot <= 2 &&
         (size_t)block_stride(6 * M_per_slot) * 8 * steps <= (size_t)kResBBytes;
}

hipError_t launch_resident(GateUpParams p, hipStream_t stream) {
  p.steps = ((p.H + 127) / 128 + kResD - 1) / kResD * kResD;
  const int tokens = 2;
  p.G = (size_t)block_stride(6 * tokens) * 8 * p.steps <= (size_t)kResBBytes ? 2 : 1;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  const bool vec = (p.H % 32) == 0;
  const int tiles = p.num_slots * ((p.I + 15) / 16);
  int nb = vec ? resident_blocks<kResD, true>(device) : resident_blocks<kResD, false>(device);
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
