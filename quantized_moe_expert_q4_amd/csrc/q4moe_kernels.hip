// Q4 expert gate/up + SwiGLU on MI355X (gfx950).
//
// Arithmetic follows the GATE_UP_SOURCE kernel of the @mlx-bun/inference
// 1.0.0 diff, page 52, kernels/glm52/streamed-experts.ts: weight nibble p of
// packed word w is input position 8w+p with weight q-8; gate and up are the
// row sums times the row's F32 scale; the tail rounds gate and up to bf16,
// takes sigmoid in F32, and rounds silu and the product to bf16.
//
// MI355X design (not a translation of the Metal kernels):
//  * The row sums are computed exactly.  Each bf16 activation of a token is
//    put on the token's fixed-point grid X = x * 2^(38 - e_top) (e_top: the
//    exponent of the token's largest |x|) and X is split into six balanced
//    base-256 digits.  Weights enter the int8 matrix core as 16*(q-8), which
//    is the high nibble of (word ^ 0x88888888) -- two bit operations per word
//    and no table.  v_mfma_i32_16x16x64_i8 accumulates in exact int32
//    (|16w * d| <= 2^14, H <= 2^16), so the sum is exact for any blocking or
//    batch width; the digits are recombined in double-double and the product
//    with the F32 scale is rounded once to F32.
//  * One work-group (256 threads, four wave64s) owns 16*RT rows of gate and up
//    of one slot; the four waves split either rows (RT) or K (KP = 4/RT).
//    Weights stream straight from HBM into registers with 16-byte buffer
//    loads (each weight read once); the digit-split activations of up to
//    G = 16*NT/6 tokens are staged per K-chunk in LDS, double-buffered, in the
//    exact register order of the MFMA B operand.
//  * Grouped calls: each work-group scans the routing ids for its slot (a
//    stable, atomic-free gather), so a whole routed step is one launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4moe_device.h"
#include "q4moe_launch.h"

namespace q4 {

constexpr int kBufBytes = 40 * 1024;   // one of the two LDS staging buffers

// One work-group: WAVES wave64s, 16*RT rows of gate and up of one slot; waves
// split rows (RT) and K (KP = WAVES/RT, interleaved K-steps).  Each wave
// streams its weights in batches of D K-steps with two batches in flight
// (ping-pong registers), across LDS chunk barriers.  The digit-split
// activations of a token group (C = 6*count columns) are staged per chunk of
// `spc` K-steps into one of two LDS buffers, laid out as
// [step][parity][k-group g][column][16 bytes]: lane (g, column) of the MFMA B
// operand reads its 16 bytes with one ds_read_b128.
template <int NT, int RT, int WAVES, int D, bool VEC>
__global__ __launch_bounds__(WAVES * 64) void gate_up_kernel(const GateUpParams a) {
  constexpr int THREADS = WAVES * 64;
  constexpr int KP = WAVES / RT;
  constexpr int G = (16 * NT) / kSlices;    // tokens per group
  static_assert(WAVES % RT == 0, "row tiles must divide the waves");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBufBytes];
  __shared__ int s_pairs[G];
  __shared__ int s_xmax[G];
  __shared__ int s_count;
  __shared__ int s_invalid;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rt = wave % RT;
  const int kp = wave / RT;
  const int slot_idx = blockIdx.y;
  const int row0 = blockIdx.x * (16 * RT);
  const int H = a.H, I = a.I;
  const int P = a.M * a.K;                  // routed pairs
  const bool grouped = a.ids != nullptr;

  const uint8_t* slot = a.slots + (uint64_t)slot_idx * a.slot_stride;
  const uint32_t wbytes = (uint32_t)((uint64_t)I * (uint32_t)(H / 2));
  const __amdgpu_buffer_rsrc_t gsrc = make_rsrc(slot + a.gate_w_off, wbytes);
  const __amdgpu_buffer_rsrc_t usrc = make_rsrc(slot + a.up_w_off, wbytes);
  const float* gscale = (const float*)(slot + a.gate_s_off);
  const float* uscale = (const float*)(slot + a.up_s_off);

  // This lane's weight row in the A operand: row (lane % 16) of tile rt.
  const int arow = row0 + rt * 16 + (lane & 15);
  const uint32_t row_off = (uint32_t)(arow < I ? arow : I - 1) * (uint32_t)(H / 2) + (uint32_t)((lane >> 4) * 16);
  const int g4 = lane >> 4;
  const int cc = lane & 15;
  const int nsteps = (H + 127) / 128;
  const int my_steps = nsteps > kp ? (nsteps - kp + KP - 1) / KP : 0;   // steps kp, kp+KP, ...
  const int my_batches = (my_steps + D - 1) / D;

  // ---- invalid routing ids (grouped): slot 0's work-groups zero-fill them ----
  if (grouped && slot_idx == 0) {
    if (tid == 0) s_invalid = 0;
    __syncthreads();
    int cnt = 0;
    for (int p = tid; p < P; p += THREADS) {
      const int e = a.ids[p];
      if (e < 0 || e >= a.num_slots) {
        ++cnt;
        for (int r = 0; r < 16 * RT; ++r) {
          const int row = row0 + r;
          if (row >= I) break;
          const uint64_t o = (uint64_t)p * I + row;
          a.out[o] = 0;
          if (a.gate_probe) a.gate_probe[o] = 0.0f;
          if (a.up_probe) a.up_probe[o] = 0.0f;
        }
      }
    }
    if (cnt) atomicAdd(&s_invalid, cnt);
    __syncthreads();
    if (blockIdx.x == 0 && tid == 0 && a.invalid_count) *a.invalid_count = s_invalid;
  }

  struct Batch {
    v4u g[D], u[D];
  };
  auto issue = [&](int b, Batch& B) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int t = kp + KP * (b * D + d);
      if (t < nsteps) {
        const uint32_t off = row_off + (uint32_t)t * 64u;
        B.g[d] = load16<VEC>(gsrc, off);
        B.u[d] = load16<VEC>(usrc, off);
      }
    }
  };

  int next_pair = 0;
  for (;;) {
    __syncthreads();  // previous group's readers of s_pairs / lds are done
    // ---- gather up to G pairs routed to this slot (stable in pair order) ----
    if (!grouped) {
      if (tid < G) s_pairs[tid] = next_pair + tid;
      if (tid == 0) s_count = min(G, P - next_pair);
    } else if (wave == 0) {
      int found = 0;
      int p = next_pair;
      while (found < G && p < P) {
        const int q = p + lane;
        const bool m = q < P && a.ids[q] == slot_idx;
        const uint64_t bal = __ballot(m);
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        if (m && found + before < G) s_pairs[found + before] = q;
        found += __popcll(bal);
        p += 64;
      }
      if (lane == 0) s_count = min(found, G);
    }
    if (tid < G) s_xmax[tid] = 0;
    __syncthreads();
    const int count = s_count;
    if (count <= 0) break;
    next_pair = grouped ? s_pairs[count - 1] + 1 : next_pair + count;

    const int C = count * kSlices;            // used B columns
    const int ntiles = (C + 15) >> 4;
    // K-steps per chunk: as many as one buffer holds, a multiple of 2*KP*D so
    // every wave's batches pair up inside a chunk (the host plan guarantees
    // the buffer holds at least 2*KP*D steps of the widest group).
    int spc = kBufBytes / (128 * C);
    spc -= spc % (2 * KP * D);
    const int nchunks = (nsteps + spc - 1) / spc;
    const int pairs_per_chunk = spc / (2 * KP * D);

    // Weights of the first two batches go out before any activation work.
    Batch B0, B1;
    issue(0, B0);

    // ---- pass 1: largest |x| (as bf16 magnitude bits) of every token ----
    for (int ti = 0; ti < count; ++ti) {
      const int t = s_pairs[ti] / a.K;
      const uint4* xr = (const uint4*)(a.x + (uint64_t)t * H);
      uint32_t mx = 0;
      for (int w8 = tid; w8 < H / 8; w8 += THREADS) {
        const uint4 v = xr[w8];
        mx = max(mx, max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu)));
        mx = max(mx, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
      }
      if (mx) atomicMax(&s_xmax[ti], (int)mx);
    }
    __syncthreads();

    // ---- stage chunk c of the digit-split activations into buffer c&1 ----
    auto stage = [&](int c) {
      uint8_t* buf = lds + (c & 1) * kBufBytes;
      const int k0c = c * spc * 128;
      const int units = spc * 16;               // 8 positions per unit
      for (int u = tid; u < count * units; u += THREADS) {
        const int ti = u / units;
        const int w8 = u - ti * units;
        const int t = s_pairs[ti] / a.K;
        const int etop1 = max((s_xmax[ti] >> 7) & 0xFF, 1);
        const int k0 = k0c + 8 * w8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k0 < H) v = *(const uint4*)(a.x + (uint64_t)t * H + k0);
        const uint32_t xb[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                                v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const uint64_t z = x_digits(xb[p], etop1);
          lo[p] = (uint32_t)z;
          hi[p] = (uint32_t)(z >> 32);
        }
        const int tl = w8 >> 4, gg = (w8 >> 2) & 3, i = w8 & 3;
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          const uint32_t u01 = perm(lo[par + 2], lo[par], 0x05010400u);
          const uint32_t u23 = perm(lo[par + 2], lo[par], 0x07030602u);
          const uint32_t v01 = perm(lo[par + 6], lo[par + 4], 0x05010400u);
          const uint32_t v23 = perm(lo[par + 6], lo[par + 4], 0x07030602u);
          const uint32_t h01 = perm(hi[par + 2], hi[par], 0x05010400u);
          const uint32_t h45 = perm(hi[par + 6], hi[par + 4], 0x05010400u);
          const uint32_t d[6] = {perm(v01, u01, 0x05040100u), perm(v01, u01, 0x07060302u),
                                 perm(v23, u23, 0x05040100u), perm(v23, u23, 0x07060302u),
                                 perm(h45, h01, 0x05040100u), perm(h45, h01, 0x07060302u)};
          uint8_t* base = buf + (((tl * 2 + par) * 4 + gg) * C + ti * kSlices) * 16 + 4 * i;
#pragma unroll
          for (int s = 0; s < kSlices; ++s) *(uint32_t*)(base + s * 16) = d[s];
        }
      }
    };

    v4i accg[NT], accu[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      accg[n] = v4i{0, 0, 0, 0};
      accu[n] = v4i{0, 0, 0, 0};
    }

    // Column this lane reads in tile n (columns past C repeat the last one;
    // their results are never read).
    auto process = [&](const Batch& B, int b, const uint8_t* buf, int step0) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int t = kp + KP * (b * D + d);
        if (t < nsteps) {
          v4i ge, go, ue, uo;
          split_weights(B.g[d], ge, go);
          split_weights(B.u[d], ue, uo);
          const int tl = t - step0;
          const uint8_t* pe = buf + ((tl * 2 + 0) * 4 + g4) * C * 16;
          const uint8_t* po = buf + ((tl * 2 + 1) * 4 + g4) * C * 16;
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            if (n < ntiles) {
              const int col = min(16 * n + cc, C - 1);
              const v4i be = *(const v4i*)(pe + col * 16);
              const v4i bo = *(const v4i*)(po + col * 16);
              accg[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ge, be, accg[n], 0, 0, 0);
              accu[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ue, be, accu[n], 0, 0, 0);
              accg[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(go, bo, accg[n], 0, 0, 0);
              accu[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(uo, bo, accu[n], 0, 0, 0);
            }
          }
        }
      }
    };

    stage(0);
    __syncthreads();
    int b = 0;
    for (int c = 0; c < nchunks; ++c) {
      if (c + 1 < nchunks) stage(c + 1);
      const uint8_t* buf = lds + (c & 1) * kBufBytes;
      const int step0 = c * spc;
      for (int pp = 0; pp < pairs_per_chunk && b < my_batches; ++pp, b += 2) {
        if (b + 1 < my_batches) issue(b + 1, B1);
        process(B0, b, buf, step0);
        if (b + 2 < my_batches) issue(b + 2, B0);
        if (b + 1 < my_batches) process(B1, b + 1, buf, step0);
      }
      __syncthreads();
    }

    // ---- combine K-parts (exact int32 adds), then the digit matrix ----
    constexpr int PART_INTS = (KP - 1) * RT * NT * 8 * 64;
    int32_t* part = (int32_t*)lds;
    int32_t* eg = (int32_t*)lds + PART_INTS;               // [16*RT][C] gate
    int32_t* eu = eg + 16 * RT * C;                        // [16*RT][C] up
    if constexpr (KP > 1) {
      if (kp > 0) {
        int32_t* dst = part + ((kp - 1) * RT + rt) * (NT * 8 * 64);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            dst[((n * 2 + 0) * 4 + r) * 64 + lane] = accg[n][r];
            dst[((n * 2 + 1) * 4 + r) * 64 + lane] = accu[n][r];
          }
      }
      __syncthreads();
      if (kp == 0) {
        for (int k2 = 1; k2 < KP; ++k2) {
          const int32_t* src = part + ((k2 - 1) * RT + rt) * (NT * 8 * 64);
#pragma unroll
          for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              accg[n][r] += src[((n * 2 + 0) * 4 + r) * 64 + lane];
              accu[n][r] += src[((n * 2 + 1) * 4 + r) * 64 + lane];
            }
        }
      }
    }
    if (kp == 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int col = 16 * n + cc;
        if (col < C) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rt * 16 + 4 * g4 + r;
            eg[row * C + col] = accg[n][r];
            eu[row * C + col] = accu[n][r];
          }
        }
      }
    }
    __syncthreads();

    // ---- recombine digits, scale, tail, store ----
    for (int item = tid; item < 16 * RT * count; item += THREADS) {
      const int rr = item % (16 * RT);
      const int ti = item / (16 * RT);
      const int row = row0 + rr;
      if (row >= I) continue;
      const int p = s_pairs[ti];
      const int xm = s_xmax[ti];
      const int e2 = max((xm >> 7) & 0xFF, 1) - 176;  // 2^(e_top - 38) and the 16x weight factor
      const int32_t* gd = eg + rr * C + ti * kSlices;
      const int32_t* ud = eu + rr * C + ti * kSlices;
      const int64_t glo = (int64_t)gd[0] + ((int64_t)gd[1] << 8) + ((int64_t)gd[2] << 16);
      const int64_t ghi = (int64_t)gd[3] + ((int64_t)gd[4] << 8) + ((int64_t)gd[5] << 16);
      const int64_t ulo = (int64_t)ud[0] + ((int64_t)ud[1] << 8) + ((int64_t)ud[2] << 16);
      const int64_t uhi = (int64_t)ud[3] + ((int64_t)ud[4] << 8) + ((int64_t)ud[5] << 16);
      float gate = round_scaled(ghi, glo, e2, gscale[row]);
      float up = round_scaled(uhi, ulo, e2, uscale[row]);
      if (xm >= 0x7F80) {  // Inf or NaN in this token's activations
        gate = __builtin_nanf("");
        up = __builtin_nanf("");
      }
      const uint64_t o = (uint64_t)p * I + row;
      a.out[o] = swiglu_tail(gate, up);
      if (a.gate_probe) a.gate_probe[o] = gate;
      if (a.up_probe) a.up_probe[o] = up;
    }
    if (count < G) break;
    if (!grouped && next_pair >= P) break;
  }
}

// ---- launch configurations ----

template <int NT, int RT, int WAVES, int D>
constexpr bool fits() {
  // the widest group must leave room for one pair of batches per wave per chunk
  return kBufBytes / (128 * ((16 * NT) / kSlices) * kSlices) >= 2 * (WAVES / RT) * D;
}

template <int NT, int RT, int WAVES, int D, bool VEC>
static hipError_t launch_one(const GateUpParams& p, int num_slots, hipStream_t stream) {
  static_assert(fits<NT, RT, WAVES, D>(), "LDS chunk too small for this shape");
  const dim3 grid((unsigned)((p.I + 16 * RT - 1) / (16 * RT)), (unsigned)num_slots, 1);
  GateUpParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gate_up_kernel<NT, RT, WAVES, D, VEC>), grid,
                         dim3(WAVES * 64), args, 0, stream);
}

template <int NT, int RT, int D>
static hipError_t launch_vec(const GateUpParams& p, int num_slots, bool vec, hipStream_t stream) {
  return vec ? launch_one<NT, RT, 8, D, true>(p, num_slots, stream)
             : launch_one<NT, RT, 8, D, false>(p, num_slots, stream);
}

template <int NT>
static hipError_t launch_rt(const GateUpParams& p, int num_slots, int rt, bool vec, hipStream_t stream) {
  switch (rt) {
    case 8: return launch_vec<NT, 8, 2>(p, num_slots, vec, stream);
    case 4: return launch_vec<NT, 4, 1>(p, num_slots, vec, stream);
    default:
      if constexpr (fits<NT, 2, 8, 1>()) return launch_vec<NT, 2, 1>(p, num_slots, vec, stream);
      return launch_vec<NT, 4, 1>(p, num_slots, vec, stream);
  }
}

LaunchPlan plan_launch(int M_per_slot, int I, int num_slots, int H) {
  LaunchPlan lp;
  lp.nt = M_per_slot <= 2 ? 1 : (M_per_slot <= 5 ? 2 : 3);
  const int64_t wg8 = (int64_t)((I + 127) / 128) * num_slots;
  const int64_t wg4 = (int64_t)((I + 63) / 64) * num_slots;
  lp.rt = wg8 >= 512 ? 8 : (wg4 >= 512 ? 4 : 2);
  lp.vec = (H % 32) == 0;
  return lp;
}

hipError_t launch_gate_up(const GateUpParams& p, int num_slots, const LaunchPlan& lp, hipStream_t stream) {
  switch (lp.nt) {
    case 1: return launch_rt<1>(p, num_slots, lp.rt, lp.vec, stream);
    case 2: return launch_rt<2>(p, num_slots, lp.rt, lp.vec, stream);
    default: return launch_rt<3>(p, num_slots, lp.rt, lp.vec, stream);
  }
}

}  // namespace q4
