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

#include "q4moe_launch.h"

namespace q4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kSlices = 6;       // digits per activation
constexpr int kFracBits = 38;    // X = x * 2^(38 - e_top): |X| <= 255 * 2^38 < 2^46
constexpr int kLdsBytes = 48 * 1024;

// K positions staged per LDS buffer: 2 buffers * KC * 16 * NT bytes = 48 KiB.
template <int NT> struct Chunk { static constexpr int KC = 128 * (12 / NT); };

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Six balanced base-256 digits (two's-complement bytes 0..5) of
// X = round(x * 2^(38 - e_top)); `etop1` is max(exponent field of the token's
// largest |x|, 1).  Entries more than 38 binades below the largest are rounded
// to the grid (half away from zero).
__device__ __forceinline__ uint64_t x_digits(uint32_t b, int etop1) {
  const uint32_t E = (b >> 7) & 0xFFu;
  const uint32_t mag = (b & 0x7Fu) | (E ? 0x80u : 0u);
  const int sh = (int)(E ? E : 1u) - etop1 + kFracBits;
  int64_t X;
  if (sh >= 0) {
    X = (int64_t)mag << sh;
  } else if (sh >= -8) {
    X = (int64_t)((mag + (1u << (-sh - 1))) >> (-sh));
  } else {
    X = 0;
  }
  if (b & 0x8000u) X = -X;
  const uint64_t C = 0x808080808080ull;  // 128 in every digit: offset to unsigned bytes
  return ((uint64_t)X + C) ^ C;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round (hi * 2^24 + lo) * 2^e2 * s to F32 once (nearest, ties to even).
// (P, c) is a double-double of the exact product with error below 2^-105 of
// it, while a non-zero distance to an F32 rounding midpoint is at least
// ~2^-95 of it (the product has at most 95 significant bits), so the sign
// test below decides every case exactly.
__device__ float round_scaled(int64_t hi, int64_t lo, int e2, float s) {
#pragma clang fp contract(off)
  const double vh = (double)hi * 16777216.0;  // exact: |hi| < 2^47
  const double vl = (double)lo;               // exact: |lo| < 2^47
  const double S = vh + vl;
  const double bb = S - vh;
  const double eS = (vh - (S - bb)) + (vl - bb);  // S + eS == vh + vl exactly
  const double sd = (double)s;
  double P = S * sd;
  const double eP = __builtin_fma(S, sd, -P);      // S*sd == P + eP exactly
  double c = eP + eS * sd;
  P = __builtin_ldexp(P, e2);
  c = __builtin_ldexp(c, e2);
  float r = (float)P;
  if (!__builtin_isfinite(r)) return r;
  const double rd = (double)r;
  const double diff = (P - rd) + c;  // true value minus r (P - rd is exact)
  if (diff != 0.0) {
    const float n = nextafterf(r, diff > 0.0 ? __builtin_inff() : -__builtin_inff());
    const double mid = 0.5 * (rd + (double)n);
    const double dm = (P - mid) + c;  // true value minus the midpoint toward n
    const bool beyond = diff > 0.0 ? (dm > 0.0) : (dm < 0.0);
    if (beyond || (dm == 0.0 && (__float_as_uint(r) & 1u))) r = n;
  }
  return r;
}

// The lane-0 tail of GATE_UP_SOURCE: gate and up rounded to bf16, sigmoid in
// F32 (exp evaluated in double and rounded once to F32), silu and the product
// each rounded to bf16.
__device__ uint16_t swiglu_tail(float gate, float up) {
#pragma clang fp contract(off)
  const float gT = bf16_val(bf16_rne(gate));
  const float uT = bf16_val(bf16_rne(up));
  const float e = (float)exp(-(double)gT);
  const float d = 1.0f + e;
  const float sig = 1.0f / d;
  const float sT = bf16_val(bf16_rne(sig));
  const float siluT = bf16_val(bf16_rne(gT * sT));
  return bf16_rne(siluT * uT);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <bool VEC>
__device__ __forceinline__ v4u load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (VEC) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  } else {
    v4u v;
    v.x = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    v.y = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off + 4, 0, 0);
    v.z = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off + 8, 0, 0);
    v.w = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off + 12, 0, 0);
    return v;
  }
}

// 16*(q-8) as int8 for the even (p = 0,2,4,6) and odd nibbles of four words.
__device__ __forceinline__ void split_weights(const v4u w, v4i& ev, v4i& od) {
  const uint32_t a0 = w.x ^ 0x88888888u, a1 = w.y ^ 0x88888888u;
  const uint32_t a2 = w.z ^ 0x88888888u, a3 = w.w ^ 0x88888888u;
  od.x = (int)(a0 & 0xF0F0F0F0u);
  od.y = (int)(a1 & 0xF0F0F0F0u);
  od.z = (int)(a2 & 0xF0F0F0F0u);
  od.w = (int)(a3 & 0xF0F0F0F0u);
  ev.x = (int)((a0 << 4) & 0xF0F0F0F0u);
  ev.y = (int)((a1 << 4) & 0xF0F0F0F0u);
  ev.z = (int)((a2 << 4) & 0xF0F0F0F0u);
  ev.w = (int)((a3 << 4) & 0xF0F0F0F0u);
}

template <int NT, int RT, bool VEC>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(const GateUpParams a) {
  constexpr int KP = kWaves / RT;
  constexpr int KC = Chunk<NT>::KC;
  constexpr int STEPS = KC / 128;           // MFMA K-steps of 128 positions per chunk
  constexpr int COLS = 16 * NT;
  constexpr int G = COLS / kSlices;         // tokens per group
  constexpr int BUF = KC * COLS;            // bytes per staging buffer

  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
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
  const uint32_t row_off = (uint32_t)(arow < I ? arow : I - 1) * (uint32_t)(H / 2);
  const int g4 = lane >> 4;
  const int nsteps_total = (H + 127) / 128;
  const int nchunks = (H + KC - 1) / KC;

  // ---- invalid routing ids (grouped): slot 0's work-groups zero-fill them ----
  if (grouped && slot_idx == 0) {
    if (tid == 0) s_invalid = 0;
    __syncthreads();
    int cnt = 0;
    for (int p = tid; p < P; p += kThreads) {
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

    // ---- pass 1: largest |x| (as bf16 magnitude bits) of every token ----
    for (int ti = 0; ti < count; ++ti) {
      const int t = s_pairs[ti] / a.K;
      const uint4* xr = (const uint4*)(a.x + (uint64_t)t * H);
      uint32_t mx = 0;
      for (int w8 = tid; w8 < H / 8; w8 += kThreads) {
        const uint4 v = xr[w8];
        mx = max(mx, max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu)));
        mx = max(mx, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
      }
      if (mx) atomicMax(&s_xmax[ti], (int)mx);
    }
    __syncthreads();

    // ---- stage chunk c of the digit-split activations into buffer c&1 ----
    auto stage = [&](int c) {
      uint8_t* buf = lds + (c & 1) * BUF;
      const int k0c = c * KC;
      for (int ti = 0; ti < count; ++ti) {
        const int t = s_pairs[ti] / a.K;
        const int etop1 = max((s_xmax[ti] >> 7) & 0xFF, 1);
        const uint16_t* xr = a.x + (uint64_t)t * H;
        for (int w8 = tid; w8 < KC / 8; w8 += kThreads) {
          const int k0 = k0c + 8 * w8;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (k0 < H) v = *(const uint4*)(xr + k0);
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
#pragma unroll
            for (int s = 0; s < kSlices; ++s) {
              const int cs = ti * kSlices + s;
              const int tile = cs >> 4, cc = cs & 15;
              const int addr = ((tl * 2 + par) * NT + tile) * 1024 + (gg * 16 + cc) * 16 + 4 * i;
              *(uint32_t*)(buf + addr) = d[s];
            }
          }
        }
      }
    };

    v4i accg[NT], accu[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      accg[n] = v4i{0, 0, 0, 0};
      accu[n] = v4i{0, 0, 0, 0};
    }

    stage(0);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      if (c + 1 < nchunks) stage(c + 1);
      const uint8_t* buf = lds + (c & 1) * BUF;
      const int steps = min(STEPS, nsteps_total - c * STEPS);
      int tl = kp;
      v4u ng = {0, 0, 0, 0}, nu = {0, 0, 0, 0};
      if (tl < steps) {
        const uint32_t off = row_off + (uint32_t)((c * STEPS + tl) * 64 + g4 * 16);
        ng = load16<VEC>(gsrc, off);
        nu = load16<VEC>(usrc, off);
      }
      for (; tl < steps; tl += KP) {
        const v4u wg = ng, wu = nu;
        if (tl + KP < steps) {
          const uint32_t off = row_off + (uint32_t)((c * STEPS + tl + KP) * 64 + g4 * 16);
          ng = load16<VEC>(gsrc, off);
          nu = load16<VEC>(usrc, off);
        }
        v4i ge, go, ue, uo;
        split_weights(wg, ge, go);
        split_weights(wu, ue, uo);
        const uint8_t* bp = buf + (tl * 2 * NT) * 1024 + lane * 16;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const v4i be = *(const v4i*)(bp + n * 1024);
          const v4i bo = *(const v4i*)(bp + (NT + n) * 1024);
          accg[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ge, be, accg[n], 0, 0, 0);
          accu[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ue, be, accu[n], 0, 0, 0);
          accg[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(go, bo, accg[n], 0, 0, 0);
          accu[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(uo, bo, accu[n], 0, 0, 0);
        }
      }
      __syncthreads();
    }

    // ---- combine K-parts (exact int32 adds) ----
    int32_t* part = (int32_t*)lds;                          // (KP-1)*RT waves * NT*2*4*64 ints
    int32_t* eg = (int32_t*)(lds + 24 * 1024);              // [16*RT][COLS] gate
    int32_t* eu = eg + 16 * RT * COLS;                      // [16*RT][COLS] up
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
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rt * 16 + 4 * g4 + r;
          const int col = n * 16 + (lane & 15);
          eg[row * COLS + col] = accg[n][r];
          eu[row * COLS + col] = accu[n][r];
        }
    }
    __syncthreads();

    // ---- recombine digits, scale, tail, store ----
    for (int item = tid; item < 16 * RT * count; item += kThreads) {
      const int rr = item % (16 * RT);
      const int ti = item / (16 * RT);
      const int row = row0 + rr;
      if (row >= I) continue;
      const int p = s_pairs[ti];
      const int xm = s_xmax[ti];
      const int e2 = max((xm >> 7) & 0xFF, 1) - 176;  // 2^(e_top - 38) and the 16x weight factor
      const int32_t* gd = eg + rr * COLS + ti * kSlices;
      const int32_t* ud = eu + rr * COLS + ti * kSlices;
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

template <int NT, int RT, bool VEC>
static hipError_t launch_one(const GateUpParams& p, int num_slots, hipStream_t stream) {
  const dim3 grid((unsigned)((p.I + 16 * RT - 1) / (16 * RT)), (unsigned)num_slots, 1);
  GateUpParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gate_up_kernel<NT, RT, VEC>), grid,
                         dim3(kThreads), args, 0, stream);
}

template <int NT, int RT>
static hipError_t launch_vec(const GateUpParams& p, int num_slots, bool vec, hipStream_t stream) {
  return vec ? launch_one<NT, RT, true>(p, num_slots, stream)
             : launch_one<NT, RT, false>(p, num_slots, stream);
}

template <int NT>
static hipError_t launch_rt(const GateUpParams& p, int num_slots, int rt, bool vec, hipStream_t stream) {
  switch (rt) {
    case 4: return launch_vec<NT, 4>(p, num_slots, vec, stream);
    case 2: return launch_vec<NT, 2>(p, num_slots, vec, stream);
    default: return launch_vec<NT, 1>(p, num_slots, vec, stream);
  }
}

LaunchPlan plan_launch(int M_per_slot, int I, int num_slots, int H) {
  LaunchPlan lp;
  lp.nt = M_per_slot <= 2 ? 1 : (M_per_slot <= 5 ? 2 : 3);
  const int64_t wg4 = (int64_t)((I + 63) / 64) * num_slots;
  const int64_t wg2 = (int64_t)((I + 31) / 32) * num_slots;
  lp.rt = wg4 >= 512 ? 4 : (wg2 >= 512 ? 2 : 1);
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
