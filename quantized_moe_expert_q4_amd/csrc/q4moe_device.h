// Device arithmetic shared by the expert kernels (single-expert and grouped
// paths, Q4 and Q8 weights, gate/up and down): activation digit split, weight
// split, exact recombination with one F32 rounding, and the SwiGLU tail of
// GATE_UP_SOURCE (diff page 52 of @mlx-bun/inference 1.0.0,
// kernels/glm52/streamed-experts.ts).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kSlices = 6;       // digits per activation
constexpr int kFracBits = 38;    // X = x * 2^(38 - e_top): |X| <= 255 * 2^38 < 2^46

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

// The digits of x_digits without branches (for code that runs them between
// matrix-core operations): the magnitude is shifted 8 bits further than X
// needs (a shift below zero leaves nothing: the value is then under half a
// unit of X) and rounded half up by those 8 bits, which gives X for every
// shift x_digits takes.
__device__ __forceinline__ uint64_t x_digits_nb(uint32_t b, int etop1) {
  const uint32_t E = (b >> 7) & 0xFFu;
  const uint64_t mag = (b & 0x7Fu) | (E ? 0x80u : 0u);
  const int s8 = (int)(E ? E : 1u) - etop1 + kFracBits + 8;  // at most kFracBits + 8
  const uint64_t Xs = s8 >= 0 ? mag << (s8 & 63) : 0ull;
  const uint64_t Xm = (Xs + 0x80u) >> 8;
  const uint64_t X = (b & 0x8000u) ? 0ull - Xm : Xm;
  const uint64_t C = 0x808080808080ull;
  return (X + C) ^ C;
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

// Round V * 2^e2 * s to F32 once (nearest, ties to even) for |V| < 2^53,
// where V converts to double exactly.  The double product is rounded to odd
// (truncated toward zero, lowest bit set when inexact; the error term of one
// FMA says which), then scaled and rounded to F32: rounding to odd at 53 >=
// 24 + 2 bits followed by rounding to nearest gives the correctly rounded
// result (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
// proved algorithms using rounding to odd", IEEE TC 2008), for normal and
// subnormal F32 results alike.  Same value as round_scaled(V >> 24, V & 0xFFFFFF, e2, s).
__device__ __forceinline__ float round_scaled53(int64_t V, int e2, float s) {
#pragma clang fp contract(off)
  const double v = (double)V;
  const double sd = (double)s;
  double P = v * sd;
  const double err = __builtin_fma(v, sd, -P);  // v*sd == P + err exactly
  if (err != 0.0 && __builtin_isfinite(P)) {
    uint64_t b = (uint64_t)__double_as_longlong(P);
    if ((err < 0.0) != (P < 0.0)) b -= 1;       // P was rounded away from zero: step back toward it
    P = __longlong_as_double((long long)(b | 1u));
  }
  return (float)__builtin_ldexp(P, e2);
}

// bf16 sigmoid of the lane-0 tail of GATE_UP_SOURCE for a bf16 gate gT:
// exp(-gT) evaluated in double and rounded once to F32, then 1 + e and 1 / d
// in F32, rounded to bf16.
__device__ uint16_t sigmoid_bf16(uint16_t gb) {
#pragma clang fp contract(off)
  const float gT = bf16_val(gb);
  const float e = (float)exp(-(double)gT);
  const float d = 1.0f + e;
  const float sig = 1.0f / d;
  return bf16_rne(sig);
}

// The lane-0 tail: gate and up rounded to bf16, the bf16 sigmoid, silu and the
// product each rounded to bf16.
__device__ uint16_t swiglu_tail(float gate, float up) {
#pragma clang fp contract(off)
  const uint16_t gb = bf16_rne(gate);
  const float gT = bf16_val(gb);
  const float uT = bf16_val(bf16_rne(up));
  const float sT = bf16_val(sigmoid_bf16(gb));
  const float siluT = bf16_val(bf16_rne(gT * sT));
  return bf16_rne(siluT * uT);
}

// The bf16 sigmoid depends on the 16 bits of gT only.  For |gT| < 2^-9
// (exponent field below 118, zeros and subnormals included) it is exactly 0.5;
// for |gT| >= 128 (field 134 and up, infinities included) it is 1 for positive
// and +0 for negative gT; NaN stays NaN.  The 4096 values in between are
// tabulated once per device (kSigTable entries: sign, field 118..133, 7-bit
// mantissa) and copied into LDS by each work-group, which keeps the double
// exp out of the per-row tail.
constexpr int kSigTable = 2 * 16 * 128;

__device__ __forceinline__ uint16_t sig_table_bits(int i) {
  // entry i -> the bf16 gT it holds
  return (uint16_t)(((i >> 11) << 15) | ((118 + ((i >> 7) & 15)) << 7) | (i & 127));
}

__device__ __forceinline__ uint16_t swiglu_tail_tab(float gate, float up, const uint16_t* tab) {
#pragma clang fp contract(off)
  const uint16_t gb = bf16_rne(gate);
  const float gT = bf16_val(gb);
  const float uT = bf16_val(bf16_rne(up));
  const int ef = (gb >> 7) & 0xFF;
  uint16_t sb;
  if (ef < 118) sb = 0x3F00;
  else if (ef < 134) sb = tab[((gb >> 15) << 11) | ((ef - 118) << 7) | (gb & 127)];
  else if (ef < 255 || (gb & 127) == 0) sb = (gb & 0x8000) ? 0x0000 : 0x3F80;
  else sb = 0x7FC0;
  const float sT = bf16_val(sb);
  const float siluT = bf16_val(bf16_rne(gT * sT));
  return bf16_rne(siluT * uT);
}

// An empty asm that takes and gives back the four words of v: keeps the
// compiler from merging selects between held registers into an indexed
// load, which would move the registers to scratch memory.
__device__ __forceinline__ void opaque4(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// The 32-bit value of another lane of the same quad: DPP quad permute CTRL
// (0xB1: lane l ^ 1, 0x4E: lane l ^ 2).
template <int CTRL>
__device__ __forceinline__ int quad_dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// Exact (row, token) sum of the four digit columns of a lane quad of an MFMA
// 16x16 int32 result (lane 16g + c holds rows 4g..4g+3 of column c; columns
// 4t..4t+3 are digits 0..3 of token t): lane j = c % 4 of the quad receives
// row 4g + j, d0 + d1 2^8 + d2 2^16 + d3 2^24.  A 4x4 transpose of the
// quad's int32 values (lane bit 1 exchanged with register bit 1, then bit 0
// with bit 0, each a DPP quad permute and a select) leaves the lane with the
// four digit sums of its row.
__device__ __forceinline__ int64_t quad_digit_sum(const v4i acc, int j) {
  const bool b1 = (j & 2) != 0, b0 = (j & 1) != 0;
  const int x0 = quad_dpp<0x4E>(acc[2]), x1 = quad_dpp<0x4E>(acc[3]);
  const int y0 = quad_dpp<0x4E>(acc[0]), y1 = quad_dpp<0x4E>(acc[1]);
  const int t0 = b1 ? x0 : acc[0], t1 = b1 ? x1 : acc[1];
  const int t2 = b1 ? acc[2] : y0, t3 = b1 ? acc[3] : y1;
  const int p0 = quad_dpp<0xB1>(t0), p1 = quad_dpp<0xB1>(t1);
  const int p2 = quad_dpp<0xB1>(t2), p3 = quad_dpp<0xB1>(t3);
  const int d0 = b0 ? p1 : t0, d1 = b0 ? t1 : p0;
  const int d2 = b0 ? p3 : t2, d3 = b0 ? t3 : p2;
  return (int64_t)d0 + ((int64_t)d1 << 8) + ((int64_t)d2 << 16) + ((int64_t)d3 << 24);
}

// Largest (MAX) or smallest value of v over the 64 lanes of a wave, returned
// wave-uniform; every lane must be active.  Two quad permutes and two row
// rotations (DPP, no LDS round trip) leave each 16-lane row's extreme in all
// of its lanes; lanes 0, 16, 32 and 48 then combine on the scalar unit.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_extreme(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}

// Orders one wave's LDS stores before its later LDS loads from other lanes
// (and those loads before later stores): a wave barrier between release and
// acquire fences, so the compiler keeps every LDS access on its side.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The base and size must be the same in every lane of the wave (they are for
// every buffer here); they are moved to scalar registers, where the compiler
// could not prove it (a slot chosen from shared memory), so that a load needs
// no loop over the lanes' distinct resources.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

// 16 bytes at byte offset off through a buffer resource (zeros past its end).
__device__ __forceinline__ uint4 load_u4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A buffer offset past every weight array (projections are below 2^31 bytes):
// such a load returns zeros without a memory access.  Loads that are issued
// only to keep the number of outstanding loads fixed use it, so that the
// compiler's wait counts stay exact.
constexpr uint32_t kOffNone = 0x80000000u;

// s_waitcnt operand that waits for every vector memory load of the wave and
// leaves the export and LDS/scalar counters alone (vmcnt 0, expcnt 7,
// lgkmcnt 15).
constexpr int kWaitVmem0 = 0x0F70;

// Cache-policy operand of the buffer loads: 0 (default) or kLoadNT, the
// non-temporal hint for bytes that are read once.
constexpr int kLoadNT = 2;

template <bool VEC, int AUX = 0>
__device__ __forceinline__ v4u load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (VEC) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
  } else {
    v4u v;
    v.x = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX);
    v.y = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off + 4, 0, AUX);
    v.z = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off + 8, 0, AUX);
    v.w = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off + 12, 0, AUX);
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


// Signed int8 weights (the Q8 family of page 52, Q8_GATE_UP_SOURCE): the
// even (positions 0,2,..,30) and odd bytes of 32 consecutive weights, the
// same operand order split_weights gives for 32 nibbles, with weight factor 1.
__device__ __forceinline__ void split_bytes(const v4u a, const v4u b, v4i& ev, v4i& od) {
  ev.x = (int)perm(a.y, a.x, 0x06040200u);
  od.x = (int)perm(a.y, a.x, 0x07050301u);
  ev.y = (int)perm(a.w, a.z, 0x06040200u);
  od.y = (int)perm(a.w, a.z, 0x07050301u);
  ev.z = (int)perm(b.y, b.x, 0x06040200u);
  od.z = (int)perm(b.y, b.x, 0x07050301u);
  ev.w = (int)perm(b.w, b.z, 0x06040200u);
  od.w = (int)perm(b.w, b.z, 0x07050301u);
}

// One lane's weights of one K-step (128 weights of a row, the lane's k-group
// holding 32 of them): 16 bytes of packed nibbles (Q4) or 32 int8 (Q8).
template <bool Q8>
struct StepW {
  v4u a;
};
template <>
struct StepW<true> {
  v4u a, b;
};

// Row bytes of one K-step and of one k-group's share of it.
template <bool Q8>
__host__ __device__ constexpr uint32_t step_row_bytes() { return Q8 ? 128u : 64u; }
template <bool Q8>
__host__ __device__ constexpr uint32_t group_bytes() { return Q8 ? 32u : 16u; }
// Bytes of one weight row of K values.
template <bool Q8>
__host__ __device__ constexpr uint32_t row_bytes(int K) { return Q8 ? (uint32_t)K : (uint32_t)(K / 2); }
// Exponent of the integer weight factor the MFMA operands carry (16 for the
// nibble split, 1 for int8 bytes), relative to the nibble split.
template <bool Q8>
__host__ __device__ constexpr int weight_exp_shift() { return Q8 ? 4 : 0; }

template <bool Q8, bool VEC>
__device__ __forceinline__ void load_step(StepW<Q8>& w, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  w.a = load16<VEC>(r, off);
  if constexpr (Q8) w.b = load16<VEC>(r, off + 16u);
}

// ---- whole-line weight loads (32 bytes per lane and step) ----
// One K-step of a 16-row tile is 16 rows x 128 bytes.  Loaded with 8 lanes
// per row, every load instruction covers whole 128-byte lines (with the
// non-temporal hint this streams ~14% faster than 4 lanes per row on
// MI355X): lane L receives bytes 16 (L % 8) .. +16 of tile rows L / 8 (.a)
// and 8 + L / 8 (.b).  line_to_tile then moves them across lanes to the
// layout the splits take, lane 16 g + r holding bytes 32 g .. 32 g + 32 of
// row r (.a the first 16): one DPP swap of odd and even lanes, a select and
// one ds_bpermute per dword.
template <bool VEC>
__device__ __forceinline__ void load_line(StepW<true>& w, __amdgpu_buffer_rsrc_t r, uint32_t off_a, uint32_t off_b) {
  w.a = load16<VEC, kLoadNT>(r, off_a);
  w.b = load16<VEC, kLoadNT>(r, off_b);
}

struct LineLanes {
  int addr_a, addr_b;  // ds_bpermute byte addresses of the lane's sources
  bool even;
};

__device__ __forceinline__ LineLanes line_lanes(int lane) {
  const int g = lane >> 4, r = lane & 15;
  // piece 2g (.a) / 2g+1 (.b) of row r: rows 0..7 come from .a of lane
  // 8r + piece, rows 8..15 from .b of lane 8(r-8) + piece, staged at the
  // neighbour lane (piece ^ 1) by the swap
  LineLanes l;
  l.addr_a = 4 * (8 * (r & 7) + 2 * g + (r >> 3));
  l.addr_b = 4 * (8 * (r & 7) + 2 * g + 1 - (r >> 3));
  l.even = (lane & 1) == 0;
  return l;
}

__device__ __forceinline__ void line_to_tile(StepW<true>& w, const LineLanes& l) {
  v4u na, nb;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // .b of the neighbour lane (quad_perm 1,0,3,2)
    const int bs = __builtin_amdgcn_mov_dpp((int)w.b[k], 0xB1, 0xF, 0xF, true);
    const int xa = l.even ? (int)w.a[k] : bs;
    const int xb = l.even ? bs : (int)w.a[k];
    na[k] = (uint32_t)__builtin_amdgcn_ds_bpermute(l.addr_a, xa);
    nb[k] = (uint32_t)__builtin_amdgcn_ds_bpermute(l.addr_b, xb);
  }
  w.a = na;
  w.b = nb;
}

__device__ __forceinline__ void split_step(const StepW<false>& w, v4i& ev, v4i& od) { split_weights(w.a, ev, od); }
__device__ __forceinline__ void split_step(const StepW<true>& w, v4i& ev, v4i& od) { split_bytes(w.a, w.b, ev, od); }

// ---- wide K-steps of packed nibbles (256 weights per row and step) ----
// A lane holds eight words (64 nibbles, K = base + 8w + p) of its k-group and
// feeds four MFMAs per step, one per plane.  Word w gives two operand dwords,
// its even nibbles (p = 0, 2, 4, 6 as bytes 0..3) and its odd ones (p = 1, 3,
// 5, 7), each nibble as the int8 16*(q-8): plane 0 holds the even dwords of
// words 0..3 (dword i from word i), plane 1 their odd dwords, planes 2 and 3
// the same for words 4..7.  Three operations per word.
__device__ __forceinline__ void split_planes(const v4u a, const v4u b, v4i (&pl)[4]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the zero-point xor is folded into each mask (one 3-input op per dword)
    pl[0][i] = (int)(((w[i] << 4) ^ 0x88888880u) & 0xF0F0F0F0u);       // p = 0, 2, 4, 6
    pl[1][i] = (int)((w[i] ^ 0x88888888u) & 0xF0F0F0F0u);              // p = 1, 3, 5, 7
    pl[2][i] = (int)(((w[4 + i] << 4) ^ 0x88888880u) & 0xF0F0F0F0u);
    pl[3][i] = (int)((w[4 + i] ^ 0x88888888u) & 0xF0F0F0F0u);
  }
}

// 4x4 byte transpose: o[s] = byte s of a, b, c, d as bytes 0..3.
__device__ __forceinline__ void transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t (&o)[4]) {
  const uint32_t ab01 = perm(b, a, 0x05010400u), ab23 = perm(b, a, 0x07030602u);  // [a0 b0 a1 b1], [a2 b2 a3 b3]
  const uint32_t cd01 = perm(d, c, 0x05010400u), cd23 = perm(d, c, 0x07030602u);
  o[0] = perm(cd01, ab01, 0x05040100u);
  o[1] = perm(cd01, ab01, 0x07060302u);
  o[2] = perm(cd23, ab23, 0x05040100u);
  o[3] = perm(cd23, ab23, 0x07060302u);
}

// Digit dwords of one word in the operand order of split_planes: v[p] holds
// four digits (bytes 0..3) of the activation at position p of the word;
// ev[s] / od[s] receive digit s of positions 0, 2, 4, 6 / 1, 3, 5, 7.
__device__ __forceinline__ void plane_digits4(const uint32_t (&v)[8], uint32_t (&ev)[4], uint32_t (&od)[4]) {
  transpose4(v[0], v[2], v[4], v[6], ev);
  transpose4(v[1], v[3], v[5], v[7], od);
}

// Byte transpose of eight digit words: lo[p]/hi[p] hold digits 0..3 / 4..5 of
// position p (p = 0..7 of one packed word); d[s] receives digit s of the four
// positions of parity `par` (p = par, par+2, par+4, par+6), one byte each --
// the byte order of one MFMA B-operand dword.
__device__ __forceinline__ void digit_words(const uint32_t (&lo)[8], const uint32_t (&hi)[8], int par,
                                            uint32_t (&d)[6]) {
  const uint32_t u01 = perm(lo[par + 2], lo[par], 0x05010400u);
  const uint32_t u23 = perm(lo[par + 2], lo[par], 0x07030602u);
  const uint32_t v01 = perm(lo[par + 6], lo[par + 4], 0x05010400u);
  const uint32_t v23 = perm(lo[par + 6], lo[par + 4], 0x07030602u);
  const uint32_t h01 = perm(hi[par + 2], hi[par], 0x05010400u);
  const uint32_t h45 = perm(hi[par + 6], hi[par + 4], 0x05010400u);
  d[0] = perm(v01, u01, 0x05040100u);
  d[1] = perm(v01, u01, 0x07060302u);
  d[2] = perm(v23, u23, 0x05040100u);
  d[3] = perm(v23, u23, 0x07060302u);
  d[4] = perm(h45, h01, 0x05040100u);
  d[5] = perm(h45, h01, 0x07060302u);
}

// Digits of the eight bf16 activations packed in one uint4 (positions 0..7).
__device__ __forceinline__ void x8_digits(const uint4 v, int etop1, uint32_t (&lo)[8], uint32_t (&hi)[8]) {
  const uint32_t xb[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                          v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint64_t z = x_digits(xb[p], etop1);
    lo[p] = (uint32_t)z;
    hi[p] = (uint32_t)(z >> 32);
  }
}

// Four-digit split for tokens whose values all lie within 22 binades of the
// largest (see digits_for): X = x * 2^(22 - e_top) is an integer below 2^30
// in magnitude, and its four balanced base-256 digits are the bytes of one
// 32-bit word.  The digits equal digits 0..3 of x_digits(b, etop1 + 16),
// whose digits 4 and 5 are then zero.  Zero values give zero digits for any
// shift; non-zero values have a shift in [0, 22].
__device__ __forceinline__ uint32_t x_digits4(uint32_t b, int etop1) {
  // X = x * 2^(156 - etop1): x = mag * 2^(max(E,1) - 134), so X = mag * 2^(max(E,1)
  // - etop1 + 22), an integer of at most 30 bits for the values this split
  // is used for; ldexp and the conversion are exact and carry the sign.
  const int X = (int)__builtin_ldexpf(__uint_as_float(b << 16), 156 - etop1);
  return ((uint32_t)X + 0x80808080u) ^ 0x80808080u;
}

// Four-digit words of eight packed bf16 activations: d[par][s] holds digit s
// of positions par, par+2, par+4, par+6 (one byte each), the byte order of
// one MFMA B-operand dword.
__device__ __forceinline__ void x8_digits4(const uint4 v, int etop1, uint32_t (&d)[2][4]) {
  const uint32_t xb[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                          v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
  uint32_t w[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) w[p] = x_digits4(xb[p], etop1);
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const uint32_t u01 = perm(w[par + 2], w[par], 0x05010400u);
    const uint32_t u23 = perm(w[par + 2], w[par], 0x07030602u);
    const uint32_t v01 = perm(w[par + 6], w[par + 4], 0x05010400u);
    const uint32_t v23 = perm(w[par + 6], w[par + 4], 0x07030602u);
    d[par][0] = perm(v01, u01, 0x05040100u);
    d[par][1] = perm(v01, u01, 0x07060302u);
    d[par][2] = perm(v23, u23, 0x05040100u);
    d[par][3] = perm(v23, u23, 0x07060302u);
  }
}

// ---- f32 activations ----
// Eight balanced base-256 digits of X = round(x * 2^(188 - etop1)) for an f32
// value x (|X| <= 2^62; `etop1` is max(exponent field of the token's largest
// |x|, 1)).  Values at most 38 binades below the largest are exact; smaller
// ones are rounded to the grid (half away from zero).  The sum of products
// is then V * 2^(etop1 - 192) with the 16x weight factor.
__device__ __forceinline__ uint64_t xf_digits(uint32_t b, int etop1) {
  const uint32_t E = (b >> 23) & 0xFFu;
  const uint32_t mag = (b & 0x7FFFFFu) | (E ? 0x800000u : 0u);
  const int sh = (int)(E ? E : 1u) - etop1 + 38;
  int64_t X;
  if (sh >= 0) {
    X = (int64_t)mag << sh;
  } else if (sh >= -24) {
    X = (int64_t)((mag + (1u << (-sh - 1))) >> (-sh));
  } else {
    X = 0;
  }
  if (b & 0x80000000u) X = -X;
  const uint64_t C = 0x8080808080808080ull;
  return ((uint64_t)X + C) ^ C;
}

// Byte transpose of eight words of four digits each (positions p = 0..7):
// d[s] receives digit s of positions par, par+2, par+4, par+6.
__device__ __forceinline__ void transpose4(const uint32_t (&w)[8], int par, uint32_t (&d)[4]) {
  const uint32_t u01 = perm(w[par + 2], w[par], 0x05010400u);
  const uint32_t u23 = perm(w[par + 2], w[par], 0x07030602u);
  const uint32_t v01 = perm(w[par + 6], w[par + 4], 0x05010400u);
  const uint32_t v23 = perm(w[par + 6], w[par + 4], 0x07030602u);
  d[0] = perm(v01, u01, 0x05040100u);
  d[1] = perm(v01, u01, 0x07060302u);
  d[2] = perm(v23, u23, 0x05040100u);
  d[3] = perm(v23, u23, 0x07060302u);
}

// Digit words of eight f32 activations (positions 0..3 in `a`, 4..7 in `b`):
// d[par][s], s = 0..7, holds digit s of positions par, par+2, par+4, par+6.
__device__ __forceinline__ void xf8_digits(const uint4 a, const uint4 b, int etop1, uint32_t (&d)[2][8]) {
  const uint32_t xb[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t lo[8], hi[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint64_t z = xf_digits(xb[p], etop1);
    lo[p] = (uint32_t)z;
    hi[p] = (uint32_t)(z >> 32);
  }
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    uint32_t l4[4], h4[4];
    transpose4(lo, par, l4);
    transpose4(hi, par, h4);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      d[par][s] = l4[s];
      d[par][4 + s] = h4[s];
    }
  }
}

// Largest f32 magnitude bits and smallest non-zero exponent field (at least
// 1; 255 if none) among eight f32 activations.
__device__ __forceinline__ void f32_range8(const uint4 a, const uint4 b, uint32_t& mx, uint32_t& mn) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  mx = 0u;
  mn = 255u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t m = w[i] & 0x7FFFFFFFu;
    mx = max(mx, m);
    if (m) mn = min(mn, max((m >> 23) & 0xFFu, 1u));
  }
}

// Exponent offset of an eight-digit f32 sum: sum(w*x) = V * 2^(etop1 - 192).
__device__ __forceinline__ int sum_exponent_f32(uint32_t xmax_bits) {
  return max((int)((xmax_bits >> 23) & 0xFFu), 1) - 192;
}

// Round (hi * 2^32 + lo) * 2^e2 * s to F32 once (nearest, ties to even),
// exactly, with integer arithmetic: the eight-digit sums have up to 88
// significant bits, so the product with the scale's 24-bit significand
// (up to 112 bits) is formed in two 64-bit words and rounded from its top
// 64 bits and a sticky bit.  A zero result has the sign of the IEEE product:
// the scale's for a zero sum, that of the two factors for a zero scale.
__device__ float round_scaled_wide(int64_t hi, int64_t lo, int e2, float s) {
  // V = hi * 2^32 + lo as a sign and a 128-bit magnitude (vh:vl)
  const int64_t lo_hi = lo >> 32;                       // arithmetic: floor(lo / 2^32)
  const uint64_t lo_lo = (uint64_t)lo & 0xFFFFFFFFull;
  const int64_t top = hi + lo_hi;                        // V = top * 2^32 + lo_lo, |top| < 2^63
  uint64_t vh, vl;
  bool neg = top < 0;
  if (!neg) {
    vh = (uint64_t)top >> 32;
    vl = ((uint64_t)top << 32) | lo_lo;
  } else {
    // |V| = -(top * 2^32 + lo_lo) = (-top) * 2^32 - lo_lo
    const uint64_t t = (uint64_t)(-top);
    uint64_t h = t >> 32, l = t << 32;
    if (lo_lo) {
      h -= (l < lo_lo) ? 1u : 0u;
      l -= lo_lo;
    }
    vh = h;
    vl = l;
  }
  const uint32_t sb = __float_as_uint(s);
  const uint32_t se = (sb >> 23) & 0xFFu;
  const uint64_t m = (sb & 0x7FFFFFu) | (se ? 0x800000u : 0u);
  const int es = (int)(se ? se : 1u) - 150;
  if (sb & 0x80000000u) neg = !neg;
  // N = |V| * m over three 32-bit limbs of |V| (|V| < 2^88)
  const uint64_t a0 = vl & 0xFFFFFFFFull, a1 = vl >> 32, a2 = vh;
  const uint64_t p0 = a0 * m, p1 = a1 * m, p2 = a2 * m;
  uint64_t nl = p0 + (p1 << 32);
  const uint64_t c = nl < p0 ? 1u : 0u;
  const uint64_t nh = (p1 >> 32) + p2 + c;
  if ((nh | nl) == 0) return __uint_as_float(neg ? 0x80000000u : 0u);   // V = 0 (neg: the scale's sign) or s = 0
  // top 64 bits T of N (its most significant bit at bit 63) and a sticky bit
  int msb;
  uint64_t T;
  bool sticky;
  if (nh) {
    const int lz = __builtin_clzll(nh);
    msb = 127 - lz;
    T = lz ? ((nh << lz) | (nl >> (64 - lz))) : nh;
    sticky = lz ? (nl << lz) != 0 : nl != 0;
  } else {
    const int lz = __builtin_clzll(nl);
    msb = 63 - lz;
    T = nl << lz;
    sticky = false;
  }
  // value = (T + below) * 2^(E), E the weight of T's bit 0
  const int E = e2 + es + msb - 63;
  const int topexp = E + 63;                              // exponent of T's leading bit
  const int keep = topexp >= -126 ? 24 : 24 - (-126 - topexp);
  float r;
  if (keep <= 0) {
    // below half of the smallest subnormal unless exactly at it with more below
    const bool up = keep == 0 && (T > (1ull << 63) || sticky);
    r = up ? __builtin_ldexpf(1.0f, -149) : 0.0f;
  } else {
    const int drop = 64 - keep;                           // >= 40
    uint64_t q = T >> drop;
    const uint64_t rem = T & ((1ull << drop) - 1ull);
    const uint64_t half = 1ull << (drop - 1);
    if (rem > half || (rem == half && (sticky || (q & 1ull)))) ++q;
    r = __builtin_ldexpf((float)q, E + drop);
  }
  return neg ? -r : r;
}

// The lane-0 tail with T = float: every conversion to T is the identity.
__device__ float swiglu_tail_f32(float gate, float up) {
#pragma clang fp contract(off)
  const float e = (float)exp(-(double)gate);
  const float d = 1.0f + e;
  const float sg = 1.0f / d;
  return (gate * sg) * up;
}

// Range of eight packed bf16 activations: the largest magnitude bits (0 if
// all are zero) and the smallest exponent field, at least 1, among the
// non-zero values (255 if none).  The field grows with the magnitude, so it
// is the field of the smallest non-zero magnitude, found as the smallest
// magnitude - 1 with zero wrapping to the top.
__device__ __forceinline__ void range8(const uint4 v, uint32_t& mx, uint32_t& mn) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t hi = 0u, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a0 = w[i] & 0x7FFFu, a1 = (w[i] >> 16) & 0x7FFFu;
    hi = max(hi, max(a0, a1));
    lo = min(lo, min(a0 - 1u, a1 - 1u));
  }
  mx = hi;
  mn = lo == 0xFFFFFFFFu ? 255u : max((lo + 1u) >> 7, 1u);
}

// Exponent offset of the recombined sum: sum(w*x) = V * 2^(etop1 - 176)
// (X = x * 2^(172 - etop1) and the 16x weight factor).
__device__ __forceinline__ int sum_exponent(int xmax_bits) { return max((xmax_bits >> 7) & 0xFF, 1) - 176; }

// Digits per value for a token whose largest |x| has bits xmax and whose
// smallest non-zero exponent field is emin: four when every value sits
// within 22 binades of the largest (x * 2^(22 - e_top) is then an integer of
// magnitude below 2^30, so the four-digit split is exact and gives the same
// sum as six digits), else six.  Non-finite tokens keep six.
__device__ __forceinline__ int digits_for(int xmax, int emin) {
  return (xmax < 0x7F80 && emin >= max((xmax >> 7) & 0xFF, 1) - (kFracBits - 16)) ? 4 : 6;
}

}  // namespace q4
