// Internal interface between the C ABI (q4moe_abi.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace q4 {

// Everything one launch of a gate/up or down kernel reads.  `ids == nullptr`
// is the single-expert call: every token routed to slot 0 with K == 1.
// With `down` set the launch is the down projection: H is the reduction
// length (the expert's intermediate size), I the number of output rows (its
// hidden size), gate_w_off/gate_s_off locate the down weights and scales, and
// gate_probe (if any) receives the F32 values before their bf16 rounding.
struct GateUpParams {
  const uint8_t* slots;      // slot 0 base (4096-aligned)
  uint64_t slot_stride;      // bytes between slots
  uint64_t gate_w_off, up_w_off, gate_s_off, up_s_off;
  const uint16_t* x;         // bf16 [M][H] (float [M][H] with xf32)
  const int32_t* ids;        // int32 [M][K] or nullptr
  uint16_t* out;             // bf16 [M*K][I] (float with xf32)
  float* gate_probe;         // F32 [M*K][I] or nullptr
  float* up_probe;           // F32 [M*K][I] or nullptr
  int32_t* invalid_count;    // grouped: number of out-of-range ids, or nullptr
  int M, K, H, I, num_slots;
  int G, steps;              // set by the launchers: tokens per group, K-steps per tile
  int wave_share;            // set by launch_resident: a SIMD's first-wave share, 1/1024
  int down;                  // 1: down projection (see above)
  int q8;                    // 1: signed int8 weights [rows][H] (else packed nibbles [rows][H/8] words)
  int xf32;                  // 1: x and out are float32 (else bf16); probes unchanged
  const uint16_t* sig;       // set by the launchers: the device's bf16 sigmoid table (sigmoid_table)
  int seg_cost;              // set by launch_chunked: a segment's set-up cost, in K-steps of one tile
};

// The bf16 sigmoid table of the SwiGLU tail on the current device
// (kSigTable entries, see q4moe_device.h), built on first use.
hipError_t sigmoid_table(const uint16_t** table);

// The library's static device scratch on the current device (q4moe_noalloc.hip):
// its device address, resolved on first use per device, and its size.
hipError_t static_scratch(void** ptr);
size_t static_scratch_bytes();

// Resident-digits kernel for token groups of at most two (decode widths):
// true when the whole-K digits of `M_per_slot` tokens fit its LDS buffer.
bool resident_fits(int M_per_slot, int H, bool q8, bool xf32);
hipError_t launch_resident(GateUpParams p, hipStream_t stream);

// Batch kernel for any width (digits staged per K-chunk).
hipError_t launch_batch(GateUpParams p, int tokens_per_slot, hipStream_t stream);

// Chunked kernel for bf16 activations and Q4 weights with a few rows per
// slot: the column tiles (1 or 2) it would take for this call, or 0 when the
// call is outside its range; and its launch.
int chunked_tiles(const GateUpParams& p);
hipError_t launch_chunked(GateUpParams p, int nt, hipStream_t stream);

// Pick and launch the kernel for a call whose slots see at most
// `tokens_per_slot` tokens (more are processed in further token groups).
hipError_t launch_gate_up(const GateUpParams& p, int tokens_per_slot, hipStream_t stream);

// Down launch whose p.M tokens are routed pairs (one input row each) and
// whose slots are expected to see `pairs_per_slot` of them: the resident
// kernel when all p.M rows fit it, else the batch kernel sized for
// `pairs_per_slot` (more are processed in further groups).
hipError_t launch_down(const GateUpParams& p, int pairs_per_slot, hipStream_t stream);

}  // namespace q4
