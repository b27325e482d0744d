// Internal interface between the C ABI (q4moe_abi.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace q4 {

// Everything one launch of the gate/up kernel reads.  `ids == nullptr` is the
// single-expert call: every token routed to slot 0 with K == 1.
struct GateUpParams {
  const uint8_t* slots;      // slot 0 base (4096-aligned)
  uint64_t slot_stride;      // bytes between slots
  uint64_t gate_w_off, up_w_off, gate_s_off, up_s_off;
  const uint16_t* x;         // bf16 [M][H]
  const int32_t* ids;        // int32 [M][K] or nullptr
  uint16_t* out;             // bf16 [M*K][I]
  float* gate_probe;         // F32 [M*K][I] or nullptr
  float* up_probe;           // F32 [M*K][I] or nullptr
  int32_t* invalid_count;    // grouped: number of out-of-range ids, or nullptr
  int M, K, H, I, num_slots;
};

// Kernel shape: NT column tiles of 16 (tokens per group = 16*NT/6), RT row
// tiles of 16 per work-group (the 4 waves split K 4/RT ways), 16-byte weight
// loads when rows are 16-byte aligned.
struct LaunchPlan {
  int nt = 1;
  int rt = 4;
  bool vec = true;
};

LaunchPlan plan_launch(int M_per_slot, int I, int num_slots, int H);
hipError_t launch_gate_up(const GateUpParams& p, int num_slots, const LaunchPlan& lp, hipStream_t stream);

}  // namespace q4
