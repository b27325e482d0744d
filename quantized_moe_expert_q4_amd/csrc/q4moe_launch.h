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
  int G, steps;              // resident kernel: tokens per group, K-steps per tile (set by the launcher)
};

using ResidentParams = GateUpParams;

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

// Grouped path: prep kernel (digits + routing plan) and persistent stream
// kernel.  Offsets are byte offsets into the caller's workspace.
struct StreamPlan {
  int nt = 1, g = 2, rw = 2, d = 3;
  bool vec = true;
  int nsteps = 0, rtc = 0, waves = 0;
  uint32_t tok_stride = 0, rec_bytes = 0;
  uint64_t off_xmax = 0, off_count = 0, off_offset = 0, off_vprefix = 0, off_pairs = 0, off_bad = 0,
           off_fixcnt = 0, off_fixrec = 0, off_digits = 0, workspace = 0;
};

struct StreamParams {
  const uint8_t* slots;
  uint64_t slot_stride;
  uint64_t gate_w_off, up_w_off, gate_s_off, up_s_off;
  const uint16_t* x;       // bf16 [M][H]
  const int32_t* ids;      // int32 [M][K]
  uint16_t* out;           // bf16 [M*K][I]
  float* gate_probe;       // or nullptr
  float* up_probe;         // or nullptr
  uint8_t* ws;             // workspace
  uint64_t off_xmax, off_count, off_offset, off_vprefix, off_pairs, off_bad, off_fixcnt, off_fixrec, off_digits;
  uint32_t tok_stride, rec_bytes;
  int M, K, H, I, num_slots;
  int G, rtc, nsteps, W;
};

// Resident-digits kernel for token groups of at most two (decode widths).
bool resident_fits(int M_per_slot, int H);
hipError_t launch_resident(ResidentParams p, hipStream_t stream);

StreamPlan plan_stream(int M, int K, int H, int I, int num_slots);
hipError_t launch_stream(const StreamParams& p, const StreamPlan& sp, hipStream_t stream);

}  // namespace q4
