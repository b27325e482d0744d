// Internal interface of the read-only streaming kernels (q4moe_stream.hip).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace q4 {

// Two arrays of `rows` rows of `row_bytes` bytes (a multiple of 128) at
// off_a and off_b in each of num_slots slots spaced slot_stride bytes apart.
struct StreamParams {
  const uint8_t* base;
  uint64_t slot_stride;
  uint64_t off_a, off_b;
  uint32_t row_bytes;
  int rows, num_slots;
  uint32_t* sink;            // one device word, written only on a value no data gives in practice
};

// pattern 0: the gate/up kernels' row-tile access; 1: lane-linear runs.
// waves 8 or 16 per work-group, depth 1, 2 or 4 units in flight per wave.
hipError_t launch_stream_read(const StreamParams& p, int pattern, int waves, int depth, hipStream_t stream);

}  // namespace q4
