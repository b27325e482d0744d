// Read-only streaming kernels over expert slots: the weight access of the
// gate/up kernels with no arithmetic, and a linear read of the same bytes.
// A measurement aid: the rate at which a kernel with this access can pull
// bytes from HBM on the device it runs on, next to which the gate/up
// kernels' own rate is read.
//
// Both read, in every slot, two arrays of `rows` rows of `row_bytes` bytes
// (the gate and up weights of a slot) once each, in units of (16-row tile,
// 128-byte step), as the resident gate/up kernel's wide K-steps do:
//  * TILE: lane l of a wave reads 32 bytes of row 16t + l % 16 at byte
//    (l / 16) * 32 + 128 s of the row, from each array (four 16-byte loads);
//  * LINEAR: the same 2 KiB of each array per unit, read as two lane-linear
//    1 KiB runs of the tile's contiguous bytes;
//  * HALF: as TILE, but lane l's two 16-byte loads take bytes (l / 16) * 16
//    and 64 + (l / 16) * 16 of the row's 128 bytes, so that each load
//    instruction covers one whole 64-byte half of every row's 128 bytes;
//  * LINE: 8 lanes per row, so that each load instruction covers whole
//    128-byte lines: lane l's two loads take bytes 16 (l % 8) of rows
//    l / 8 and 8 + l / 8 of the tile.
// Each pattern also runs with the non-temporal load hint.
// One persistent work-group of WAVES waves per CU; work-group b takes the
// tiles [bT/NB, (b+1)T/NB) and its waves split the (tile, step) units into
// contiguous ranges, each with D units of loads in flight in a register ring.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4moe_device.h"
#include "q4moe_stream.h"

namespace q4 {

namespace {

struct Ring {
  v4u a0, a1, b0, b1;
};

template <int WAVES, int D, int PAT, int AUX>
__global__ __launch_bounds__(WAVES * 64) void stream_read_kernel(const StreamParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tpsl = (p.rows + 15) / 16;                         // tiles per slot
  const int S = (int)(p.row_bytes / 128u);                     // steps per tile
  const int T = p.num_slots * tpsl;
  const int NB = gridDim.x;
  const int v0 = (int)((int64_t)blockIdx.x * T / NB), v1 = (int)((int64_t)(blockIdx.x + 1) * T / NB);
  const int N = (v1 - v0) * S;
  const int ua = (int)((int64_t)wave * N / WAVES), ub = (int)((int64_t)(wave + 1) * N / WAVES);
  const uint32_t abytes = (uint32_t)p.rows * p.row_bytes;

  // load cursor: tile v, step s, and the two arrays' resources of v's slot
  int cv = v0 + ua / S, cs = ua - (ua / S) * S, left = ub - ua;
  __amdgpu_buffer_rsrc_t ra, rb;
  int ct = 0;
  auto seek = [&]() {
    const int e = cv / tpsl;
    ct = cv - e * tpsl;
    const uint8_t* slot = p.base + (uint64_t)e * p.slot_stride;
    ra = make_rsrc(slot + p.off_a, abytes);
    rb = make_rsrc(slot + p.off_b, abytes);
  };
  seek();
  auto issue = [&](Ring& r, uint32_t dep) {
    uint32_t off;
    if (PAT == 1) {
      off = (uint32_t)ct * 16u * p.row_bytes + (uint32_t)cs * 2048u + (uint32_t)lane * 16u;
    } else if (PAT == 3) {
      const int row = ct * 16 + (lane >> 3);
      off = (uint32_t)min(row, p.rows - 1) * p.row_bytes + (uint32_t)(lane & 7) * 16u + (uint32_t)cs * 128u;
    } else {
      const int row = ct * 16 + (lane & 15);
      off = (uint32_t)min(row, p.rows - 1) * p.row_bytes + (uint32_t)(lane >> 4) * (PAT == 2 ? 16u : 32u) +
            (uint32_t)cs * 128u;
    }
    off = (left > 0 ? off : kOffNone) + dep;                   // past the range: zeros, no access
    const uint32_t second = PAT == 1 ? 1024u : (PAT == 2 ? 64u : (PAT == 3 ? 8u * p.row_bytes : 16u));
    r.a0 = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, AUX);
    r.a1 = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(off + second), 0, AUX);
    r.b0 = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)off, 0, AUX);
    r.b1 = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(off + second), 0, AUX);
    if (left > 0) {
      --left;
      if (++cs == S) {
        cs = 0;
        ++cv;
        if (left > 0) seek();
      }
    }
  };

  Ring ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) issue(ring[d], 0u);
  uint32_t acc = 0;
  for (int u = ua; u < ub; u += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const Ring& r = ring[d];
      const v4u x = r.a0 ^ r.a1 ^ r.b0 ^ r.b1;
      const uint32_t t = x.x ^ x.y ^ x.z ^ x.w;
      // the refill's offset depends on the slot's value through an empty asm,
      // so the loads issue after the slot is read and land in its registers
      // (else the compiler double-buffers the ring and drains it at the loop's
      // back edge)
      uint32_t dep = 0u;
      asm volatile("" : "+v"(dep) : "v"(t));
      issue(ring[d], dep);
      acc ^= t;
    }
  }
  // the loads' values feed a store the compiler cannot rule out
  if (acc == 0x9E3779B9u) p.sink[0] = acc + (uint32_t)lane;
}

template <int WAVES, int D, int PAT, int AUX>
hipError_t launch_t(const StreamParams& p, hipStream_t stream) {
  int device = 0, cus = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0) cus = 256;
  const int tiles = p.num_slots * ((p.rows + 15) / 16);
  const int nb = cus < tiles ? cus : tiles;
  StreamParams q = p;
  void* args[] = {&q};
  // dynamic LDS the kernel does not use, so that one work-group runs per CU,
  // as for the gate/up kernels
  return hipLaunchKernel(reinterpret_cast<const void*>(&stream_read_kernel<WAVES, D, PAT, AUX>), dim3((unsigned)nb),
                         dim3(WAVES * 64), args, 96 * 1024, stream);
}

}  // namespace

template <int WAVES, int D, int AUX>
hipError_t launch_wda(const StreamParams& p, int pattern, hipStream_t stream) {
  if (pattern == 1) return launch_t<WAVES, D, 1, AUX>(p, stream);
  if (pattern == 2) return launch_t<WAVES, D, 2, AUX>(p, stream);
  if (pattern == 3) return launch_t<WAVES, D, 3, AUX>(p, stream);
  return launch_t<WAVES, D, 0, AUX>(p, stream);
}

// pattern bit 2: the non-temporal load hint
template <int WAVES, int D>
hipError_t launch_wd(const StreamParams& p, int pattern, hipStream_t stream) {
  return (pattern & 4) ? launch_wda<WAVES, D, kLoadNT>(p, pattern & 3, stream)
                       : launch_wda<WAVES, D, 0>(p, pattern & 3, stream);
}

hipError_t launch_stream_read(const StreamParams& p, int pattern, int waves, int depth, hipStream_t stream) {
  if (waves == 8) {
    if (depth == 1) return launch_wd<8, 1>(p, pattern, stream);
    if (depth == 2) return launch_wd<8, 2>(p, pattern, stream);
    return launch_wd<8, 4>(p, pattern, stream);
  }
  if (depth == 1) return launch_wd<16, 1>(p, pattern, stream);
  if (depth == 2) return launch_wd<16, 2>(p, pattern, stream);
  return launch_wd<16, 4>(p, pattern, stream);
}

}  // namespace q4
