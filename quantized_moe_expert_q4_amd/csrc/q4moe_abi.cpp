// C ABI of the Q4/Q8 expert library: argument validation and dispatch.
//
// Validation mirrors validateCall (page 52 of the @mlx-bun/inference 1.0.0
// diff, kernels/glm52/streamed-experts.ts) and validateRange (page 51,
// kernels/glm52/layout.ts): positive sizes, H divisible by the 8 weights of a
// packed word, input [M, H] with M >= 1, every slot field inside the slot, a
// page-aligned slot pointer.  The Q8 family takes the same rules with one
// weight per byte; its H % 8 (and, for down, I % 8) rule is this library's:
// the kernels read activations in 8-value units.  The pages' "divisible by 4" rule comes from their
// 4-rows-per-threadgroup grid and does not apply to these kernels, and the
// pages' 16 KiB page alignment is read as 4096 bytes (device allocations).
#include <stdint.h>
#include <string.h>

#include <string>

#include "q4moe.h"
#include "q4moe_launch.h"
#include "q4moe_stream.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int ok() {
  g_err.clear();
  return Q4_OK;
}

constexpr uint64_t kSlotAlign = 4096;
constexpr int64_t kMaxH = 65536;
constexpr int64_t kMaxM = 65535;
constexpr int64_t kMaxPairs = 65536;
constexpr int64_t kMaxSlots = 65535;
constexpr uint64_t kMaxWeightBytes = (1ull << 31) - 16;
constexpr size_t kWorkspaceBytes = 256;  // [0]: number of out-of-range ids

// Call formats: int8 weights (else packed nibbles) and f32 activations and
// outputs (else bf16), or'ed together.
constexpr unsigned kQ8 = 1u, kF32 = 2u;

// Bytes of one weight row of K weights: packed nibbles (Q4, two per byte) or
// int8 (Q8, one per byte), the weightsPerByte of the two families on page 52.
uint64_t weight_row_bytes(bool q8, int64_t K) { return q8 ? (uint64_t)K : (uint64_t)(K / 2); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_range(uint64_t offset, uint64_t length, uint64_t slot_bytes, const char* label) {
  if (offset > slot_bytes || length > slot_bytes - offset)
    return fail(Q4_ERR_RANGE, std::string(label) + " exceeds the canonical expert slot");
  return Q4_OK;
}

int check_dims(unsigned fmt, int64_t M, int64_t H, int64_t I) {
  if (H <= 0) return fail(Q4_ERR_INVALID_ARGUMENT, "hidden size must be a positive integer");
  if (I <= 0) return fail(Q4_ERR_INVALID_ARGUMENT, "intermediate size must be a positive integer");
  if (H % 8 != 0)
    return fail(Q4_ERR_INVALID_ARGUMENT, std::string((fmt & kQ8) ? "Q8" : "Q4") + " expert dimensions must be divisible by 8");
  if (M < 1)
    return fail(Q4_ERR_INVALID_ARGUMENT, std::string((fmt & kQ8) ? "Q8" : "Q4") + " expert gate/up requires input [M,H] with M >= 1");
  if (H > kMaxH) return fail(Q4_ERR_UNSUPPORTED, "hidden size above 65536 is not supported");
  if (M > kMaxM) return fail(Q4_ERR_UNSUPPORTED, "more than 65535 tokens per call is not supported");
  if ((uint64_t)I * weight_row_bytes((fmt & kQ8) != 0, H) > kMaxWeightBytes)
    return fail(Q4_ERR_UNSUPPORTED, "a projection above 2^31 - 16 bytes is not supported");
  return Q4_OK;
}

int check_layout(unsigned fmt, const q4_slot_layout* L, int64_t H, int64_t I) {
  if (!L) return fail(Q4_ERR_INVALID_ARGUMENT, "slot layout must not be null");
  if (L->slot_bytes == 0) return fail(Q4_ERR_INVALID_ARGUMENT, "expert slot bytes must be a positive integer");
  const uint64_t wb = (uint64_t)I * weight_row_bytes((fmt & kQ8) != 0, H);
  int rc;
  if (L->down_weight_offset != Q4_OFFSET_ABSENT &&
      (rc = check_range(L->down_weight_offset, wb, L->slot_bytes, "down weights")))
    return rc;
  if ((rc = check_range(L->gate_weight_offset, wb, L->slot_bytes, "gate weights"))) return rc;
  if ((rc = check_range(L->up_weight_offset, wb, L->slot_bytes, "up weights"))) return rc;
  if (L->down_scale_offset != Q4_OFFSET_ABSENT &&
      (rc = check_range(L->down_scale_offset, 4 * (uint64_t)H, L->slot_bytes, "down scales")))
    return rc;
  if ((rc = check_range(L->gate_scale_offset, 4 * (uint64_t)I, L->slot_bytes, "gate scales"))) return rc;
  if ((rc = check_range(L->up_scale_offset, 4 * (uint64_t)I, L->slot_bytes, "up scales"))) return rc;
  if (L->gate_weight_offset % 16 || L->up_weight_offset % 16)
    return fail(Q4_ERR_ALIGNMENT, "gate and up weight offsets must be multiples of 16 bytes");
  if (L->gate_scale_offset % 4 || L->up_scale_offset % 4)
    return fail(Q4_ERR_ALIGNMENT, "gate and up scale offsets must be multiples of 4 bytes");
  return Q4_OK;
}

// Extra rules of a call that reads the down fields (DOWN_SOURCE and
// validateCall, page 52): both dimensions divisible by 8, the down fields
// present and aligned for the kernels' loads.
int check_down_layout(unsigned fmt, const q4_slot_layout* L, int64_t I) {
  if (I % 8 != 0)
    return fail(Q4_ERR_INVALID_ARGUMENT, std::string((fmt & kQ8) ? "Q8" : "Q4") + " expert dimensions must be divisible by 8");
  if (I > kMaxH) return fail(Q4_ERR_UNSUPPORTED, "intermediate size above 65536 is not supported by the down projection");
  if (L->down_weight_offset == Q4_OFFSET_ABSENT || L->down_scale_offset == Q4_OFFSET_ABSENT)
    return fail(Q4_ERR_INVALID_ARGUMENT, "the down projection needs down weight and scale offsets");
  if (L->down_weight_offset % 16) return fail(Q4_ERR_ALIGNMENT, "down weight offset must be a multiple of 16 bytes");
  if (L->down_scale_offset % 4) return fail(Q4_ERR_ALIGNMENT, "down scale offset must be a multiple of 4 bytes");
  return Q4_OK;
}

int check_io(unsigned fmt, const void* x, const void* out, const void* gate_probe, const void* up_probe) {
  if (!x) return fail(Q4_ERR_INVALID_ARGUMENT, "input x must be a non-null device pointer");
  if (!out) return fail(Q4_ERR_INVALID_ARGUMENT, "output must be a non-null device pointer");
  if (!aligned(x, 16)) return fail(Q4_ERR_ALIGNMENT, "input x must be 16-byte aligned");
  if ((fmt & kF32) ? !aligned(out, 4) : !aligned(out, 2))
    return fail(Q4_ERR_ALIGNMENT, (fmt & kF32) ? "output must be 4-byte aligned" : "output must be 2-byte aligned");
  if ((gate_probe && !aligned(gate_probe, 4)) || (up_probe && !aligned(up_probe, 4)))
    return fail(Q4_ERR_ALIGNMENT, "gate/up probes must be 4-byte aligned");
  return Q4_OK;
}

int check_single(unsigned fmt, const void* slot, const q4_slot_layout* layout, const void* x, int64_t M, int64_t H,
                 int64_t I, const void* out, const void* gp, const void* up) {
  int rc;
  if ((rc = check_dims(fmt, M, H, I))) return rc;
  if (!slot) return fail(Q4_ERR_INVALID_ARGUMENT, "expert slot pointer must be a non-null device pointer");
  if (!aligned(slot, kSlotAlign))
    return fail(Q4_ERR_ALIGNMENT, "expert slot pointer must be page-aligned (4096 bytes) for direct device access");
  if ((rc = check_layout(fmt, layout, H, I))) return rc;
  if ((rc = check_io(fmt, x, out, gp, up))) return rc;
  return ok();
}

int check_grouped(unsigned fmt, const void* base, uint64_t stride, int64_t num_slots, const q4_slot_layout* layout,
                  const void* x, int64_t M, const int32_t* ids, int64_t K, int64_t H, int64_t I,
                  const void* out, const void* gp, const void* up, const void* ws, size_t ws_bytes) {
  int rc;
  if ((rc = check_dims(fmt, M, H, I))) return rc;
  if (K < 1) return fail(Q4_ERR_INVALID_ARGUMENT, "top-k must be a positive integer");
  if (num_slots < 1) return fail(Q4_ERR_INVALID_ARGUMENT, "number of slots must be a positive integer");
  if (num_slots > kMaxSlots) return fail(Q4_ERR_UNSUPPORTED, "more than 65535 slots is not supported");
  if (K > kMaxPairs || M * K > kMaxPairs)
    return fail(Q4_ERR_UNSUPPORTED, "more than 65536 routed pairs per call is not supported");
  if (!base) return fail(Q4_ERR_INVALID_ARGUMENT, "expert slot pointer must be a non-null device pointer");
  if (!aligned(base, kSlotAlign))
    return fail(Q4_ERR_ALIGNMENT, "expert slot pointer must be page-aligned (4096 bytes) for direct device access");
  if (stride % kSlotAlign) return fail(Q4_ERR_ALIGNMENT, "slot stride must be a multiple of 4096 bytes");
  if ((rc = check_layout(fmt, layout, H, I))) return rc;
  if (stride < layout->slot_bytes) return fail(Q4_ERR_RANGE, "slot stride is shorter than the slot");
  if ((uint64_t)(num_slots - 1) > (UINT64_MAX - layout->slot_bytes) / stride)
    return fail(Q4_ERR_RANGE, "slot array exceeds the address space");
  if (!ids) return fail(Q4_ERR_INVALID_ARGUMENT, "slot ids must be a non-null device pointer");
  if (!aligned(ids, 4)) return fail(Q4_ERR_ALIGNMENT, "slot ids must be 4-byte aligned");
  if ((rc = check_io(fmt, x, out, gp, up))) return rc;
  if (!ws) return fail(Q4_ERR_WORKSPACE, "workspace must be a non-null device pointer");
  if (!aligned(ws, 256)) return fail(Q4_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (ws_bytes < q4_grouped_workspace_bytes(M, K, num_slots))
    return fail(Q4_ERR_WORKSPACE, "workspace is smaller than q4_grouped_workspace_bytes()");
  return ok();
}

q4::GateUpParams make_params(unsigned fmt, const void* base, uint64_t stride, int64_t num_slots, const q4_slot_layout* layout,
                             const void* x, int64_t M, const int32_t* ids, int64_t K, int64_t H, int64_t I,
                             void* out, float* gp, float* up, void* ws) {
  q4::GateUpParams p{};
  p.slots = static_cast<const uint8_t*>(base);
  p.slot_stride = stride;
  p.gate_w_off = layout->gate_weight_offset;
  p.up_w_off = layout->up_weight_offset;
  p.gate_s_off = layout->gate_scale_offset;
  p.up_s_off = layout->up_scale_offset;
  p.x = static_cast<const uint16_t*>(x);
  p.ids = ids;
  p.out = static_cast<uint16_t*>(out);
  p.gate_probe = gp;
  p.up_probe = up;
  p.invalid_count = static_cast<int32_t*>(ws);
  p.M = (int)M;
  p.K = (int)K;
  p.H = (int)H;
  p.I = (int)I;
  p.num_slots = (int)num_slots;
  p.q8 = (fmt & kQ8) ? 1 : 0;
  p.xf32 = (fmt & kF32) ? 1 : 0;
  return p;
}

// The down projection as a kernel launch: x = mid (one row of I per token),
// output rows H, the down fields in the gate/scale slots of the parameters.
q4::GateUpParams down_params(q4::GateUpParams p, const q4_slot_layout* layout, int64_t H, int64_t I) {
  p.gate_w_off = p.up_w_off = layout->down_weight_offset;
  p.gate_s_off = p.up_s_off = layout->down_scale_offset;
  p.H = (int)I;
  p.I = (int)H;
  p.up_probe = nullptr;
  p.down = 1;
  return p;
}

// pairs_per_slot > 0: a down launch whose slots see about that many of its
// p.M routed pairs (the caller's token count: top-k ids are distinct per token)
int launch(const q4::GateUpParams& p, q4_stream_t stream, int pairs_per_slot = 0) {
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = p.down ? q4::launch_down(p, pairs_per_slot > 0 ? pairs_per_slot : p.M, s)
                              : q4::launch_gate_up(p, p.M, s);
  if (e != hipSuccess) return fail(Q4_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ok();
}

int run_single(unsigned fmt, const void* slot, const q4_slot_layout* layout, const void* x, int64_t M, int64_t H, int64_t I,
               void* out, float* gp, float* up, q4_stream_t stream) {
  const int rc = check_single(fmt, slot, layout, x, M, H, I, out, gp, up);
  if (rc) return rc;
  return launch(make_params(fmt, slot, layout->slot_bytes, 1, layout, x, M, nullptr, 1, H, I, out, gp, up, nullptr),
                stream);
}

int run_grouped(unsigned fmt, const void* base, uint64_t stride, int64_t num_slots, const q4_slot_layout* layout,
                const void* x, int64_t M, const int32_t* ids, int64_t K, int64_t H, int64_t I, void* out,
                float* gp, float* up, void* ws, size_t ws_bytes, q4_stream_t stream) {
  const int rc = check_grouped(fmt, base, stride, num_slots, layout, x, M, ids, K, H, I, out, gp, up, ws, ws_bytes);
  if (rc) return rc;
  return launch(make_params(fmt, base, stride, num_slots, layout, x, M, ids, K, H, I, out, gp, up, ws), stream);
}

int check_down_single(unsigned fmt, const void* slot, const q4_slot_layout* layout, const void* mid, int64_t M, int64_t H,
                      int64_t I, const void* out, const void* probe) {
  int rc;
  if ((rc = check_single(fmt, slot, layout, mid, M, H, I, out, probe, nullptr))) return rc;
  if ((rc = check_down_layout(fmt, layout, I))) return rc;
  return ok();
}

int check_down_grouped(unsigned fmt, const void* base, uint64_t stride, int64_t num_slots, const q4_slot_layout* layout,
                       const void* mid, int64_t M, const int32_t* ids, int64_t K, int64_t H, int64_t I,
                       const void* out, const void* probe, const void* ws, size_t ws_bytes) {
  int rc;
  if ((rc = check_grouped(fmt, base, stride, num_slots, layout, mid, M, ids, K, H, I, out, probe, nullptr, ws, ws_bytes)))
    return rc;
  if ((rc = check_down_layout(fmt, layout, I))) return rc;
  if (M * K > kMaxM) return fail(Q4_ERR_UNSUPPORTED, "more than 65535 routed pairs per down call is not supported");
  return ok();
}

int run_down_single(unsigned fmt, const void* slot, const q4_slot_layout* layout, const void* mid, int64_t M, int64_t H,
                    int64_t I, void* out, float* probe, q4_stream_t stream) {
  const int rc = check_down_single(fmt, slot, layout, mid, M, H, I, out, probe);
  if (rc) return rc;
  return launch(down_params(make_params(fmt, slot, layout->slot_bytes, 1, layout, mid, M, nullptr, 1, H, I, out, probe,
                                        nullptr, nullptr),
                            layout, H, I),
                stream);
}

// Pair p = t*K + j reads its own input row mid[p] against slot ids[p]: the
// launch sees M*K tokens routed one each (K = 1) through the same id array.
int run_down_grouped(unsigned fmt, const void* base, uint64_t stride, int64_t num_slots, const q4_slot_layout* layout,
                     const void* mid, int64_t M, const int32_t* ids, int64_t K, int64_t H, int64_t I, void* out,
                     float* probe, void* ws, size_t ws_bytes, q4_stream_t stream) {
  const int rc = check_down_grouped(fmt, base, stride, num_slots, layout, mid, M, ids, K, H, I, out, probe, ws, ws_bytes);
  if (rc) return rc;
  return launch(down_params(make_params(fmt, base, stride, num_slots, layout, mid, M * K, ids, 1, H, I, out, probe,
                                        nullptr, ws),
                            layout, H, I),
                stream, (int)M);
}

}  // namespace

extern "C" {

int q4_expert_gate_up(const void* slot, const q4_slot_layout* layout, const void* x_bf16, int64_t M, int64_t H,
                      int64_t I, void* out_bf16, q4_stream_t stream) {
  return run_single(0u, slot, layout, x_bf16, M, H, I, out_bf16, nullptr, nullptr, stream);
}

int q4_expert_gate_up_probe(const void* slot, const q4_slot_layout* layout, const void* x_bf16, int64_t M,
                            int64_t H, int64_t I, void* out_bf16, float* gate_f32, float* up_f32,
                            q4_stream_t stream) {
  return run_single(0u, slot, layout, x_bf16, M, H, I, out_bf16, gate_f32, up_f32, stream);
}

size_t q4_grouped_workspace_bytes(int64_t M, int64_t K, int64_t num_slots) {
  if (M < 1 || K < 1 || num_slots < 1 || M > kMaxM || K > kMaxPairs || num_slots > kMaxSlots || M * K > kMaxPairs)
    return 0;
  return kWorkspaceBytes;
}

int q4_expert_gate_up_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                              const q4_slot_layout* layout, const void* x_bf16, int64_t M,
                              const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_bf16,
                              void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  return run_grouped(0u, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, out_bf16, nullptr,
                     nullptr, workspace, workspace_bytes, stream);
}

int q4_expert_gate_up_grouped_noalloc(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                                      const q4_slot_layout* layout, const void* x_bf16, int64_t M,
                                      const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_bf16,
                                      int32_t* invalid_count, q4_stream_t stream) {
  // the grouped call's workspace, here the library's static scratch
  const size_t need = q4_grouped_workspace_bytes(M, K, num_slots);
  if (need > q4::static_scratch_bytes())
    return fail(Q4_ERR_UNSUPPORTED, "the call needs " + std::to_string(need) +
                                        " bytes of workspace, more than the library's static scratch of " +
                                        std::to_string(q4::static_scratch_bytes()));
  if (invalid_count && !aligned(invalid_count, 4))
    return fail(Q4_ERR_ALIGNMENT, "invalid_count must be 4-byte aligned");
  // host-side checks first: a rejected call touches no device state
  int rc = check_grouped(0u, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, out_bf16,
                         nullptr, nullptr, reinterpret_cast<void*>(uintptr_t(256)), q4::static_scratch_bytes());
  if (rc) return rc;
  void* ws = nullptr;
  hipError_t e = q4::static_scratch(&ws);
  if (e != hipSuccess)
    return fail(Q4_ERR_HIP, std::string("static scratch unavailable: ") + hipGetErrorString(e));
  rc = run_grouped(0u, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, out_bf16, nullptr,
                   nullptr, ws, q4::static_scratch_bytes(), stream);
  if (rc || !invalid_count) return rc;
  e = hipMemcpyAsync(invalid_count, ws, sizeof(int32_t), hipMemcpyDeviceToDevice,
                     reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(Q4_ERR_HIP, std::string("invalid-id count copy failed: ") + hipGetErrorString(e));
  return ok();
}

int q4_expert_gate_up_grouped_probe(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                                    const q4_slot_layout* layout, const void* x_bf16, int64_t M,
                                    const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_bf16,
                                    float* gate_f32, float* up_f32, void* workspace, size_t workspace_bytes,
                                    q4_stream_t stream) {
  return run_grouped(0u, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, out_bf16, gate_f32,
                     up_f32, workspace, workspace_bytes, stream);
}

int q4_validate_gate_up(const void* slot, const q4_slot_layout* layout, const void* x_bf16, int64_t M, int64_t H,
                        int64_t I, const void* out_bf16) {
  return check_single(0u, slot, layout, x_bf16, M, H, I, out_bf16, nullptr, nullptr);
}

int q4_validate_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                        const q4_slot_layout* layout, const void* x_bf16, int64_t M, const int32_t* slot_ids,
                        int64_t K, int64_t H, int64_t I, const void* out_bf16, const void* workspace,
                        size_t workspace_bytes) {
  return check_grouped(0u, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, out_bf16, nullptr,
                       nullptr, workspace, workspace_bytes);
}

int q4_expert_down(const void* slot, const q4_slot_layout* layout, const void* mid_bf16, int64_t M, int64_t H,
                   int64_t I, void* out_bf16, q4_stream_t stream) {
  return run_down_single(0u, slot, layout, mid_bf16, M, H, I, out_bf16, nullptr, stream);
}

int q4_expert_down_probe(const void* slot, const q4_slot_layout* layout, const void* mid_bf16, int64_t M, int64_t H,
                         int64_t I, void* out_bf16, float* down_f32, q4_stream_t stream) {
  return run_down_single(0u, slot, layout, mid_bf16, M, H, I, out_bf16, down_f32, stream);
}

int q4_expert_down_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                           const q4_slot_layout* layout, const void* mid_bf16, int64_t M, const int32_t* slot_ids,
                           int64_t K, int64_t H, int64_t I, void* out_bf16, void* workspace, size_t workspace_bytes,
                           q4_stream_t stream) {
  return run_down_grouped(0u, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                          nullptr, workspace, workspace_bytes, stream);
}

int q4_expert_down_grouped_probe(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                                 const q4_slot_layout* layout, const void* mid_bf16, int64_t M,
                                 const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_bf16,
                                 float* down_f32, void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  return run_down_grouped(0u, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                          down_f32, workspace, workspace_bytes, stream);
}

int q4_expert_forward(const void* slot, const q4_slot_layout* layout, const void* x_bf16, int64_t M, int64_t H,
                      int64_t I, void* mid_bf16, void* out_bf16, q4_stream_t stream) {
  int rc;
  if ((rc = check_single(0u, slot, layout, x_bf16, M, H, I, mid_bf16, nullptr, nullptr))) return rc;
  if ((rc = check_down_single(0u, slot, layout, mid_bf16, M, H, I, out_bf16, nullptr))) return rc;
  if ((rc = run_single(0u, slot, layout, x_bf16, M, H, I, mid_bf16, nullptr, nullptr, stream))) return rc;
  return run_down_single(0u, slot, layout, mid_bf16, M, H, I, out_bf16, nullptr, stream);
}

int q4_expert_forward_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                              const q4_slot_layout* layout, const void* x_bf16, int64_t M, const int32_t* slot_ids,
                              int64_t K, int64_t H, int64_t I, void* mid_bf16, void* out_bf16, void* workspace,
                              size_t workspace_bytes, q4_stream_t stream) {
  int rc;
  if ((rc = check_grouped(0u, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, mid_bf16,
                          nullptr, nullptr, workspace, workspace_bytes)))
    return rc;
  if ((rc = check_down_grouped(0u, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                               nullptr, workspace, workspace_bytes)))
    return rc;
  if ((rc = run_grouped(0u, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, mid_bf16, nullptr,
                        nullptr, workspace, workspace_bytes, stream)))
    return rc;
  return run_down_grouped(0u, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                          nullptr, workspace, workspace_bytes, stream);
}

int q4_validate_down(const void* slot, const q4_slot_layout* layout, const void* mid_bf16, int64_t M, int64_t H,
                     int64_t I, const void* out_bf16) {
  return check_down_single(0u, slot, layout, mid_bf16, M, H, I, out_bf16, nullptr);
}

int q4_validate_down_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                             const q4_slot_layout* layout, const void* mid_bf16, int64_t M, const int32_t* slot_ids,
                             int64_t K, int64_t H, int64_t I, const void* out_bf16, const void* workspace,
                             size_t workspace_bytes) {
  return check_down_grouped(0u, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                            nullptr, workspace, workspace_bytes);
}


// ---- the Q8 family (signed int8 weights, page 52 Q8_GATE_UP_SOURCE / Q8_DOWN_SOURCE) ----

int q8_expert_gate_up(const void* slot, const q4_slot_layout* layout, const void* x_bf16, int64_t M, int64_t H,
                      int64_t I, void* out_bf16, q4_stream_t stream) {
  return run_single(kQ8, slot, layout, x_bf16, M, H, I, out_bf16, nullptr, nullptr, stream);
}

int q8_expert_gate_up_probe(const void* slot, const q4_slot_layout* layout, const void* x_bf16, int64_t M,
                            int64_t H, int64_t I, void* out_bf16, float* gate_f32, float* up_f32,
                            q4_stream_t stream) {
  return run_single(kQ8, slot, layout, x_bf16, M, H, I, out_bf16, gate_f32, up_f32, stream);
}

int q8_expert_gate_up_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                              const q4_slot_layout* layout, const void* x_bf16, int64_t M,
                              const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_bf16,
                              void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  return run_grouped(kQ8, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, out_bf16, nullptr,
                     nullptr, workspace, workspace_bytes, stream);
}

int q8_expert_gate_up_grouped_probe(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                                    const q4_slot_layout* layout, const void* x_bf16, int64_t M,
                                    const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_bf16,
                                    float* gate_f32, float* up_f32, void* workspace, size_t workspace_bytes,
                                    q4_stream_t stream) {
  return run_grouped(kQ8, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, out_bf16, gate_f32,
                     up_f32, workspace, workspace_bytes, stream);
}

int q8_validate_gate_up(const void* slot, const q4_slot_layout* layout, const void* x_bf16, int64_t M, int64_t H,
                        int64_t I, const void* out_bf16) {
  return check_single(kQ8, slot, layout, x_bf16, M, H, I, out_bf16, nullptr, nullptr);
}

int q8_validate_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                        const q4_slot_layout* layout, const void* x_bf16, int64_t M, const int32_t* slot_ids,
                        int64_t K, int64_t H, int64_t I, const void* out_bf16, const void* workspace,
                        size_t workspace_bytes) {
  return check_grouped(kQ8, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, out_bf16, nullptr,
                       nullptr, workspace, workspace_bytes);
}

int q8_expert_down(const void* slot, const q4_slot_layout* layout, const void* mid_bf16, int64_t M, int64_t H,
                   int64_t I, void* out_bf16, q4_stream_t stream) {
  return run_down_single(kQ8, slot, layout, mid_bf16, M, H, I, out_bf16, nullptr, stream);
}

int q8_expert_down_probe(const void* slot, const q4_slot_layout* layout, const void* mid_bf16, int64_t M, int64_t H,
                         int64_t I, void* out_bf16, float* down_f32, q4_stream_t stream) {
  return run_down_single(kQ8, slot, layout, mid_bf16, M, H, I, out_bf16, down_f32, stream);
}

int q8_expert_down_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                           const q4_slot_layout* layout, const void* mid_bf16, int64_t M, const int32_t* slot_ids,
                           int64_t K, int64_t H, int64_t I, void* out_bf16, void* workspace, size_t workspace_bytes,
                           q4_stream_t stream) {
  return run_down_grouped(kQ8, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                          nullptr, workspace, workspace_bytes, stream);
}

int q8_expert_down_grouped_probe(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                                 const q4_slot_layout* layout, const void* mid_bf16, int64_t M,
                                 const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_bf16,
                                 float* down_f32, void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  return run_down_grouped(kQ8, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                          down_f32, workspace, workspace_bytes, stream);
}

int q8_expert_forward(const void* slot, const q4_slot_layout* layout, const void* x_bf16, int64_t M, int64_t H,
                      int64_t I, void* mid_bf16, void* out_bf16, q4_stream_t stream) {
  int rc;
  if ((rc = check_single(kQ8, slot, layout, x_bf16, M, H, I, mid_bf16, nullptr, nullptr))) return rc;
  if ((rc = check_down_single(kQ8, slot, layout, mid_bf16, M, H, I, out_bf16, nullptr))) return rc;
  if ((rc = run_single(kQ8, slot, layout, x_bf16, M, H, I, mid_bf16, nullptr, nullptr, stream))) return rc;
  return run_down_single(kQ8, slot, layout, mid_bf16, M, H, I, out_bf16, nullptr, stream);
}

int q8_expert_forward_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                              const q4_slot_layout* layout, const void* x_bf16, int64_t M, const int32_t* slot_ids,
                              int64_t K, int64_t H, int64_t I, void* mid_bf16, void* out_bf16, void* workspace,
                              size_t workspace_bytes, q4_stream_t stream) {
  int rc;
  if ((rc = check_grouped(kQ8, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, mid_bf16,
                          nullptr, nullptr, workspace, workspace_bytes)))
    return rc;
  if ((rc = check_down_grouped(kQ8, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                               nullptr, workspace, workspace_bytes)))
    return rc;
  if ((rc = run_grouped(kQ8, slots_base, slot_stride, num_slots, layout, x_bf16, M, slot_ids, K, H, I, mid_bf16, nullptr,
                        nullptr, workspace, workspace_bytes, stream)))
    return rc;
  return run_down_grouped(kQ8, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                          nullptr, workspace, workspace_bytes, stream);
}

int q8_validate_down(const void* slot, const q4_slot_layout* layout, const void* mid_bf16, int64_t M, int64_t H,
                     int64_t I, const void* out_bf16) {
  return check_down_single(kQ8, slot, layout, mid_bf16, M, H, I, out_bf16, nullptr);
}

int q8_validate_down_grouped(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                             const q4_slot_layout* layout, const void* mid_bf16, int64_t M, const int32_t* slot_ids,
                             int64_t K, int64_t H, int64_t I, const void* out_bf16, const void* workspace,
                             size_t workspace_bytes) {
  return check_down_grouped(kQ8, slots_base, slot_stride, num_slots, layout, mid_bf16, M, slot_ids, K, H, I, out_bf16,
                            nullptr, workspace, workspace_bytes);
}


// ---- f32 activations and outputs (page 52: validateCall accepts float32 input, execute returns the input's dtype) ----

int q4_expert_gate_up_f32(const void* slot, const q4_slot_layout* layout, const void* x_f32, int64_t M, int64_t H,
                      int64_t I, void* out_f32, q4_stream_t stream) {
  return run_single(kF32, slot, layout, x_f32, M, H, I, out_f32, nullptr, nullptr, stream);
}

int q4_expert_gate_up_probe_f32(const void* slot, const q4_slot_layout* layout, const void* x_f32, int64_t M,
                            int64_t H, int64_t I, void* out_f32, float* gate_f32, float* up_f32,
                            q4_stream_t stream) {
  return run_single(kF32, slot, layout, x_f32, M, H, I, out_f32, gate_f32, up_f32, stream);
}

int q4_expert_gate_up_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                              const q4_slot_layout* layout, const void* x_f32, int64_t M,
                              const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_f32,
                              void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  return run_grouped(kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, out_f32, nullptr,
                     nullptr, workspace, workspace_bytes, stream);
}

int q4_expert_gate_up_grouped_probe_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                                    const q4_slot_layout* layout, const void* x_f32, int64_t M,
                                    const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_f32,
                                    float* gate_f32, float* up_f32, void* workspace, size_t workspace_bytes,
                                    q4_stream_t stream) {
  return run_grouped(kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, out_f32, gate_f32,
                     up_f32, workspace, workspace_bytes, stream);
}

int q4_validate_gate_up_f32(const void* slot, const q4_slot_layout* layout, const void* x_f32, int64_t M, int64_t H,
                        int64_t I, const void* out_f32) {
  return check_single(kF32, slot, layout, x_f32, M, H, I, out_f32, nullptr, nullptr);
}

int q4_validate_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                        const q4_slot_layout* layout, const void* x_f32, int64_t M, const int32_t* slot_ids,
                        int64_t K, int64_t H, int64_t I, const void* out_f32, const void* workspace,
                        size_t workspace_bytes) {
  return check_grouped(kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, out_f32, nullptr,
                       nullptr, workspace, workspace_bytes);
}

int q4_expert_down_f32(const void* slot, const q4_slot_layout* layout, const void* mid_f32, int64_t M, int64_t H,
                   int64_t I, void* out_f32, q4_stream_t stream) {
  return run_down_single(kF32, slot, layout, mid_f32, M, H, I, out_f32, nullptr, stream);
}

int q4_expert_down_probe_f32(const void* slot, const q4_slot_layout* layout, const void* mid_f32, int64_t M, int64_t H,
                         int64_t I, void* out_f32, float* down_f32, q4_stream_t stream) {
  return run_down_single(kF32, slot, layout, mid_f32, M, H, I, out_f32, down_f32, stream);
}

int q4_expert_down_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                           const q4_slot_layout* layout, const void* mid_f32, int64_t M, const int32_t* slot_ids,
                           int64_t K, int64_t H, int64_t I, void* out_f32, void* workspace, size_t workspace_bytes,
                           q4_stream_t stream) {
  return run_down_grouped(kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                          nullptr, workspace, workspace_bytes, stream);
}

int q4_expert_down_grouped_probe_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                                 const q4_slot_layout* layout, const void* mid_f32, int64_t M,
                                 const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_f32,
                                 float* down_f32, void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  return run_down_grouped(kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                          down_f32, workspace, workspace_bytes, stream);
}

int q4_expert_forward_f32(const void* slot, const q4_slot_layout* layout, const void* x_f32, int64_t M, int64_t H,
                      int64_t I, void* mid_f32, void* out_f32, q4_stream_t stream) {
  int rc;
  if ((rc = check_single(kF32, slot, layout, x_f32, M, H, I, mid_f32, nullptr, nullptr))) return rc;
  if ((rc = check_down_single(kF32, slot, layout, mid_f32, M, H, I, out_f32, nullptr))) return rc;
  if ((rc = run_single(kF32, slot, layout, x_f32, M, H, I, mid_f32, nullptr, nullptr, stream))) return rc;
  return run_down_single(kF32, slot, layout, mid_f32, M, H, I, out_f32, nullptr, stream);
}

int q4_expert_forward_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                              const q4_slot_layout* layout, const void* x_f32, int64_t M, const int32_t* slot_ids,
                              int64_t K, int64_t H, int64_t I, void* mid_f32, void* out_f32, void* workspace,
                              size_t workspace_bytes, q4_stream_t stream) {
  int rc;
  if ((rc = check_grouped(kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, mid_f32,
                          nullptr, nullptr, workspace, workspace_bytes)))
    return rc;
  if ((rc = check_down_grouped(kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                               nullptr, workspace, workspace_bytes)))
    return rc;
  if ((rc = run_grouped(kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, mid_f32, nullptr,
                        nullptr, workspace, workspace_bytes, stream)))
    return rc;
  return run_down_grouped(kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                          nullptr, workspace, workspace_bytes, stream);
}

int q4_validate_down_f32(const void* slot, const q4_slot_layout* layout, const void* mid_f32, int64_t M, int64_t H,
                     int64_t I, const void* out_f32) {
  return check_down_single(kF32, slot, layout, mid_f32, M, H, I, out_f32, nullptr);
}

int q4_validate_down_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                             const q4_slot_layout* layout, const void* mid_f32, int64_t M, const int32_t* slot_ids,
                             int64_t K, int64_t H, int64_t I, const void* out_f32, const void* workspace,
                             size_t workspace_bytes) {
  return check_down_grouped(kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                            nullptr, workspace, workspace_bytes);
}

int q8_expert_gate_up_f32(const void* slot, const q4_slot_layout* layout, const void* x_f32, int64_t M, int64_t H,
                      int64_t I, void* out_f32, q4_stream_t stream) {
  return run_single(kQ8 | kF32, slot, layout, x_f32, M, H, I, out_f32, nullptr, nullptr, stream);
}

int q8_expert_gate_up_probe_f32(const void* slot, const q4_slot_layout* layout, const void* x_f32, int64_t M,
                            int64_t H, int64_t I, void* out_f32, float* gate_f32, float* up_f32,
                            q4_stream_t stream) {
  return run_single(kQ8 | kF32, slot, layout, x_f32, M, H, I, out_f32, gate_f32, up_f32, stream);
}

int q8_expert_gate_up_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                              const q4_slot_layout* layout, const void* x_f32, int64_t M,
                              const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_f32,
                              void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  return run_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, out_f32, nullptr,
                     nullptr, workspace, workspace_bytes, stream);
}

int q8_expert_gate_up_grouped_probe_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                                    const q4_slot_layout* layout, const void* x_f32, int64_t M,
                                    const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_f32,
                                    float* gate_f32, float* up_f32, void* workspace, size_t workspace_bytes,
                                    q4_stream_t stream) {
  return run_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, out_f32, gate_f32,
                     up_f32, workspace, workspace_bytes, stream);
}

int q8_validate_gate_up_f32(const void* slot, const q4_slot_layout* layout, const void* x_f32, int64_t M, int64_t H,
                        int64_t I, const void* out_f32) {
  return check_single(kQ8 | kF32, slot, layout, x_f32, M, H, I, out_f32, nullptr, nullptr);
}

int q8_validate_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                        const q4_slot_layout* layout, const void* x_f32, int64_t M, const int32_t* slot_ids,
                        int64_t K, int64_t H, int64_t I, const void* out_f32, const void* workspace,
                        size_t workspace_bytes) {
  return check_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, out_f32, nullptr,
                       nullptr, workspace, workspace_bytes);
}

int q8_expert_down_f32(const void* slot, const q4_slot_layout* layout, const void* mid_f32, int64_t M, int64_t H,
                   int64_t I, void* out_f32, q4_stream_t stream) {
  return run_down_single(kQ8 | kF32, slot, layout, mid_f32, M, H, I, out_f32, nullptr, stream);
}

int q8_expert_down_probe_f32(const void* slot, const q4_slot_layout* layout, const void* mid_f32, int64_t M, int64_t H,
                         int64_t I, void* out_f32, float* down_f32, q4_stream_t stream) {
  return run_down_single(kQ8 | kF32, slot, layout, mid_f32, M, H, I, out_f32, down_f32, stream);
}

int q8_expert_down_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                           const q4_slot_layout* layout, const void* mid_f32, int64_t M, const int32_t* slot_ids,
                           int64_t K, int64_t H, int64_t I, void* out_f32, void* workspace, size_t workspace_bytes,
                           q4_stream_t stream) {
  return run_down_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                          nullptr, workspace, workspace_bytes, stream);
}

int q8_expert_down_grouped_probe_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                                 const q4_slot_layout* layout, const void* mid_f32, int64_t M,
                                 const int32_t* slot_ids, int64_t K, int64_t H, int64_t I, void* out_f32,
                                 float* down_f32, void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  return run_down_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                          down_f32, workspace, workspace_bytes, stream);
}

int q8_expert_forward_f32(const void* slot, const q4_slot_layout* layout, const void* x_f32, int64_t M, int64_t H,
                      int64_t I, void* mid_f32, void* out_f32, q4_stream_t stream) {
  int rc;
  if ((rc = check_single(kQ8 | kF32, slot, layout, x_f32, M, H, I, mid_f32, nullptr, nullptr))) return rc;
  if ((rc = check_down_single(kQ8 | kF32, slot, layout, mid_f32, M, H, I, out_f32, nullptr))) return rc;
  if ((rc = run_single(kQ8 | kF32, slot, layout, x_f32, M, H, I, mid_f32, nullptr, nullptr, stream))) return rc;
  return run_down_single(kQ8 | kF32, slot, layout, mid_f32, M, H, I, out_f32, nullptr, stream);
}

int q8_expert_forward_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                              const q4_slot_layout* layout, const void* x_f32, int64_t M, const int32_t* slot_ids,
                              int64_t K, int64_t H, int64_t I, void* mid_f32, void* out_f32, void* workspace,
                              size_t workspace_bytes, q4_stream_t stream) {
  int rc;
  if ((rc = check_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, mid_f32,
                          nullptr, nullptr, workspace, workspace_bytes)))
    return rc;
  if ((rc = check_down_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                               nullptr, workspace, workspace_bytes)))
    return rc;
  if ((rc = run_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, x_f32, M, slot_ids, K, H, I, mid_f32, nullptr,
                        nullptr, workspace, workspace_bytes, stream)))
    return rc;
  return run_down_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                          nullptr, workspace, workspace_bytes, stream);
}

int q8_validate_down_f32(const void* slot, const q4_slot_layout* layout, const void* mid_f32, int64_t M, int64_t H,
                     int64_t I, const void* out_f32) {
  return check_down_single(kQ8 | kF32, slot, layout, mid_f32, M, H, I, out_f32, nullptr);
}

int q8_validate_down_grouped_f32(const void* slots_base, uint64_t slot_stride, int64_t num_slots,
                             const q4_slot_layout* layout, const void* mid_f32, int64_t M, const int32_t* slot_ids,
                             int64_t K, int64_t H, int64_t I, const void* out_f32, const void* workspace,
                             size_t workspace_bytes) {
  return check_down_grouped(kQ8 | kF32, slots_base, slot_stride, num_slots, layout, mid_f32, M, slot_ids, K, H, I, out_f32,
                            nullptr, workspace, workspace_bytes);
}

int q4_stream_read(const void* slots_base, uint64_t slot_stride, int64_t num_slots, uint64_t offset_a,
                   uint64_t offset_b, int64_t rows, int64_t row_bytes, int pattern, int waves, int depth, void* sink,
                   q4_stream_t stream) {
  if (!slots_base || !sink) return fail(Q4_ERR_INVALID_ARGUMENT, "slots and sink must be non-null device pointers");
  if (!aligned(slots_base, 16) || !aligned(sink, 4) || offset_a % 16 || offset_b % 16 || slot_stride % 16)
    return fail(Q4_ERR_ALIGNMENT, "slots, stride and offsets must be 16-byte aligned, sink 4-byte aligned");
  if (num_slots < 1 || num_slots > kMaxSlots || rows < 1 || row_bytes < 128 || row_bytes % 128)
    return fail(Q4_ERR_INVALID_ARGUMENT, "need 1 <= num_slots <= 65535, rows >= 1 and row_bytes a positive multiple of 128");
  if ((uint64_t)rows * (uint64_t)row_bytes > kMaxWeightBytes)
    return fail(Q4_ERR_UNSUPPORTED, "an array above 2^31 - 16 bytes is not supported");
  const uint64_t len = (uint64_t)rows * (uint64_t)row_bytes;
  if (offset_a > slot_stride || len > slot_stride - offset_a || offset_b > slot_stride || len > slot_stride - offset_b)
    return fail(Q4_ERR_RANGE, "an array exceeds the slot stride");
  if (pattern < 0 || pattern > 7)
    return fail(Q4_ERR_INVALID_ARGUMENT,
                "pattern must be 0 (row tiles), 1 (linear), 2 (half-line row tiles) or 3 (whole-line row tiles), "
                "plus 4 for non-temporal loads");
  if ((waves != 8 && waves != 16) || (depth != 1 && depth != 2 && depth != 4))
    return fail(Q4_ERR_UNSUPPORTED, "waves must be 8 or 16 and depth 1, 2 or 4");
  q4::StreamParams p{};
  p.base = static_cast<const uint8_t*>(slots_base);
  p.slot_stride = slot_stride;
  p.off_a = offset_a;
  p.off_b = offset_b;
  p.row_bytes = (uint32_t)row_bytes;
  p.rows = (int)rows;
  p.num_slots = (int)num_slots;
  p.sink = static_cast<uint32_t*>(sink);
  const hipError_t e = q4::launch_stream_read(p, pattern, waves, depth, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(Q4_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ok();
}

const char* q4_last_error(void) { return g_err.c_str(); }

int q4_abi_version(void) { return 5; }

}  // extern "C"
