/*
 * q4moe.h -- C ABI of the MI355X (gfx950) Q4/Q8 expert library: gate/up +
 * SwiGLU, the down projection and the whole expert, over expert slots.
 *
 * What is computed (diff of @mlx-bun/inference 1.0.0, page 52,
 * kernels/glm52/streamed-experts.ts, GATE_UP_SOURCE and its launch in
 * Glm52CanonicalMetalExecutor.execute):
 *
 *   for every token m and intermediate row i of one expert slot
 *     gate[m,i] = (sum_k (qg[i,k] - 8) * x[m,k]) * gate_scale[i]      (F32)
 *     up[m,i]   = (sum_k (qu[i,k] - 8) * x[m,k]) * up_scale[i]        (F32)
 *     gT = bf16(gate), uT = bf16(up)
 *     sT = bf16(1 / (1 + exp(-gT)))          (evaluated in F32)
 *     out[m,i] = bf16(bf16(gT * sT) * uT)
 *
 *   q[i,k] is nibble (k % 8) -- bits 4*(k%8) .. 4*(k%8)+3 -- of the
 *   little-endian uint32 word (i*H/8 + k/8) of the projection's packed rows.
 *   Every bf16 rounding is round-to-nearest-even.
 *
 * Accumulation.  The library computes each sum exactly (integer matrix-core
 * arithmetic on a fixed-point split of each bf16 x into six signed 8-bit
 * digits) and rounds (sum * scale) once to F32.  The pages accumulate in F32 FMA order,
 * which is one rounding-order approximation of the same value.  Activations
 * whose magnitudes span more than 2^38 within one token have their smallest
 * entries rounded to the token's 2^-38-relative grid (error below
 * 2^-37 * max|x| per entry).  Results are identical for every batch width,
 * kernel shape and routing (batch-invariant).
 *
 * Slot layout (page 51, kernels/glm52/layout.ts, Glm52CanonicalMetalLayout
 * and validateRange): every field is a byte offset from the slot base.
 *
 * Conventions for every entry point:
 *   - Device pointers are borrowed.  The caller owns the slots, x, out, ids,
 *     probes and workspace and keeps them alive until the stream has completed
 *     the call (the lease rule of glm52CanonicalQ4SlotView, page 52).
 *   - Calls are asynchronous on `stream`; the library never synchronises and
 *     allocates no device memory.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     invalid argument nothing is enqueued and a negative status is returned.
 *     q4_last_error() then describes the failure.
 *   - Non-finite activations are outside the contract: a token whose x holds
 *     an Inf or NaN gets NaN gate/up and a NaN output row.
 */
#ifndef Q4MOE_H
#define Q4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP stream handle (hipStream_t); NULL is the default stream. */
typedef struct ihipStream_t *q4_stream_t;

#define Q4_OFFSET_ABSENT UINT64_MAX

/* Status codes. */
enum {
  Q4_OK = 0,
  Q4_ERR_INVALID_ARGUMENT = -1, /* null pointer, non-positive size, H % 8 != 0 */
  Q4_ERR_ALIGNMENT = -2,        /* slot/stride not 4096-aligned, offsets/x/out misaligned */
  Q4_ERR_RANGE = -3,            /* a slot field does not fit inside slot_bytes */
  Q4_ERR_UNSUPPORTED = -4,      /* sizes beyond the library's limits (below) */
  Q4_ERR_HIP = -5,              /* the kernel launch failed */
  Q4_ERR_WORKSPACE = -6         /* workspace missing or smaller than required */
};

/* Limits: 8 <= H <= 65536 with H % 8 == 0; 1 <= I; I*H/2 <= 2^31 - 16;
 * 1 <= M <= 65535; grouped: 1 <= K, M*K <= 65536, 1 <= num_slots <= 65535. */

/*
 * Byte offsets of an expert slot's fields from the slot base (page 51,
 * Glm52CanonicalMetalLayout).  gate/up weights: uint32 [I][H/8] little-endian,
 * 16-byte aligned offsets.  gate/up scales: float32 [I], 4-byte aligned.
 * The down fields are read by the down and whole-expert calls only; for the
 * gate/up calls they may be Q4_OFFSET_ABSENT, otherwise they are range-checked
 * (down weights I*H/2 bytes, down scales 4*H bytes) as on page 52
 * (validateCall).
 */
typedef struct {
  uint64_t slot_bytes;
  uint64_t gate_weight_offset;
  uint64_t up_weight_offset;
  uint64_t gate_scale_offset;
  uint64_t up_scale_offset;
  uint64_t down_weight_offset;
  uint64_t down_scale_offset;
} q4_slot_layout;

/*
 * Single expert: out[M][I] (bf16) for x[M][H] (bf16) against one slot.
 *   slot      device pointer to the slot base, 4096-byte aligned
 *             (our reading of the page-aligned slot rule of
 *             glm52CanonicalQ4SlotView; the pages use 16 KiB pages).
 *   layout    host pointer to the field offsets.
 *   x_bf16    device, row-major [M][H], 16-byte aligned.
 *   out_bf16  device, row-major [M][I], 2-byte aligned.
 * Returns Q4_OK or a negative status.
 */
int q4_expert_gate_up(const void *slot, const q4_slot_layout *layout,
                      const void *x_bf16, int64_t M, int64_t H, int64_t I,
                      void *out_bf16, q4_stream_t stream);

/* As q4_expert_gate_up, and also writes the F32 gate and up values before
 * their bf16 rounding to gate_f32/up_f32 ([M][I] each, 4-byte aligned);
 * either may be NULL.  Same kernels; used by parity tests. */
int q4_expert_gate_up_probe(const void *slot, const q4_slot_layout *layout,
                            const void *x_bf16, int64_t M, int64_t H, int64_t I,
                            void *out_bf16, float *gate_f32, float *up_f32,
                            q4_stream_t stream);

/* Bytes of device workspace a grouped call of M tokens with top-K routing over
 * num_slots slots needs (a multiple of 256), or 0 for sizes outside the
 * limits.  The workspace receives the count of out-of-range ids; its size may
 * grow with these sizes in later versions, so callers should always ask. */
size_t q4_grouped_workspace_bytes(int64_t M, int64_t K, int64_t num_slots);

/*
 * Grouped call over routed expert slots.  Pair (t, j) runs token t against
 * slot slot_ids[t*K + j] and writes out[t][j][:] (bf16 [M][K][I]); each pair
 * is independent of the others (row independence, page 52).  Slots are
 * num_slots slots of one layout spaced slot_stride bytes apart from
 * slots_base (both 4096-aligned, slot_stride >= slot_bytes).
 *   slot_ids  device int32 [M][K]; duplicates are allowed.  An id outside
 *             [0, num_slots) yields zero gate/up/out for that pair, and the
 *             number of such ids is stored as int32 at workspace[0].
 *   workspace device, >= q4_grouped_workspace_bytes(M, K, num_slots)
 *             bytes, 256-byte aligned; contents on entry are ignored.  Calls
 *             that share one workspace must not overlap in time.
 */
int q4_expert_gate_up_grouped(const void *slots_base, uint64_t slot_stride,
                              int64_t num_slots, const q4_slot_layout *layout,
                              const void *x_bf16, int64_t M,
                              const int32_t *slot_ids, int64_t K,
                              int64_t H, int64_t I, void *out_bf16,
                              void *workspace, size_t workspace_bytes,
                              q4_stream_t stream);

/* As q4_expert_gate_up_grouped with optional F32 gate/up probes [M][K][I]. */
int q4_expert_gate_up_grouped_probe(const void *slots_base, uint64_t slot_stride,
                                    int64_t num_slots, const q4_slot_layout *layout,
                                    const void *x_bf16, int64_t M,
                                    const int32_t *slot_ids, int64_t K,
                                    int64_t H, int64_t I, void *out_bf16,
                                    float *gate_f32, float *up_f32,
                                    void *workspace, size_t workspace_bytes,
                                    q4_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the grouped
 * call of q4_expert_gate_up_grouped, same arguments, kernels and results, with
 * the workspace replaced by a static scratch array the library holds on each
 * GPU (256 bytes per device, kept until the process ends; its address is
 * resolved on the first call on each device).  No device memory is allocated
 * or freed by the call.
 *   invalid_count  device int32, 4-byte aligned, or NULL: receives the number
 *                  of ids outside [0, num_slots) (a device-to-device copy on
 *                  `stream` after the kernels).
 * A call whose workspace need (q4_grouped_workspace_bytes) exceeds the scratch
 * is rejected with Q4_ERR_UNSUPPORTED.  All calls on one GPU share its
 * scratch, which keeps the last call's contents: calls that overlap in time
 * on one GPU (other streams, other threads) race and must be serialised by
 * the caller.
 */
int q4_expert_gate_up_grouped_noalloc(const void *slots_base, uint64_t slot_stride,
                                      int64_t num_slots, const q4_slot_layout *layout,
                                      const void *x_bf16, int64_t M,
                                      const int32_t *slot_ids, int64_t K,
                                      int64_t H, int64_t I, void *out_bf16,
                                      int32_t *invalid_count, q4_stream_t stream);

/* Host-only argument checks of the two calls (no device access, nothing
 * enqueued): the same validation the entry points run first.  Pointers are
 * only tested for NULL and alignment. */
int q4_validate_gate_up(const void *slot, const q4_slot_layout *layout,
                        const void *x_bf16, int64_t M, int64_t H, int64_t I,
                        const void *out_bf16);
int q4_validate_grouped(const void *slots_base, uint64_t slot_stride,
                        int64_t num_slots, const q4_slot_layout *layout,
                        const void *x_bf16, int64_t M, const int32_t *slot_ids,
                        int64_t K, int64_t H, int64_t I, const void *out_bf16,
                        const void *workspace, size_t workspace_bytes);

/*
 * Down projection (page 52, DOWN_SOURCE): for every token m and hidden row h
 *
 *   down[m,h] = (sum_i (qd[h,i] - 8) * mid[m,i]) * down_scale[h]     (F32)
 *   out[m,h]  = bf16(down[m,h])                                 (nearest even)
 *
 * qd[h,i] is nibble (i % 8) of the little-endian uint32 word (h*I/8 + i/8) of
 * the down weights (uint32 [H][I/8] at down_weight_offset, 16-byte aligned);
 * down scales are float32 [H] at down_scale_offset (4-byte aligned).  The sum
 * is exact and rounded once to F32 with the scale, as for gate/up.  Needs
 * I % 8 == 0, I <= 65536 and both down offsets present (not
 * Q4_OFFSET_ABSENT).
 *   mid_bf16  device, row-major [M][I], 16-byte aligned.
 *   out_bf16  device, row-major [M][H], 2-byte aligned.
 * Returns Q4_OK or a negative status.
 */
int q4_expert_down(const void *slot, const q4_slot_layout *layout,
                   const void *mid_bf16, int64_t M, int64_t H, int64_t I,
                   void *out_bf16, q4_stream_t stream);

/* As q4_expert_down, and also writes the F32 values before their bf16
 * rounding to down_f32 ([M][H], 4-byte aligned; NULL to skip). */
int q4_expert_down_probe(const void *slot, const q4_slot_layout *layout,
                         const void *mid_bf16, int64_t M, int64_t H, int64_t I,
                         void *out_bf16, float *down_f32, q4_stream_t stream);

/*
 * Grouped down projection.  Pair (t, j) runs its own input row
 * mid[t][j][:] (bf16 [M][K][I], the layout the grouped gate/up call writes)
 * against slot slot_ids[t*K + j] and writes out[t][j][:] (bf16 [M][K][H]).
 * Slots, ids and workspace as for q4_expert_gate_up_grouped (workspace size
 * from q4_grouped_workspace_bytes(M, K, num_slots)); an id outside
 * [0, num_slots) gives a zero output row and is counted in workspace[0].
 * Needs M*K <= 65535.
 */
int q4_expert_down_grouped(const void *slots_base, uint64_t slot_stride,
                           int64_t num_slots, const q4_slot_layout *layout,
                           const void *mid_bf16, int64_t M,
                           const int32_t *slot_ids, int64_t K,
                           int64_t H, int64_t I, void *out_bf16,
                           void *workspace, size_t workspace_bytes,
                           q4_stream_t stream);

/* As q4_expert_down_grouped with an optional F32 probe [M][K][H]. */
int q4_expert_down_grouped_probe(const void *slots_base, uint64_t slot_stride,
                                 int64_t num_slots, const q4_slot_layout *layout,
                                 const void *mid_bf16, int64_t M,
                                 const int32_t *slot_ids, int64_t K,
                                 int64_t H, int64_t I, void *out_bf16,
                                 float *down_f32,
                                 void *workspace, size_t workspace_bytes,
                                 q4_stream_t stream);

/*
 * The whole expert of one slot (page 52, Glm52CanonicalMetalExecutor.execute:
 * the gate/up kernel, then the down kernel on its bf16 output):
 *   mid = q4_expert_gate_up(x), out = q4_expert_down(mid).
 *   mid_bf16  device [M][I], 16-byte aligned, caller-owned: receives the
 *             gate/up + SwiGLU output (the library allocates nothing).
 *   out_bf16  device [M][H].
 * Both steps are validated before either is enqueued.
 */
int q4_expert_forward(const void *slot, const q4_slot_layout *layout,
                      const void *x_bf16, int64_t M, int64_t H, int64_t I,
                      void *mid_bf16, void *out_bf16, q4_stream_t stream);

/* Grouped whole expert: q4_expert_gate_up_grouped into mid [M][K][I], then
 * q4_expert_down_grouped into out [M][K][H] (per-pair expert outputs, before
 * any weighting across the K experts).  One workspace serves both steps. */
int q4_expert_forward_grouped(const void *slots_base, uint64_t slot_stride,
                              int64_t num_slots, const q4_slot_layout *layout,
                              const void *x_bf16, int64_t M,
                              const int32_t *slot_ids, int64_t K,
                              int64_t H, int64_t I, void *mid_bf16,
                              void *out_bf16, void *workspace,
                              size_t workspace_bytes, q4_stream_t stream);

/* Host-only argument checks of the down calls (as q4_validate_gate_up). */
int q4_validate_down(const void *slot, const q4_slot_layout *layout,
                     const void *mid_bf16, int64_t M, int64_t H, int64_t I,
                     const void *out_bf16);
int q4_validate_down_grouped(const void *slots_base, uint64_t slot_stride,
                             int64_t num_slots, const q4_slot_layout *layout,
                             const void *mid_bf16, int64_t M,
                             const int32_t *slot_ids, int64_t K, int64_t H,
                             int64_t I, const void *out_bf16,
                             const void *workspace, size_t workspace_bytes);

/*
 * The Q8 family (page 52, Q8_GATE_UP_SOURCE, Q8_DOWN_SOURCE and
 * Glm52CanonicalQ8MetalExecutor): the same calls, arguments, layout struct
 * and results as their q4_ namesakes, with signed int8 weights, one byte per
 * weight and no zero point:
 *   gate/up weights  int8 [I][H] row-major at gate/up_weight_offset
 *                    (I*H bytes each), weight = the byte read as int8;
 *   down weights     int8 [H][I] row-major at down_weight_offset (H*I bytes);
 *   scales           float32 per row, as for Q4.
 * Weight offsets are 16-byte aligned.  H % 8 == 0 (and I % 8 == 0 for the
 * down and whole-expert calls) is this library's rule, not the pages': the
 * kernels read activations in 8-value units.  Sums are exact and rounded once
 * to F32 with the row scale, as for Q4.
 */
int q8_expert_gate_up(const void *slot, const q4_slot_layout *layout,
                      const void *x_bf16, int64_t M, int64_t H, int64_t I,
                      void *out_bf16, q4_stream_t stream);
int q8_expert_gate_up_probe(const void *slot, const q4_slot_layout *layout,
                            const void *x_bf16, int64_t M, int64_t H, int64_t I,
                            void *out_bf16, float *gate_f32, float *up_f32,
                            q4_stream_t stream);
int q8_expert_gate_up_grouped(const void *slots_base, uint64_t slot_stride,
                              int64_t num_slots, const q4_slot_layout *layout,
                              const void *x_bf16, int64_t M,
                              const int32_t *slot_ids, int64_t K,
                              int64_t H, int64_t I, void *out_bf16,
                              void *workspace, size_t workspace_bytes,
                              q4_stream_t stream);
int q8_expert_gate_up_grouped_probe(const void *slots_base, uint64_t slot_stride,
                                    int64_t num_slots, const q4_slot_layout *layout,
                                    const void *x_bf16, int64_t M,
                                    const int32_t *slot_ids, int64_t K,
                                    int64_t H, int64_t I, void *out_bf16,
                                    float *gate_f32, float *up_f32,
                                    void *workspace, size_t workspace_bytes,
                                    q4_stream_t stream);
int q8_expert_down(const void *slot, const q4_slot_layout *layout,
                   const void *mid_bf16, int64_t M, int64_t H, int64_t I,
                   void *out_bf16, q4_stream_t stream);
int q8_expert_down_probe(const void *slot, const q4_slot_layout *layout,
                         const void *mid_bf16, int64_t M, int64_t H, int64_t I,
                         void *out_bf16, float *down_f32, q4_stream_t stream);
int q8_expert_down_grouped(const void *slots_base, uint64_t slot_stride,
                           int64_t num_slots, const q4_slot_layout *layout,
                           const void *mid_bf16, int64_t M,
                           const int32_t *slot_ids, int64_t K,
                           int64_t H, int64_t I, void *out_bf16,
                           void *workspace, size_t workspace_bytes,
                           q4_stream_t stream);
int q8_expert_down_grouped_probe(const void *slots_base, uint64_t slot_stride,
                                 int64_t num_slots, const q4_slot_layout *layout,
                                 const void *mid_bf16, int64_t M,
                                 const int32_t *slot_ids, int64_t K,
                                 int64_t H, int64_t I, void *out_bf16,
                                 float *down_f32,
                                 void *workspace, size_t workspace_bytes,
                                 q4_stream_t stream);
int q8_expert_forward(const void *slot, const q4_slot_layout *layout,
                      const void *x_bf16, int64_t M, int64_t H, int64_t I,
                      void *mid_bf16, void *out_bf16, q4_stream_t stream);
int q8_expert_forward_grouped(const void *slots_base, uint64_t slot_stride,
                              int64_t num_slots, const q4_slot_layout *layout,
                              const void *x_bf16, int64_t M,
                              const int32_t *slot_ids, int64_t K,
                              int64_t H, int64_t I, void *mid_bf16,
                              void *out_bf16, void *workspace,
                              size_t workspace_bytes, q4_stream_t stream);
int q8_validate_gate_up(const void *slot, const q4_slot_layout *layout,
                        const void *x_bf16, int64_t M, int64_t H, int64_t I,
                        const void *out_bf16);
int q8_validate_grouped(const void *slots_base, uint64_t slot_stride,
                        int64_t num_slots, const q4_slot_layout *layout,
                        const void *x_bf16, int64_t M, const int32_t *slot_ids,
                        int64_t K, int64_t H, int64_t I, const void *out_bf16,
                        const void *workspace, size_t workspace_bytes);
int q8_validate_down(const void *slot, const q4_slot_layout *layout,
                     const void *mid_bf16, int64_t M, int64_t H, int64_t I,
                     const void *out_bf16);
int q8_validate_down_grouped(const void *slots_base, uint64_t slot_stride,
                             int64_t num_slots, const q4_slot_layout *layout,
                             const void *mid_bf16, int64_t M,
                             const int32_t *slot_ids, int64_t K, int64_t H,
                             int64_t I, const void *out_bf16,
                             const void *workspace, size_t workspace_bytes);

/*
 * f32 activations (page 52: validateCall accepts bfloat16 or float32 input,
 * execute gives every output the input's dtype).  Each call below is its
 * namesake without the _f32 suffix with x (and mid) float32 instead of bf16
 * -- same shapes, 16-byte aligned -- and float32 outputs (4-byte aligned).
 * With T = float the tail's conversions are identities:
 *   s = 1 / (1 + exp(-gate)), out = (gate * s) * up     (each an F32 operation;
 *   exp evaluated to within the F32 rounding of the exact value)
 * and the down output is its F32 value.  Each f32 value is split into eight
 * signed 8-bit digits on its token's largest exponent, so sums are exact for
 * values at most 38 binades below the token's largest |x| (smaller entries
 * are rounded to that grid) and rounded once to F32 with the row scale.
 */
int q4_expert_gate_up_f32(const void *slot, const q4_slot_layout *layout,
                          const void *x_f32, int64_t M, int64_t H, int64_t I,
                          void *out_f32, q4_stream_t stream);
int q4_expert_gate_up_probe_f32(const void *slot, const q4_slot_layout *layout,
                                const void *x_f32, int64_t M, int64_t H, int64_t I,
                                void *out_f32, float *gate_f32, float *up_f32,
                                q4_stream_t stream);
int q4_expert_gate_up_grouped_f32(const void *slots_base, uint64_t slot_stride,
                                  int64_t num_slots, const q4_slot_layout *layout,
                                  const void *x_f32, int64_t M, const int32_t *slot_ids,
                                  int64_t K, int64_t H, int64_t I, void *out_f32,
                                  void *workspace, size_t workspace_bytes,
                                  q4_stream_t stream);
int q4_expert_gate_up_grouped_probe_f32(const void *slots_base, uint64_t slot_stride,
                                        int64_t num_slots, const q4_slot_layout *layout,
                                        const void *x_f32, int64_t M,
                                        const int32_t *slot_ids, int64_t K, int64_t H,
                                        int64_t I, void *out_f32, float *gate_f32,
                                        float *up_f32, void *workspace,
                                        size_t workspace_bytes, q4_stream_t stream);
int q4_validate_gate_up_f32(const void *slot, const q4_slot_layout *layout,
                            const void *x_f32, int64_t M, int64_t H, int64_t I,
                            const void *out_f32);
int q4_validate_grouped_f32(const void *slots_base, uint64_t slot_stride,
                            int64_t num_slots, const q4_slot_layout *layout,
                            const void *x_f32, int64_t M, const int32_t *slot_ids,
                            int64_t K, int64_t H, int64_t I, const void *out_f32,
                            const void *workspace, size_t workspace_bytes);
int q4_expert_down_f32(const void *slot, const q4_slot_layout *layout,
                       const void *mid_f32, int64_t M, int64_t H, int64_t I,
                       void *out_f32, q4_stream_t stream);
int q4_expert_down_probe_f32(const void *slot, const q4_slot_layout *layout,
                             const void *mid_f32, int64_t M, int64_t H, int64_t I,
                             void *out_f32, float *down_f32, q4_stream_t stream);
int q4_expert_down_grouped_f32(const void *slots_base, uint64_t slot_stride,
                               int64_t num_slots, const q4_slot_layout *layout,
                               const void *mid_f32, int64_t M, const int32_t *slot_ids,
                               int64_t K, int64_t H, int64_t I, void *out_f32,
                               void *workspace, size_t workspace_bytes,
                               q4_stream_t stream);
int q4_expert_down_grouped_probe_f32(const void *slots_base, uint64_t slot_stride,
                                     int64_t num_slots, const q4_slot_layout *layout,
                                     const void *mid_f32, int64_t M,
                                     const int32_t *slot_ids, int64_t K, int64_t H,
                                     int64_t I, void *out_f32, float *down_f32,
                                     void *workspace, size_t workspace_bytes,
                                     q4_stream_t stream);
int q4_expert_forward_f32(const void *slot, const q4_slot_layout *layout,
                          const void *x_f32, int64_t M, int64_t H, int64_t I,
                          void *mid_f32, void *out_f32, q4_stream_t stream);
int q4_expert_forward_grouped_f32(const void *slots_base, uint64_t slot_stride,
                                  int64_t num_slots, const q4_slot_layout *layout,
                                  const void *x_f32, int64_t M, const int32_t *slot_ids,
                                  int64_t K, int64_t H, int64_t I, void *mid_f32,
                                  void *out_f32, void *workspace,
                                  size_t workspace_bytes, q4_stream_t stream);
int q4_validate_down_f32(const void *slot, const q4_slot_layout *layout,
                         const void *mid_f32, int64_t M, int64_t H, int64_t I,
                         const void *out_f32);
int q4_validate_down_grouped_f32(const void *slots_base, uint64_t slot_stride,
                                 int64_t num_slots, const q4_slot_layout *layout,
                                 const void *mid_f32, int64_t M,
                                 const int32_t *slot_ids, int64_t K, int64_t H,
                                 int64_t I, const void *out_f32, const void *workspace,
                                 size_t workspace_bytes);
int q8_expert_gate_up_f32(const void *slot, const q4_slot_layout *layout,
                          const void *x_f32, int64_t M, int64_t H, int64_t I,
                          void *out_f32, q4_stream_t stream);
int q8_expert_gate_up_probe_f32(const void *slot, const q4_slot_layout *layout,
                                const void *x_f32, int64_t M, int64_t H, int64_t I,
                                void *out_f32, float *gate_f32, float *up_f32,
                                q4_stream_t stream);
int q8_expert_gate_up_grouped_f32(const void *slots_base, uint64_t slot_stride,
                                  int64_t num_slots, const q4_slot_layout *layout,
                                  const void *x_f32, int64_t M, const int32_t *slot_ids,
                                  int64_t K, int64_t H, int64_t I, void *out_f32,
                                  void *workspace, size_t workspace_bytes,
                                  q4_stream_t stream);
int q8_expert_gate_up_grouped_probe_f32(const void *slots_base, uint64_t slot_stride,
                                        int64_t num_slots, const q4_slot_layout *layout,
                                        const void *x_f32, int64_t M,
                                        const int32_t *slot_ids, int64_t K, int64_t H,
                                        int64_t I, void *out_f32, float *gate_f32,
                                        float *up_f32, void *workspace,
                                        size_t workspace_bytes, q4_stream_t stream);
int q8_validate_gate_up_f32(const void *slot, const q4_slot_layout *layout,
                            const void *x_f32, int64_t M, int64_t H, int64_t I,
                            const void *out_f32);
int q8_validate_grouped_f32(const void *slots_base, uint64_t slot_stride,
                            int64_t num_slots, const q4_slot_layout *layout,
                            const void *x_f32, int64_t M, const int32_t *slot_ids,
                            int64_t K, int64_t H, int64_t I, const void *out_f32,
                            const void *workspace, size_t workspace_bytes);
int q8_expert_down_f32(const void *slot, const q4_slot_layout *layout,
                       const void *mid_f32, int64_t M, int64_t H, int64_t I,
                       void *out_f32, q4_stream_t stream);
int q8_expert_down_probe_f32(const void *slot, const q4_slot_layout *layout,
                             const void *mid_f32, int64_t M, int64_t H, int64_t I,
                             void *out_f32, float *down_f32, q4_stream_t stream);
int q8_expert_down_grouped_f32(const void *slots_base, uint64_t slot_stride,
                               int64_t num_slots, const q4_slot_layout *layout,
                               const void *mid_f32, int64_t M, const int32_t *slot_ids,
                               int64_t K, int64_t H, int64_t I, void *out_f32,
                               void *workspace, size_t workspace_bytes,
                               q4_stream_t stream);
int q8_expert_down_grouped_probe_f32(const void *slots_base, uint64_t slot_stride,
                                     int64_t num_slots, const q4_slot_layout *layout,
                                     const void *mid_f32, int64_t M,
                                     const int32_t *slot_ids, int64_t K, int64_t H,
                                     int64_t I, void *out_f32, float *down_f32,
                                     void *workspace, size_t workspace_bytes,
                                     q4_stream_t stream);
int q8_expert_forward_f32(const void *slot, const q4_slot_layout *layout,
                          const void *x_f32, int64_t M, int64_t H, int64_t I,
                          void *mid_f32, void *out_f32, q4_stream_t stream);
int q8_expert_forward_grouped_f32(const void *slots_base, uint64_t slot_stride,
                                  int64_t num_slots, const q4_slot_layout *layout,
                                  const void *x_f32, int64_t M, const int32_t *slot_ids,
                                  int64_t K, int64_t H, int64_t I, void *mid_f32,
                                  void *out_f32, void *workspace,
                                  size_t workspace_bytes, q4_stream_t stream);
int q8_validate_down_f32(const void *slot, const q4_slot_layout *layout,
                         const void *mid_f32, int64_t M, int64_t H, int64_t I,
                         const void *out_f32);
int q8_validate_down_grouped_f32(const void *slots_base, uint64_t slot_stride,
                                 int64_t num_slots, const q4_slot_layout *layout,
                                 const void *mid_f32, int64_t M,
                                 const int32_t *slot_ids, int64_t K, int64_t H,
                                 int64_t I, const void *out_f32, const void *workspace,
                                 size_t workspace_bytes);

/* Message for the last failing call on this thread ("" after success). */
const char *q4_last_error(void);

/*
 * Measurement aid (no part of the method): reads, in each of num_slots slots
 * spaced slot_stride bytes apart from slots_base, two arrays of `rows` rows
 * of row_bytes bytes at offset_a and offset_b (for an expert slot: its gate
 * and up weights), each byte once, with no arithmetic.
 *   pattern 0  the gate/up kernels' weight access: 16-row tiles, 128 bytes of
 *              each row per step, 32 bytes per lane;
 *   pattern 1  the same bytes per step as two lane-linear 1 KiB runs;
 *   pattern 2  16-row tiles, 128 bytes of each row per step, lane l's two
 *              16-byte loads at (l / 16) * 16 and 64 + (l / 16) * 16: each
 *              load instruction covers one 64-byte half of every row's 128;
 *   pattern 3  16-row tiles, 128 bytes of each row per step, 8 lanes per row:
 *              each load instruction covers whole 128-byte lines of 8 rows;
 *   pattern+4  the same with the non-temporal load hint (bytes read once).
 *   waves      8 or 16 waves per work-group (one work-group per CU);
 *   depth      steps in flight per wave: 1, 2 or 4.
 *   sink       device, one 4-byte word; written only on a data value that
 *              real data practically never gives (keeps the loads live).
 * Needs row_bytes a positive multiple of 128, 16-byte aligned slots_base,
 * slot_stride and offsets, offset + rows*row_bytes <= slot_stride, and
 * rows*row_bytes <= 2^31 - 16.  Asynchronous on `stream`.
 */
int q4_stream_read(const void *slots_base, uint64_t slot_stride, int64_t num_slots,
                   uint64_t offset_a, uint64_t offset_b, int64_t rows, int64_t row_bytes,
                   int pattern, int waves, int depth, void *sink, q4_stream_t stream);

/* ABI version: 5 (1 plus the down projection and whole-expert calls, the Q8
 * family, f32 activations, the (M, K, num_slots) workspace query and the
 * streaming-read measurement aid). */
int q4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4MOE_H */
