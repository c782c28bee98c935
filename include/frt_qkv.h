/* frt_qkv.h -- C ABI of the attention-input path on MI355X (gfx950):
 * residual add + RMSNorm + E4M3 quantise (the same K1 as the FFN chain),
 * then the fused QKV projection on FP8 operands with a split + rotary
 * embedding epilogue, written as bf16 Q, K and V.
 *
 * Defined on the pages: FlashRT architecture doc, component "Kernel
 * library" (the "qkv split + RoPE" fusion among the memory-bound kernels);
 * itsolotime article section 5.2 (the Pi0 / Pi0.5 specs' FusedQKV weight:
 * the q, k and v projections of a layer fused into one matrix, transposed
 * and quantised, with head interleave counts and, for Pi0, the input norm
 * weight folded in).
 *
 * Arithmetic (every rounding point):
 *   K1 as in frt_ffn.h: r' = bf16(r + y); x = RMSNorm(r') (or AdaRMSNorm);
 *     xq = e4m3(f32(x * inv_x)), inv_x = f32(1 / s_x)
 *   A[m][n] = sum_k dec(xq[m][k]) * dec(W[n][k]) accumulated in fp32, W the
 *     fused rows [Wq; Wk; Wv] quantised with ONE per-tensor scale s_w;
 *     v_n = f32(A * alpha), alpha = f32(s_x * s_w)
 *   Q and K heads (half-split rotation: dimension d < hd/2 pairs with
 *   d + hd/2), (c, s) = table[pos[m]][d]:
 *     out[d]        = bf16(f32(f32(v_d * c) - f32(v_{d+hd/2} * s)))
 *     out[d + hd/2] = bf16(f32(f32(v_{d+hd/2} * c) + f32(v_d * s)))
 *   V heads: bf16(v).
 *   Rotary table entry (p, i): f32(cos(p * base^(-2i/hd))) and f32(sin(..)),
 *   evaluated in fp64 on the device at plan creation.
 *
 * Layouts: Q [M][nq][hd], K [M][nkv][hd], V [M][nkv][hd] bf16, row-major;
 * rotary table [max_pos][hd/2] of (cos, sin) fp32 pairs.  On the device the
 * fused weight is packed so that the two 16-row groups holding dimensions
 * d and d + hd/2 of one head sit side by side (the pages' head interleave):
 * each rotation pair then meets in one lane of the matrix-core output.
 *
 * Ownership and errors follow frt_ffn.h: the caller owns the workspace and
 * the streams; every call returns an frt_status and frt_last_error() holds
 * the text of the last failure on the calling thread.
 */
#ifndef FRT_QKV_H
#define FRT_QKV_H

#include <stddef.h>
#include <stdint.h>

#include "frt_ffn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Problem description.  Requirements: M >= 1, H a multiple of 128 and at most
 * 16384, nq >= 1, nkv >= 1, hd a multiple of 32 and at most 512, max_pos >= 1,
 * eps > 0, rope_base > 1.  Flags: FRT_FLAG_NORM_FUSE (fold the norm weight
 * into the fused QKV codes per input column) or FRT_FLAG_ADA_NORM
 * (AdaRMSNorm modulation from the io.mod slot), not both. */
typedef struct {
  int32_t M;          /* rows (tokens) per forward                       */
  int32_t H;          /* hidden size (K of the GEMM)                     */
  int32_t nq;         /* query heads                                     */
  int32_t nkv;        /* key / value heads                               */
  int32_t hd;         /* head dimension                                  */
  int32_t max_pos;    /* rotary table rows: positions 0 .. max_pos-1      */
  float eps;          /* RMSNorm epsilon                                 */
  float rope_base;    /* rotary frequency base                           */
  int32_t device;     /* HIP device ordinal                              */
  uint32_t flags;     /* FRT_FLAG_NORM_FUSE / FRT_FLAG_ADA_NORM           */
} frt_qkv_desc;

typedef struct frt_qkv_plan frt_qkv_plan;

/* Fixed device addresses inside the workspace (stable for the plan's life,
 * so a captured graph replays on whatever the caller writes there). */
typedef struct {
  void *r_in;   /* bf16 [M][H] residual entering the block (caller writes)   */
  void *y_in;   /* bf16 [M][H] previous sub-block output (caller writes;      */
                /*   zeros after plan creation)                              */
  void *pos;    /* int32 [M] rotary positions (caller writes, each in          */
                /*   [0, max_pos); the kernels clamp others into range)      */
  void *mod;    /* bf16 [2][H] AdaRMSNorm scale, shift (ADA plans) or NULL    */
  void *r_out;  /* bf16 [M][H] r' = bf16(r + y)                               */
  void *xq;     /* e4m3 [M][H] quantised normalised rows                      */
  void *q;      /* bf16 [M][nq][hd]                                           */
  void *k;      /* bf16 [M][nkv][hd]                                          */
  void *v;      /* bf16 [M][nkv][hd]                                          */
  void *rope;   /* fp32 [max_pos][hd/2][2] (cos, sin) rotary table            */
} frt_qkv_io;

/* Workspace bytes a plan for `desc` needs; FRT_ERR_INVALID_ARG for an
 * invalid descriptor. */
frt_status frt_qkv_workspace_size(const frt_qkv_desc *desc, size_t *bytes);

/* Carve the plan out of `d_workspace` (device memory, 256-byte aligned, at
 * least frt_qkv_workspace_size bytes, owned by the caller and kept alive
 * until destroy), zero the slots and build the rotary table on the device
 * (synchronous).  Allocates no device memory. */
frt_status frt_qkv_plan_create(const frt_qkv_desc *desc, void *d_workspace, size_t bytes,
                               frt_qkv_plan **out);
frt_status frt_qkv_plan_destroy(frt_qkv_plan *plan);

/* Quantise the fused weight from device bf16 [nq*hd][H], [nkv*hd][H],
 * [nkv*hd][H] (nn.Linear layout) and copy the norm weight bf16 [H] (folded
 * and replaced by ones under FRT_FLAG_NORM_FUSE; unused under
 * FRT_FLAG_ADA_NORM).  One scale s_w = f32(amax / 448) over all three
 * matrices.  Runs on `stream` and synchronises it. */
frt_status frt_qkv_quant_weights(frt_qkv_plan *plan, const void *d_wq, const void *d_wk, const void *d_wv,
                                 const void *d_norm_w, void *stream);

/* Copy the fused codes to host memory in plain row order [(nq+2nkv)*hd][H]. */
frt_status frt_qkv_export_weight_codes(const frt_qkv_plan *plan, void *host_dst);

/* Measurement pass: s_x = f32(amax / 448) of the normalised rows over
 * `nbatch` device batches of `rows` (<= M) rows (d_y_batches may be NULL for
 * zero Y).  Synchronous. */
frt_status frt_qkv_calibrate(frt_qkv_plan *plan, const void *const *d_r_batches,
                             const void *const *d_y_batches, int32_t nbatch, int32_t rows, void *stream);

/* host_out[0] = s_x, host_out[1] = s_w (0 until set). */
frt_status frt_qkv_get_scales(const frt_qkv_plan *plan, float *host_out);
/* Install s_x (finite, > 0): the calibration cache-hit path. */
frt_status frt_qkv_set_act_scale(frt_qkv_plan *plan, float s_x);
/* Check host positions (each in [0, max_pos)) and copy them into io.pos
 * (synchronous). */
frt_status frt_qkv_set_positions(frt_qkv_plan *plan, const int32_t *host_pos, void *stream);

frt_status frt_qkv_io_get(const frt_qkv_plan *plan, frt_qkv_io *out);

/* Eager forward on `stream`: K1 then the QKV GEMM with its epilogue.
 * FRT_ERR_STATE until weights and s_x are set. */
frt_status frt_qkv_forward(frt_qkv_plan *plan, void *stream);
/* Average microseconds of kernel `which` (0: K1, 1: QKV GEMM) over `reps`
 * back-to-back launches timed with HIP events on `stream`. */
frt_status frt_qkv_time_kernel(frt_qkv_plan *plan, int32_t which, int32_t reps, void *stream, float *avg_us);
/* Capture the forward as a graph (relaxed mode, `stream` must not be the
 * null stream) and replay it; FRT_ERR_STATE for a replay with no graph or
 * after the weights or scale changed. */
frt_status frt_qkv_graph_capture(frt_qkv_plan *plan, void *stream);
frt_status frt_qkv_graph_replay(frt_qkv_plan *plan, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FRT_QKV_H */
