/*
 * frt_ffn.h -- C ABI of the fused FP8 transformer-FFN chain for AMD MI355X
 * (gfx950).
 *
 * The operation (FlashRT pages):
 *   - itsolotime article, section 7.2 (the encoder FFN loop): a high
 *     precision residual stream, RMSNorm, gate and up projections, a fused
 *     gated activation (GEGLU / SiLU family) that re-quantises its output,
 *     the down projection, and the residual add;
 *   - itsolotime article, section 7.1 and the FlashRT project page ("main
 *     ideas"): FP8 E4M3 weights and activations with per-tensor scales;
 *   - FlashRT architecture doc, component "Kernel library": residual + norm
 *     + quant fusions as hand-written kernels;
 *   - FlashRT architecture doc, component "Calibration": a measurement pass
 *     records amax per FP8 GEMM input, then alpha = act_scale * weight_scale
 *     is baked into the captured graph as host scalars;
 *   - FlashRT architecture doc, component "CUDA Graph" and the layer
 *     diagram's "C ABI execution contract: Buffer / Graph / Plan": the
 *     captured forward takes only device pointers, allocates nothing,
 *     lives for the process lifetime, and replay before capture is an error
 *     (itsolotime article, section 4.1: relaxed capture of one stream).
 *
 * Per layer i (0-based) the chain maps slots (R[i], Y[i]) -> (R[i+1], Y[i+1]):
 *   R[i+1] = bf16(R[i] + Y[i])                         new residual
 *   XQ[i]  = e4m3(RMSNorm(R[i+1]) * w_norm[i] / s_x[i])  kernel 1
 *   HQ[i]  = e4m3(act(XQ Wg^T a_g, XQ Wu^T a_u) / s_h[i]) kernel 2 (gate/up)
 *   Y[i+1] = bf16(HQ Wd^T a_d)                          kernel 3 (down)
 * and after the last layer Z = bf16(R[L] + Y[L]).  a_g = s_x s_g,
 * a_u = s_x s_u, a_d = s_h s_d.  GeGLU: gelu_tanh(g) * u; SwiGLU: silu(g) * u;
 * non-gated GELU: gelu_tanh(u) (no gate projection).
 *
 * Conventions:
 *   - bf16 tensors are row-major uint16 bit patterns, E4M3 tensors are
 *     row-major bytes (OCP E4M3FN: bias 7, max 448, saturating quantisers).
 *   - Weights are passed in nn.Linear layout [out, in], bf16.
 *   - Every pointer argument marked "device" must point to device memory of
 *     the plan's device; "host" pointers are ordinary host memory.
 *   - The caller owns all device memory, including the workspace the plan is
 *     carved from.  The library never calls hipMalloc / hipFree.
 *   - No function throws; each returns a frt_status.  On failure
 *     frt_last_error() (thread-local) names the failing check or HIP call.
 *   - Calls on one plan must not overlap (a plan holds no lock).
 */
#ifndef FRT_FFN_H
#define FRT_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FRT_OK = 0,
  FRT_ERR_INVALID_ARG = 1, /* bad pointer / dimension / index              */
  FRT_ERR_HIP = 2,         /* a HIP runtime call failed (named in last_error) */
  FRT_ERR_STATE = 3,       /* call out of order (e.g. replay before capture) */
  FRT_ERR_UNSUPPORTED = 4, /* valid but unsupported (e.g. wrong device arch) */
  FRT_ERR_WORKSPACE = 5    /* workspace too small or misaligned              */
} frt_status;

typedef enum {
  FRT_ACT_GEGLU_TANH = 0, /* gelu_tanh(gate) * up            */
  FRT_ACT_SWIGLU = 1,     /* silu(gate) * up                 */
  FRT_ACT_GELU_TANH = 2   /* gelu_tanh(up), no gate weights  */
} frt_act;

/* Plan flags.
 * FRT_FLAG_FP8_MFMA_DOWN: run the down projection on the FP8 matrix cores
 *   (twice the f16 rate).  Their adder truncates each product below 2^-13 of
 *   the largest operand-exponent sum of its group of 8 along K, so the bf16
 *   block output differs from an fp32-accumulated sum by up to ~1e-3
 *   relative (within the block tolerance), but a deep chain drifts several
 *   times further than any fp32-accumulated order (the 18-layer M=788 chain:
 *   Z cosine 0.9917 against the oracle's chain, against 0.9991 without the
 *   flag), so it is opt-in.  Without it every GEMM runs on the f16 matrix
 *   cores with exactly converted E4M3 operands (fp32-accurate accumulation). */
#define FRT_FLAG_FP8_MFMA_DOWN 1u
/* FRT_FLAG_FUSED_NORM: for M <= 16 (when M*H <= 32768) run the add +
 *   RMSNorm + quantise step inside the gate/up GEMV kernel (two kernels per
 *   layer); every workgroup recomputes the rows' norm from the L2-resident
 *   inputs (the previous down GEMV's split-K partial sums included).
 *   Results are identical to the separate kernels.  Not the default: it
 *   measures slower than the default decode layer, whose norm is split
 *   between a short slice-sum kernel and the gate/up GEMV's prologue (each
 *   wave quantises the activations of its own K range).  Ignored for other
 *   shapes. */
#define FRT_FLAG_FUSED_NORM 2u
/* FRT_FLAG_FP8_MFMA_GATEUP: the gate/up GEMM for M > 64 (the GEMM paths;
 *   the GEMVs of smaller M keep the f16 cores) runs on the FP8 matrix cores
 *   (same accumulation behaviour as FRT_FLAG_FP8_MFMA_DOWN).  Its re-quantised
 *   HQ codes miss the byte tolerance (about 1.4e-3 of them flip, against
 *   1e-4), so it stays opt-in. */
#define FRT_FLAG_FP8_MFMA_GATEUP 4u
/* FRT_FLAG_NORM_FUSE (itsolotime article, section 5.2: the Pi0 decoder spec
 *   folds each RMSNorm weight into the gate/up matrices): frt_quant_weights
 *   quantises f32(W[i][k] * w_norm[k]) for the gate and up matrices (exact
 *   products of two bf16 values) and the norm step multiplies by 1. */
#define FRT_FLAG_NORM_FUSE 8u
/* FRT_FLAG_ADA_NORM (same section: Pi0.5 modulates through AdaRMSNorm Dense
 *   layers instead): the norm step computes
 *   x = f32(f32(f32(r' * inv_rms) * f32(1 + scale[k])) + shift[k]) with the
 *   per-layer bf16 vectors in the plan's modulation slots (frt_ffn_io
 *   mod_slots; zeros after plan creation, i.e. unit scale and no shift); the
 *   RMSNorm weight is not used.  The caller writes new modulation (from its
 *   conditioning Dense layers) into the slots before a replay, like the
 *   inputs.  Excludes FRT_FLAG_NORM_FUSE and FRT_FLAG_FUSED_NORM. */
#define FRT_FLAG_ADA_NORM 16u
/* FRT_FLAG_MXFP4 (itsolotime article, section 7.2: the NVFP4 encoder FFN --
 *   AWQ pre-scale, 4-bit gate/up and down GEMMs, a gated combine that
 *   re-quantises to 4 bits, a high-precision residual -- here in the OCP
 *   MXFP4 format on gfx950's block-scaled FP4 matrix instructions):
 *   weights, XQ and HQ are FP4 E2M1 codes with one E8M0 exponent e (scale
 *   2^(e-127)) per 32 values along K; e = floor(log2(amax)) - 2 + 127 per
 *   block, elements rounded to nearest (ties to the even mantissa) and
 *   saturated at 6.  No activation scales: frt_calibrate returns
 *   FRT_ERR_UNSUPPORTED and the forward needs none.  The residual stays bf16.
 *     K1: x as without the flag, then xs = f32(x * f32(1/s[k])) with the
 *         layer's AWQ scale s (frt_set_awq; 1 by default), XQ = MXFP4(xs)
 *     gate/up: weights f32(W[i][k] * s[k]) in MXFP4; g, u fp32-accumulated
 *         block-scaled products; h = act(g) * u; HQ = MXFP4(h) along I
 *     down: Y = bf16(fp32-accumulated block-scaled products)
 *   M <= 64 runs GEMVs, larger M the block-scaled prefill GEMM (128 x 256
 *   tiles for gate/up, 128 x 128 with K split into fp32 partials for down).
 *   Requires H and I multiples of 512; excludes the FP8, fused-norm and
 *   norm-fusion flags.  Slots: each XQ slot holds codes [M][H/2] (two per
 *   byte, low nibble first) followed by the exponents of row m, 32-block b:
 *   for M <= 64 (rows padded to a multiple of 16) at byte
 *   (((m/16) * (H/512) + b/16) * 64 + (b%4) * 16 + m%16) * 4 + (b/4)%4;
 *   for M > 64 (rows padded to a multiple of 128) at byte
 *   ((m/64) * (H/128) + b/4) * 256 + ((b%4) * 16 + m%16) * 4 + (m/16)%4.
 *   HQ likewise with I. */
#define FRT_FLAG_MXFP4 32u

/* Problem description.  Requirements: M >= 1, L >= 1, H and I multiples of
 * 128, H <= 16384, I <= 32768, M*H <= 2^31 and M*I <= 2^31, act in frt_act,
 * eps > 0.  `device` is the HIP
 * device ordinal the plan and its workspace live on.  `flags` is a bitwise OR
 * of FRT_FLAG_* values (0 for the defaults). */
typedef struct {
  int32_t M, H, I, L;
  int32_t act;
  float eps;
  int32_t device;
  uint32_t flags;
} frt_ffn_desc;

typedef struct frt_plan frt_plan; /* opaque */

/* Fixed device addresses inside the plan's workspace, valid until
 * frt_ffn_plan_destroy (the architecture doc's slot pointers that stay stable
 * across capture and replay).  Slot i of a per-layer array starts at
 * base + i * stride bytes. */
typedef struct {
  void *r_slots;  /* bf16 [L+1][M][H]: R[0] (input) .. R[L]       */
  void *y_slots;  /* bf16 [L+1][M][H]: Y[0] (input) .. Y[L]       */
  void *xq_slots; /* e4m3 [L][M][H]:   XQ[0] .. XQ[L-1]           */
  void *hq_slots; /* e4m3 [L][M][I]:   HQ[0] .. HQ[L-1]           */
  void *z_out;    /* bf16 [M][H]:      Z = bf16(R[L] + Y[L])      */
  size_t stride_rh;  /* bytes between R (and Y) slots = M*H*2      */
  size_t stride_xq;  /* bytes between XQ slots = M*H              */
  size_t stride_hq;  /* bytes between HQ slots = M*I              */
  void *mod_slots;   /* bf16 [L][2][H]: AdaRMSNorm scale, shift per layer
                        (FRT_FLAG_ADA_NORM plans; NULL otherwise)   */
  size_t stride_mod; /* bytes between layers' modulation = 2*H*2   */
} frt_ffn_io;

/* Workspace bytes a plan for `desc` needs (weights, slots, split-K partials,
 * counters, calibration scratch).  Fails with FRT_ERR_INVALID_ARG on a bad
 * desc.  Pure host computation. */
frt_status frt_ffn_workspace_size(const frt_ffn_desc *desc, size_t *bytes);

/* Create a plan over a caller-owned device workspace of at least
 * frt_ffn_workspace_size bytes, 256-byte aligned, on desc->device.  Zeroes
 * the plan's counters and slot Y[0] on the null stream and synchronises.
 * Checks that the device is gfx950 (FRT_ERR_UNSUPPORTED otherwise).
 * *out receives the plan (host memory owned by the library). */
frt_status frt_ffn_plan_create(const frt_ffn_desc *desc, void *d_workspace, size_t bytes,
                               frt_plan **out);

/* Destroy a plan (and its captured graph).  The workspace stays the
 * caller's.  NULL is accepted. */
frt_status frt_ffn_plan_destroy(frt_plan *plan);

/* Quantise one layer's weights into the plan (architecture doc, component
 * "Weights": transpose/Quant transforms with per-tensor scales collected in a
 * table; itsolotime article section 5.2: FusedGateUp).  Per tensor T:
 * s = amax(|T|) > 0 ? f32(amax/448) : 1, code = e4m3(f32(T * f32(1/s))).
 *   d_w_gate  device bf16 [I,H] (must be NULL for FRT_ACT_GELU_TANH)
 *   d_w_up    device bf16 [I,H]
 *   d_w_down  device bf16 [H,I]
 *   d_norm_w  device bf16 [H] RMSNorm weight (copied into the plan; with
 *             FRT_FLAG_NORM_FUSE folded into the gate/up matrices and the
 *             plan's norm weight set to 1; unused with FRT_FLAG_ADA_NORM)
 * Runs on `stream` and synchronises it (the scales are host scalars).  The
 * caller may free the bf16 inputs after return.  Marks a captured graph
 * stale. */
frt_status frt_quant_weights(frt_plan *plan, int32_t layer, const void *d_w_gate,
                             const void *d_w_up, const void *d_w_down, const void *d_norm_w,
                             void *stream);

/* Copy one layer's quantised weight codes out in canonical nn.Linear layout
 * (which: 0 gate [I,H], 1 up [I,H], 2 down [H,I]) into host memory of
 * I*H bytes.  Synchronous. */
frt_status frt_export_weight_codes(const frt_plan *plan, int32_t layer, int32_t which,
                                   void *host_dst);

/* MXFP4 plans: copy layer `layer`'s weight `which` (0 gate, 1 up, 2 down) to
 * host memory in plain row order: codes [rows][cols/2] (two per byte, low
 * nibble first) and E8M0 exponents [rows][cols/32] (nn.Linear [out][in]
 * orientation, K = in along the blocks).  FRT_ERR_STATE for other plans. */
frt_status frt_export_mxfp4_weights(const frt_plan *plan, int32_t layer, int32_t which, void *host_codes,
                                    void *host_exponents);

/* MXFP4 plans: set layer `layer`'s AWQ pre-scale from device bf16 [H] (each
 * finite and > 0; the pages' activation-aware pre-scale, computed by the
 * caller from its calibration statistics).  The next frt_quant_weights of
 * the layer multiplies the gate/up weights by it per input column, and K1
 * multiplies the normalised activations by f32(1/s).  Marks the layer's
 * weights unset (quantise again after it).  Synchronous. */
frt_status frt_set_awq(frt_plan *plan, int32_t layer, const void *d_awq, void *stream);

/* Calibration measurement pass (architecture doc, component "Calibration",
 * phase (a); the predict() flow's cache-miss path "run 1 fwd, record amax").
 * Runs layers [layer_begin, layer_end) with unquantised fp32 activations and
 * the quantised weights (codes times their scale) over `nbatch` batches of
 * `rows` (1..M) rows and records per layer amax(|x|) (gate/up input) and
 * amax(|h|) (down input) over all batches; sets s_x = f32(amax_x/448) and
 * s_h = f32(amax_h/448) (1 when amax is 0) for those layers only.  The
 * whole-chain calibration is layer_begin = 0, layer_end = L.
 *   d_r_batches  host array of nbatch device pointers, bf16 [rows][H]: the
 *                residual entering layer_begin
 *   d_y_batches  host array of nbatch device pointers (bf16 [rows][H]): the
 *                previous block output entering layer_begin, or NULL (zeros)
 * The weights of those layers must be set.  Synchronises `stream`.  Marks a
 * captured graph stale. */
frt_status frt_calibrate(frt_plan *plan, const void *const *d_r_batches,
                         const void *const *d_y_batches, int32_t nbatch, int32_t rows,
                         int32_t layer_begin, int32_t layer_end, void *stream);

/* Read all per-layer scales into host memory as float[L][5] =
 * {s_x, s_g, s_u, s_h, s_d} (s_g = 1 for the non-gated activation; s_x, s_h
 * are 0 until calibrated or set).  The forward needs every layer's s_x and
 * s_h set (FRT_ERR_STATE otherwise). */
frt_status frt_get_scales(const frt_plan *plan, float *host_out);

/* Install static activation scales float[L][2] = {s_x, s_h} from host memory
 * (the calibration cache-hit path: "load JSON, bake alpha").  Every value
 * must be finite and > 0.  Marks a captured graph stale. */
frt_status frt_set_act_scales(frt_plan *plan, const float *host_in);

/* Fixed device addresses of the plan's activation slots. */
frt_status frt_ffn_io_get(const frt_plan *plan, frt_ffn_io *out);

/* Which kernels the plan's forward runs, as FRT_PATH_* bits (fixed at plan
 * creation from M, H, I, the flags and the FRT_* environment overrides):
 *   FRT_PATH_GEMV: M <= 16, the decode GEMVs (else multi-tile GEMVs or GEMMs)
 *   FRT_PATH_NORM_SPLIT: the decode norm split into slice sums and the
 *     gate/up GEMV's own quantisation
 *   FRT_PATH_DOWN_WHOLE_COLUMN: the whole-column down GEMV (M <= 4, E4M3 or
 *     MXFP4), which forms the next layer's R' and norm slice sums (no norm
 *     kernel between layers; the down matrix is held in its column-quad
 *     layout)
 *   FRT_PATH_DOWN_SPLIT_K: the down projection's K is split over
 *     workgroups, the fp32 partials summed by the next kernel
 *   FRT_PATH_GATEUP_OCTETS: the decode gate/up GEMV's workgroups own eight
 *     gate and eight up columns (the gated gate/up matrix held in octet
 *     order) instead of sixteen of each
 * For tests and logs; FRT_ERR_INVALID_ARG on a NULL argument. */
#define FRT_PATH_GEMV 1u
#define FRT_PATH_NORM_SPLIT 2u
#define FRT_PATH_DOWN_WHOLE_COLUMN 4u
#define FRT_PATH_DOWN_SPLIT_K 8u
#define FRT_PATH_GATEUP_OCTETS 16u
frt_status frt_ffn_plan_path(const frt_plan *plan, uint32_t *path_bits);

/* The FRT_PATH_* bits a plan created from `desc` would have, under the
 * current environment, without creating it: host only, no device call.
 * FRT_ERR_INVALID_ARG on a NULL pointer or an invalid descriptor (as
 * frt_ffn_workspace_size). */
frt_status frt_ffn_desc_path(const frt_ffn_desc *desc, uint32_t *path_bits);

/* Eager forward of layers [layer_begin, layer_end) on `stream`: reads slots
 * R[layer_begin], Y[layer_begin], writes the later slots; when layer_end == L
 * also writes Z.  Asynchronous: no allocation, no host synchronisation.
 * Requires all weights and activation scales (FRT_ERR_STATE otherwise). */
frt_status frt_ffn_forward_range(frt_plan *plan, int32_t layer_begin, int32_t layer_end,
                                 void *stream);

/* For callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid it), beyond the
 * plan's workspace they already own: frt_ffn_forward_range with the
 * forward's scratch -- the down projection's split-K fp32 partial sums and
 * the decode norm's fp64 slice sums of squares -- in the library's static
 * device array (16 MiB per GPU, held until the process ends) instead of the
 * workspace's scratch region.  Same kernels, launch configuration and
 * results as frt_ffn_forward_range, bit for bit.  Allocates nothing and calls
 * no allocating routine; the first call on a device looks up the array's
 * address there.  Nothing in the array needs to start at zero (every call
 * writes what it reads).  FRT_ERR_UNSUPPORTED (with the sizes in
 * frt_last_error) when the plan needs more scratch than the array holds:
 * 4*M*H per split-K partial plus 8*M*ceil(H/512) of slice sums (the five
 * FFN workloads of the benchmark fit).  All calls on one GPU share its
 * array: calls that overlap in time on one GPU (other streams, other plans,
 * other host threads) race; serialise them. */
frt_status frt_ffn_forward_range_static_scratch(frt_plan *plan, int32_t layer_begin, int32_t layer_end,
                                                void *stream);

/* Eager forward of the whole chain: frt_ffn_forward_range(plan, 0, L). */
frt_status frt_ffn_forward(frt_plan *plan, void *stream);

/* Capture the whole-chain forward on `stream` (not the null stream) in
 * relaxed stream-capture mode and instantiate it; replaces an earlier graph.
 * The scales and pointers in force are baked into the graph. */
frt_status frt_graph_capture(frt_plan *plan, void *stream);

/* Launch the captured graph on `stream`.  FRT_ERR_STATE if nothing was
 * captured ("No graph captured") or the graph is stale (weights or scales
 * changed after capture).  Asynchronous; the caller synchronises. */
frt_status frt_graph_replay(frt_plan *plan, void *stream);

/* Eager forward of the whole chain with a HIP event recorded on `stream`
 * before and after every kernel; writes each kernel's duration in
 * milliseconds to host_ms[L][3] = {norm+quantise, gate/up GEMM, down GEMM}
 * (with the norm fused into gate/up, the first entry times an empty slot;
 * with the split decode norm (M <= 16, the default there) the first entry
 * is the slice-sum kernel and the gate/up entry includes the quantisation;
 * with the whole-column down GEMV (M <= 4, the default there) the first
 * entry runs only in layer 0, later layers' R' and slice sums coming from
 * the previous down GEMV).
 * Same kernels and launch configuration as frt_ffn_forward.  Synchronises
 * `stream`.  For measuring per-kernel time inside a running program. */
frt_status frt_ffn_forward_profiled(frt_plan *plan, void *stream, float *host_ms);

/* Average duration in microseconds of one kernel kind (which: 0 norm +
 * quantise (the slice-sum kernel under the split decode norm; with the
 * whole-column down GEMV it runs in layer 0 only and the average is over
 * all layers), 1 gate/up GEMM (including the norm when fused, the
 * quantisation when split), 2 down GEMM (with the whole-column down GEMV,
 * also the next layer's residual add and slice sums)):
 * launches it for every layer, `reps` times, back to back on `stream`
 * between two HIP events (same kernels and launch configuration as the
 * forward).  The activation slots are left undefined (run the forward or
 * replay again before reading them).  Synchronises `stream`. */
frt_status frt_ffn_time_kernel(frt_plan *plan, int32_t which, int32_t reps, void *stream,
                               float *avg_us);

/* Device E4M3 quantiser as used by every kernel: out[i] = e4m3(in[i]) with
 * saturation to +-448 and round-to-nearest-even.  d_in device float[n],
 * d_out device uint8[n].  Asynchronous on `stream`.  For tests of the
 * conversion. */
frt_status frt_e4m3_encode_f32(const void *d_in, void *d_out, int64_t n, void *stream);

/* Thread-local description of the last failure on this thread ("" if none). */
const char *frt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FRT_FFN_H */
