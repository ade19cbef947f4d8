/*
 * qlora.h -- C ABI of the MI355X (gfx950) NF4 + double-quantized frozen linear with a
 * 16-bit LoRA side path.
 *
 * The method (pages cited by title and section):
 *   - "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Quantization in one paragraph":
 *     absmax blocks of 64 weights, each weight stored as the index of the nearest of 16
 *     levels; dequantization is a lookup times the block constant.
 *   - "QLoRA: Quantize Base Weights to 4-Bit", Section 2 "1. 4-bit NormalFloat": the 16
 *     levels come from standard-normal quantiles; "2. Double Quantization": the FP32 block
 *     constants are re-quantized to 8-bit floats in groups of 256 with one FP32 constant
 *     per group, after subtracting their mean ("QLoRA -- Fine-Tuning a 65B Model on One
 *     GPU", "Double quantization: the constants are not free").
 *   - "QLoRA: Quantize Base Weights to 4-Bit", Section 3: weights are dequantized to BF16
 *     on chip for every matmul, and the adapter branch (alpha/r) B (A x) is added.
 *   - "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Where the gradients actually go":
 *     the input gradient runs through the dequantized weights; only A and B get gradients;
 *     the 4-bit tensor is never written.
 *
 * Conventions for every entry point:
 *   - Row-major.  W is [d_out, d_in] (h = W x), X is [M, d_in], Y is [M, d_out],
 *     A is [r, d_in], B is [d_out, r].  BF16 tensors are passed as uint16_t bit patterns.
 *   - "device" pointers are HIP device memory on the current device; "host" pointers are
 *     ordinary host memory.  The caller owns every buffer; the library never allocates
 *     device memory in fwd/bwd and never frees anything it was given.
 *   - Every call returns a status (0 = QLORA_OK, negative = error, see qlora_strerror).
 *     Arguments are validated before any launch; on an error nothing is launched.
 *     Work is enqueued on the caller's stream `stream` (0 = null stream).  Except where
 *     stated, calls do not synchronize, so device-side faults surface on the stream.
 *   - Workspaces.  The first QLORA_WS_COUNTER_BYTES bytes of every workspace hold the
 *     arrival counters of the split reductions (the last workgroup to finish a row group or
 *     column tile adds the partial results in a fixed order).  They must be zero before the
 *     workspace is first used: allocate it zero-filled, or call qlora_workspace_init once.
 *     Every call leaves them zero again, so one workspace serves any sequence of calls of
 *     any kind and shape, and calls captured in a HIP graph can be replayed.
 *   - Concurrency.  Calls that share a workspace must not overlap in time (e.g. run on two
 *     streams at once).  The library keeps no device state of its own, so calls with
 *     separate workspaces may overlap, on one device or several.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of arrival counters at the head of every workspace (512 KiB: one 32-bit word per
 * 64-column tile of dA and of dB, each dimension at most 2^22). */
#define QLORA_WS_COUNTER_BYTES ((size_t)524288)

/* Bytes of the fixed per-device scratch of qlora_linear_fwd_noalloc (16 MiB). */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)16777216)

enum qlora_status {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_ARG = -1, /* null or misaligned pointer, M outside [1, 2^24), r outside
                                 [1, 128], alpha not finite */
  QLORA_ERR_BAD_SHAPE = -2,   /* d_in % 64 != 0, d_out % 16 != 0, d_in or d_out > 2^22,
                                 d_out * d_in > 2^32 (32-bit buffer offsets) */
  QLORA_ERR_UNSUPPORTED = -3, /* block sizes other than (64, 256), unknown codebook or format */
  QLORA_ERR_NONFINITE = -4,   /* NaN or Inf in the weights given to qlora_quantize */
  QLORA_ERR_WORKSPACE = -5,   /* workspace pointer null or smaller than required */
  QLORA_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed */
  QLORA_ERR_SCRATCH = -7      /* the call needs more than the fixed scratch of the no-allocation
                                 entry point */
};

/* First-level codebooks: the 16 levels a 4-bit code indexes ("QLoRA: Quantize Base Weights
 * to 4-Bit", Section 2 "1. 4-bit NormalFloat", compares NF4 with standard INT4 and FP4). */
enum qlora_codebook {
  QLORA_CB_NF4 = 0,  /* NormalFloat: normal-quantile levels, exact 0 and +-1 (the method) */
  QLORA_CB_INT4 = 1, /* 16 evenly spaced levels -1 + 2i/15 (no zero level) */
  QLORA_CB_FP4 = 2   /* E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 over 6, both signs (15 levels) */
};

/* Second-level format of the block constants ("QLoRA: Quantize Base Weights to 4-Bit",
 * Section 2 "2. Double Quantization"; the pages call the 8-bit format both a float and an
 * integer, and give FP32 constants, 0.5 bits/param, as the case without it). */
enum qlora_dq_format {
  QLORA_DQ_E4M3 = 0, /* OCP FP8 E4M3, group constant max|d| / 448 (the method) */
  QLORA_DQ_E5M2 = 1, /* OCP FP8 E5M2, group constant max|d| / 57344 */
  QLORA_DQ_INT8 = 2, /* symmetric 8-bit integer, group constant max|d| / 127 */
  QLORA_DQ_NONE = 3  /* no double quantization: one FP32 constant per block in code8 */
};

/* A quantized weight tensor.  The struct and the buffers it points to belong to the
 * caller.  Sizes come from qlora_quant_sizes (or qlora_format_sizes for another second-level
 * format).  After qlora_quantize fills it, it is read-only to every other entry point.
 *
 *   codes : device uint8[d_out * d_in / 2].  4-bit level indices, row-major; each aligned
 *           run of 8 weights e0..e7 is 4 bytes, byte i = e_i | (e_{i+4} << 4).
 *   code8 : device uint8[d_out * d_in / 64].  One 8-bit code per block of 64 consecutive
 *           weights (the double-quantized, mean-shifted block constant; E4M3 by default).
 *           With QLORA_DQ_NONE: device float[d_out * d_in / 64], the constants themselves.
 *   c2s   : device float[ceil(n_blocks / 256)].  The FP32 second-level constant of each
 *           group of 256 consecutive blocks (flattened order).  Unused (may be NULL) with
 *           QLORA_DQ_NONE.
 *   mu    : device float[1].  The mean of all first-level constants of the tensor.  Unused
 *           (may be NULL) with QLORA_DQ_NONE.
 *   block1, block2 : must be 64 and 256.
 *   codebook  : an enum qlora_codebook value; 0, the default, is NF4.
 *   dq_format : an enum qlora_dq_format value; 0, the default, is E4M3.  The fused decode of the
 *           weight-streaming and mid-size kernels reads E4M3 only; other formats are decoded
 *           once per call into a BF16 copy at every token count (more workspace). */
typedef struct qlora_nf4dq {
  uint8_t *codes;
  uint8_t *code8;
  float *c2s;
  float *mu;
  int64_t d_out;
  int64_t d_in;
  int32_t block1;
  int32_t block2;
  int32_t codebook;
  int32_t dq_format;
} qlora_nf4dq_t;

/* Bytes of the three buffers of a [d_out, d_in] tensor (mu is always 4 bytes): 4 bits per
 * weight, one 8-bit constant per block of 64 and one FP32 constant per group of 256 blocks,
 * the 0.5 + 0.127 bits of overhead worked out on "QLoRA: Quantize Base Weights to 4-Bit",
 * Section 2 "2. Double Quantization" (and "QLoRA -- Fine-Tuning a 65B Model on One GPU",
 * "Double quantization: the constants are not free").
 * Host only.  Errors: INVALID_ARG (null outputs), BAD_SHAPE. */
int qlora_quant_sizes(int64_t d_out, int64_t d_in, size_t *codes_bytes, size_t *code8_bytes,
                      size_t *c2s_bytes);

/* The same for a given second-level format: with QLORA_DQ_NONE code8 holds 4 bytes per
 * block and there is no c2s.  Host only.  Errors: as above, UNSUPPORTED (unknown format). */
int qlora_format_sizes(int64_t d_out, int64_t d_in, int dq_format, size_t *codes_bytes,
                       size_t *code8_bytes, size_t *c2s_bytes);

/* Workspace bytes needed by one call of `op` (QLORA_OP_*) at these sizes, for E4M3
 * constants (qlora_workspace_size) or the given second-level format.  The count includes the
 * QLORA_WS_COUNTER_BYTES head.  Host only.
 * Errors: INVALID_ARG (null output, unknown op, M or r out of range), BAD_SHAPE, UNSUPPORTED. */
enum qlora_op { QLORA_OP_QUANTIZE = 0, QLORA_OP_FWD = 1, QLORA_OP_BWD = 2 };
int qlora_workspace_size(int op, int64_t M, int64_t d_out, int64_t d_in, int32_t r,
                         size_t *ws_bytes);
int qlora_workspace_size_fmt(int op, int64_t M, int64_t d_out, int64_t d_in, int32_t r,
                             int dq_format, size_t *ws_bytes);

/* Zero the counter head of a workspace (device memory of ws_bytes >= QLORA_WS_COUNTER_BYTES
 * bytes) on `stream`, so it is ready for its first use; the rest is left as it is.  Needed
 * once per workspace unless it was allocated zero-filled.  Uses a fill kernel, not a memset,
 * so it may also be captured in a HIP graph.  No synchronization.
 * Errors: INVALID_ARG (null pointer), WORKSPACE (ws_bytes too small), HIP. */
int qlora_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* The FP32 NF4 table the library uses (host memory, 16 floats), built from the
 * normal-quantile formula of "QLoRA: Quantize Base Weights to 4-Bit", Section 2
 * "1. 4-bit NormalFloat", with the tail level at Q(1/34) and each side scaled to its
 * extreme so the endpoints are exactly -1 and +1 ("QLoRA -- Fine-Tuning a 65B Model on
 * One GPU", "NF4"). */
int qlora_nf4_codebook(float out16[16]);

/* The FP32 levels of any first-level codebook (QLORA_CB_*), host memory, 16 floats.
 * Errors: INVALID_ARG (null output or unknown codebook). */
int qlora_codebook(int codebook, float out16[16]);

/* Quantize FP32 weights W (device, [d_out, d_in], d_in % 64 == 0) into *Wq, whose
 * buffers the caller allocated ("QLoRA -- Fine-Tuning a 65B Model on One GPU", "Quantization
 * in one paragraph" for the absmax blocks and the nearest level, "NF4" for the table;
 * "QLoRA: Quantize Base Weights to 4-Bit", Section 2 "2. Double Quantization" for the
 * second level).  First level: c1 = max|w| per 64-block, code = nearest
 * level of Wq->codebook to fl32(w / c1), ties to the lower level; an all-zero block gets
 * the level nearest 0 (the zero level of NF4).
 * Double quantization: mu = FP32 of the exact mean of all c1; d = fl32(c1 - mu); per group
 * of 256 blocks c2s = fl32(max|d| / 448) and code8 = E4M3(fl32(d / c2s)) rounded to
 * nearest, ties to even (0 when c2s == 0).  Other second-level formats use 57344 and E5M2,
 * or 127 and a round-half-even integer; QLORA_DQ_NONE stores c1 in code8 (mu not written).
 * ws: device, qlora_workspace_size(QLORA_OP_QUANTIZE) bytes.  host_mu: host float, may be
 * NULL.  SYNCHRONIZES `stream` once (to fold the exact mean on the host).
 * Errors: INVALID_ARG, BAD_SHAPE, UNSUPPORTED, NONFINITE (then Wq's contents are
 * unspecified), WORKSPACE, HIP. */
int qlora_quantize(const float *W, const qlora_nf4dq_t *Wq, float *host_mu, void *ws,
                   size_t ws_bytes, hipStream_t stream);

/* Quantize BF16 weights (device uint16 bit patterns [d_out, d_in]): the same steps as
 * qlora_quantize applied to their exact FP32 values.  A 16-bit checkpoint is quantized as
 * it stands ("QLoRA: Quantize Base Weights to 4-Bit", Section 1: the frozen base otherwise
 * sits in memory in 16-bit precision), and so is a merged export from qlora_merge when a
 * 4-bit copy of it is wanted ("QLoRA -- Fine-Tuning a 65B Model on One GPU", "Pitfalls":
 * merge in 16 bits, then quantize the merged result).  Same buffers, workspace, single
 * synchronization and errors as qlora_quantize; W must be 16-byte aligned. */
int qlora_quantize_bf16(const uint16_t *W, const qlora_nf4dq_t *Wq, float *host_mu, void *ws,
                        size_t ws_bytes, hipStream_t stream);

/* Dequantize to BF16 (device uint16[d_out, d_in]), bit-exact:
 *   c1_hat = fl32(fl32(E4M3(code8) * c2s) + mu),  w_hat = bf16_rne(fl32(q[code] * c1_hat)).
 * A lookup times the recovered block constant ("QLoRA -- Fine-Tuning a 65B Model on One
 * GPU", "Quantization in one paragraph"), after undoing the second level ("QLoRA: Quantize
 * Base Weights to 4-Bit", Section 2 "2. Double Quantization"), rounded to the BF16 compute
 * type (same page, Section 3).  For export and tests; the linear entry points decode as part
 * of their own kernels.
 * Errors: INVALID_ARG, BAD_SHAPE, UNSUPPORTED, HIP. */
int qlora_dequantize(const qlora_nf4dq_t *Wq, uint16_t *W_bf16, hipStream_t stream);

/* Merged export: W_out = bf16_rne(fl32(w_hat + s * (B A))), s = fl32(alpha / r), with
 * w_hat the bit-exact dequantized base (as qlora_dequantize) and B A summed in FP32 from
 * the BF16 adapters ("QLoRA: Quantize Base Weights to 4-Bit", "Interview questions": the
 * base is dequantized to 16 bits and the adapter folded in, W = W_dequant + (alpha/r) B A,
 * for a 16-bit checkpoint with no adapter left at inference; "QLoRA -- Fine-Tuning a 65B
 * Model on One GPU", "Pitfalls": the fold is done in 16 bits, not inside the 4-bit format).
 *   A [r, d_in], B [d_out, r]: device BF16 adapters (A 16-byte aligned; B too when r % 8 == 0).
 *   W_out [d_out, d_in]: device BF16, overwritten; 16-byte aligned.
 * The quantized weight is only read; to re-quantize, pass W_out to qlora_quantize_bf16.
 * No workspace, no synchronization.  Errors: INVALID_ARG (null or misaligned pointer, r
 * outside [1, 128], alpha not finite), BAD_SHAPE, UNSUPPORTED, HIP. */
int qlora_merge(const qlora_nf4dq_t *Wq, const uint16_t *A, const uint16_t *B, int32_t r,
                float alpha, uint16_t *W_out, hipStream_t stream);

/* Forward: Y = X w_hat^T + (alpha / r) T B^T with T = X A^T, FP32 accumulation, BF16 out
 * ("QLoRA: Quantize Base Weights to 4-Bit", Section 3; "QLoRA -- Fine-Tuning a 65B Model
 * on One GPU", "Where the gradients actually go").
 *   X [M, d_in], A [r, d_in], B [d_out, r]: device BF16 inputs.
 *   Y [M, d_out]: device BF16 output (overwritten).
 *   T_save [M, r]: device BF16, receives bf16(T) for the backward; may be NULL.
 *   ws: device workspace of qlora_workspace_size(QLORA_OP_FWD) bytes.
 * M <= 16 runs one weight-streaming launch that decodes the 4-bit codes on chip; 16 < M <
 * 1024 runs the fused GEMM that decodes each weight tile on chip; M >= 1024 (and any M for
 * second-level formats other than E4M3) first decodes the weight once into a BF16 copy in the
 * workspace (2 d_out d_in bytes), then runs a plain BF16 MFMA GEMM over it.
 * Errors: INVALID_ARG, BAD_SHAPE, UNSUPPORTED, WORKSPACE, HIP. */
int qlora_linear_fwd(const qlora_nf4dq_t *Wq, const uint16_t *X, int64_t M, const uint16_t *A,
                     const uint16_t *B, int32_t r, float alpha, uint16_t *Y, uint16_t *T_save,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* qlora_linear_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments, results and
 * errors as qlora_linear_fwd, minus the workspace: the call uses a fixed array of
 * QLORA_NOALLOC_SCRATCH_BYTES that the library holds on each device until the process ends,
 * and calls no hipMalloc, hipFree or other allocating routine (diagnostic timing events are
 * not recorded for its launches).
 *   Limit: calls whose workspace need (qlora_workspace_size_fmt, QLORA_OP_FWD) exceeds that
 *   size return QLORA_ERR_SCRATCH before any launch.  That admits every M < 1024 at the
 *   workload shapes (at most 12 MiB, 8192 x 28672 at M = 16); M >= 1024 needs the decoded
 *   weight copy and is refused except for small weights.
 *   Set-up: the first call on a device (with that device current) looks the array up and
 *   zeroes its counter head on `stream`; make that first call outside graph capture.
 *   Concurrency: every call on a device shares that device's array, which keeps the last
 *   call's contents (the counter head is left zero), so calls that overlap on one device
 *   race; serialize them (one stream, or events).
 * Errors: as qlora_linear_fwd, SCRATCH instead of WORKSPACE. */
int qlora_linear_fwd_noalloc(const qlora_nf4dq_t *Wq, const uint16_t *X, int64_t M,
                             const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                             uint16_t *Y, uint16_t *T_save, hipStream_t stream);

/* The forward of several linears that read the same input, e.g. the q, k and v projections or
 * the gate and up projections of a decoder layer: for i < count,
 *   Y[i] = X w_hat_i^T + (alpha / r) (X A[i]^T) B[i]^T      (as qlora_linear_fwd)
 *   Wq: host array of count (1..4) weight descriptors, all with the same d_in.
 *   A, B, Y: host arrays of count device pointers (A[i] [r, d_in], B[i] [d_out_i, r], Y[i]
 *            [M, d_out_i], BF16).  T_save: host array of count device pointers (each may be
 *            NULL) or NULL.  X [M, d_in], r and alpha are shared.
 *   ws: device workspace of qlora_workspace_size_multi() bytes.
 * For M <= 16 with E4M3 constants, one codebook, every d_out a multiple of 256 and at least 32M
 * weights in all, the linears run as one weight-streaming launch (start-up and split-K
 * hand-off paid once for the group); otherwise this is count calls of qlora_linear_fwd in
 * order, on the same workspace.  Results match qlora_linear_fwd within its rounding (the
 * reduction split can differ).  Errors: as qlora_linear_fwd; BAD_SHAPE when d_in differs. */
int qlora_workspace_size_multi(int count, const qlora_nf4dq_t *const *Wq, int64_t M, int32_t r,
                               size_t *ws_bytes);
int qlora_linear_fwd_multi(int count, const qlora_nf4dq_t *const *Wq, const uint16_t *X, int64_t M,
                           const uint16_t *const *A, const uint16_t *const *B, int32_t r, float alpha,
                           uint16_t *const *Y, uint16_t *const *T_save, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* The MLP block of a decoder layer with all three projections stored NF4 + DQ and adapted
 * ("QLoRA -- Fine-Tuning a 65B Model on One GPU", "Seeing it in code": adapters on every
 * linear, gate_proj / up_proj / down_proj among them; gradient checkpointing on, as "QLoRA:
 * Quantize Base Weights to 4-Bit", "In production", also asks).  The pages name the three
 * projections but not the activation between them; the one those names denote is used:
 *   G = gate(X), U = up(X)          (one qlora_linear_fwd_multi call: a single launch at M <= 16)
 *   H = bf16(silu(G) * U),  silu(g) = g / (1 + e^-g)   (FP32 from the BF16 G, U)
 *   Y = down(H)
 *   Wg, Wu: [f, d]; Wd: [d, f]; X [M, d], Y [M, d]: device BF16.
 *   A, B: host arrays of 3 device pointers in the order gate, up, down (A[i] [r, d_in_i],
 *         B[i] [d_out_i, r]); r and alpha shared.
 *   G_save, U_save: device BF16 [M, f] that receive G and U for the backward, or NULL.
 *   ws: device workspace of qlora_mlp_workspace_size(QLORA_OP_FWD or QLORA_OP_BWD) bytes.
 * The backward takes dY [M, d] and returns dX [M, d] (the sum of the input gradients through
 * gate and up, added in FP32 and rounded once more), and dA[i], dB[i] (host arrays of 3
 * device pointers, gate, up, down), as qlora_linear_bwd does per projection.  With
 * G_saved = U_saved = NULL it recomputes G and U from X (checkpointing); H is always
 * recomputed.  Errors: as qlora_linear_fwd / bwd; BAD_SHAPE when the shapes do not chain. */
int qlora_mlp_workspace_size(int op, int64_t M, const qlora_nf4dq_t *Wg, const qlora_nf4dq_t *Wu,
                             const qlora_nf4dq_t *Wd, int32_t r, size_t *ws_bytes);
int qlora_mlp_fwd(const qlora_nf4dq_t *Wg, const qlora_nf4dq_t *Wu, const qlora_nf4dq_t *Wd,
                  const uint16_t *X, int64_t M, const uint16_t *const *A, const uint16_t *const *B,
                  int32_t r, float alpha, uint16_t *Y, uint16_t *G_save, uint16_t *U_save, void *ws,
                  size_t ws_bytes, hipStream_t stream);
int qlora_mlp_bwd(const qlora_nf4dq_t *Wg, const qlora_nf4dq_t *Wu, const qlora_nf4dq_t *Wd,
                  const uint16_t *X, const uint16_t *dY, int64_t M, const uint16_t *const *A,
                  const uint16_t *const *B, int32_t r, float alpha, const uint16_t *G_saved,
                  const uint16_t *U_saved, uint16_t *dX, uint16_t *const *dA, uint16_t *const *dB,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/* Backward of qlora_linear_fwd ("QLoRA -- Fine-Tuning a 65B Model on One GPU", "Where the
 * gradients actually go": the input gradient flows through the dequantized weights, only A
 * and B receive gradients, the 4-bit tensor is never written).  With G = dY B:
 *   dX = dY w_hat + (alpha/r) G A      [M, d_in]   (may be NULL: not computed)
 *   dA = (alpha/r) G^T X               [r, d_in]
 *   dB = (alpha/r) dY^T T, T = X A^T   [d_out, r]
 * dY [M, d_out], X, A, B: device BF16 inputs.  T_saved: device BF16 [M, r] from the
 * forward, or NULL to recompute it.  Outputs are device BF16 and overwritten (not
 * accumulated).  The quantized weights are only read.  dX runs as the forward does: the
 * fused transposed-tile GEMM below 1024 tokens, else the transposed BF16 copy in the
 * workspace and the plain BF16 GEMM.
 * Errors: INVALID_ARG, BAD_SHAPE, UNSUPPORTED, WORKSPACE, HIP. */
int qlora_linear_bwd(const qlora_nf4dq_t *Wq, const uint16_t *X, const uint16_t *dY, int64_t M,
                     const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                     const uint16_t *T_saved, uint16_t *dX, uint16_t *dA, uint16_t *dB, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/* One AdamW step over a flat array of n trainable adapter parameters (all of a model's A
 * and B laid end to end, so one call updates them all).  The pages keep, per trainable
 * parameter, an FP32 master weight and FP32 first and second moments (12 bytes) beside the
 * 16-bit weight and 16-bit gradient ("QLoRA: Quantize Base Weights to 4-Bit", Section 1 and
 * Section 4's optimizer term; "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Paged
 * optimizers"); the update is the published AdamW with decoupled, lr-scaled decay:
 *   theta *= 1 - lr*wd;  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   theta -= lr/(1-b1^step) * m / (sqrt(v)/sqrt(1-b2^step) + eps);  param = bf16_rne(theta)
 *   master, m, v : device float[n], updated in place, 16-byte aligned.
 *   grad         : device BF16[n] (e.g. the dA / dB written by qlora_linear_bwd into slices
 *                  of one flat buffer), 8-byte aligned.
 *   param        : device BF16[n] working copy, overwritten; may be NULL; 8-byte aligned.
 *   step         : 1 for the first step (bias correction).
 * Paging of the states to host memory is not done.  n == 0 is a no-op.
 * Errors: INVALID_ARG (n < 0, step < 1, null or misaligned pointer, lr < 0, beta outside
 * [0, 1), eps <= 0, weight_decay < 0, a non-finite scalar), HIP. */
int qlora_adamw_step(float *master, float *m, float *v, const uint16_t *grad, uint16_t *param,
                     int64_t n, int64_t step, float lr, float beta1, float beta2, float eps,
                     float weight_decay, hipStream_t stream);

/* Diagnostic: the device E4M3 encoder used by qlora_quantize, applied elementwise to n
 * floats (device in, device out), so it can be checked exhaustively.  |in| <= 448 is
 * rounded to nearest, ties to even; larger magnitudes go to 448.  Errors: INVALID_ARG, HIP. */
int qlora_e4m3_encode(const float *in, uint8_t *out, int64_t n, hipStream_t stream);

/* Diagnostic kernel timing.  While enabled, the library brackets every launch of the
 * selected kernels below with a pair of hipEvents recorded on the launch stream.
 * qlora_timing_enable takes a bit mask over the kernel ids (bit i selects id i; 0 turns
 * timing off); launches of unselected kernels carry no events.  qlora_timing_read waits
 * for the events of one kernel id and returns their summed duration (ms) and the launch
 * count since the last read, then resets that id.  Host only; events are created by the
 * library and reused.  Errors: INVALID_ARG (bad id or null output), HIP. */
enum qlora_kernel_id {
  QLORA_K_QUANT_PASS1 = 0, /* quantize: codes, first-level constants, exponent sums */
  QLORA_K_QUANT_PASS2 = 1, /* quantize: 8-bit constant codes and their scales */
  QLORA_K_DEQUANT = 2,     /* BF16 w_hat (standalone, and the forward copy for M >= 1024) */
  QLORA_K_GEMV_FWD = 3,    /* forward, M <= 16 */
  QLORA_K_GEMM_FWD = 4,    /* forward GEMM, M > 16 */
  QLORA_K_GEMM_DX = 5,     /* dX GEMM */
  QLORA_K_LORA_DOWN = 6,   /* T = X A^T and G = dY B */
  QLORA_K_LORA_GRAD = 7,   /* dA and dB */
  QLORA_K_DEQUANT_T = 8,   /* BF16 w_hat^T, the dX copy for M >= 1024 */
  QLORA_K_MERGE = 9,       /* merged export w_hat + s B A */
  QLORA_K_ADAMW = 10,      /* adapter optimizer step */
  QLORA_K_COUNT = 11
};
int qlora_timing_enable(int kernel_mask);
int qlora_timing_read(int kernel_id, double *total_ms, int64_t *launches);

/* Human-readable text of a status code (static storage). */
const char *qlora_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
