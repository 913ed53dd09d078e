/*
 * qlora_nf4.h - C ABI of the QLoRA NF4 hot path on AMD Instinct MI355X (gfx950).
 *
 * The library implements, as hand-written HIP kernels, the data-parallel hot
 * path of QLoRA:
 *   - block-wise NF4 quantization of a frozen base weight with absmax scaling
 *     (QLoRA vs ChatGPT page, capability "NF4 4-bit quantization"; the NF4
 *     type has an exact zero and uses all 16 values: ai-papercheck review of
 *     the QLoRA paper, finding on paper p.5 Section 3),
 *   - double quantization of the absmax constants to 8 bits with their own
 *     scales (QLoRA vs ChatGPT page, capability "double quantization";
 *     Guanaco topic page, "Core Architecture & Training"),
 *   - dequantization, block by block,
 *   - the QLoRA linear layer: on-the-fly NF4 dequantization of the frozen
 *     base plus a full-precision low-rank adapter, forward and backward, with
 *     gradients only for the adapter and the input (QLoRA vs ChatGPT page,
 *     capability rows "LoRA on the quantized base" and "training pipeline").
 *
 * Conventions shared by every entry point
 *   Layout      Row-major, contiguous, no strides. W is [rows = N, cols = K]
 *               (out_features x in_features); X is [M, K]; Y and dY are
 *               [M, N]; A is [r, K]; B is [N, r].
 *   Pointers    Every tensor pointer is a DEVICE pointer owned by the caller.
 *               The qlora_nf4_weight struct itself lives in host memory; its
 *               members are device pointers. Device pointers must be 16-byte
 *               aligned (any hipMalloc / torch allocation is).
 *   Memory      The library allocates nothing. Scratch space is a caller-owned
 *               device workspace sized by the *_workspace_bytes queries.
 *   Streams     `stream` is a hipStream_t passed as void* (NULL = the default
 *               stream). Calls only enqueue work; no host synchronization.
 *   Outputs     Overwritten, never accumulated.
 *   Errors      Arguments are checked on the host before anything is
 *               launched; a failed check returns a negative qlora_status and
 *               launches nothing. A failed launch returns QLORA_ERR_HIP.
 *               qlora_last_error() gives a message for the calling thread.
 *   Finiteness  Inputs must be finite; NaN/Inf are not checked on the GPU.
 *   Threads     Entry points are thread-safe; calls on one stream run in
 *               order.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_NF4_BLOCK 64   /* weight elements per absmax constant          */
#define QLORA_DQ_BLOCK 256   /* absmax constants per double-quantization block */

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = -1,       /* a required pointer is NULL                    */
  QLORA_ERR_SHAPE = -2,      /* a size is out of range or inconsistent        */
  QLORA_ERR_DTYPE = -3,      /* dtype outside qlora_dtype or not allowed here */
  QLORA_ERR_WORKSPACE = -4,  /* workspace NULL or smaller than required       */
  QLORA_ERR_HIP = -5,        /* a HIP call or kernel launch failed            */
  QLORA_ERR_ALIGN = -6,      /* a device pointer is not 16-byte aligned       */
  QLORA_ERR_FORMAT = -7      /* a weight format outside qlora_format          */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;

/*
 * Weight formats: the levels and whether the absmax constants are
 * double-quantized. The default (0) is NF4 + DQ. The other three are the
 * comparison rows of the paper's Table 4 (QLoRA review, findings on paper p.8
 * Table 4: NFloat4, NFloat4 + DQ, Float4):
 *   bit 0 set: no double quantization, the fp32 absmax constants are stored;
 *   bit 1 set: FP4 levels, the 4-bit float with 1 sign, 2 exponent (bias 1,
 *              subnormal at exponent 0) and 1 mantissa bit, divided by its
 *              largest magnitude 6: 15 distinct levels ascending with 0 at
 *              index 7, and +1 repeated at index 15 (never produced).
 * Codes, blocks, packing and the nearest-level rule are the same for all.
 */
typedef enum {
  QLORA_FMT_NF4_DQ = 0,
  QLORA_FMT_NF4 = 1,
  QLORA_FMT_FP4_DQ = 2,
  QLORA_FMT_FP4 = 3
} qlora_format;

/*
 * 4-bit weight of `rows x cols` elements, n = rows*cols, flattened row-major,
 * in `format` (a qlora_format; 0 = NF4 + DQ, the layout described here).
 * nb = ceil(n/64) blocks, nd = ceil(nb/256) DQ blocks.
 *   codes     ceil(n/2) bytes; element 2j is the high nibble of byte j,
 *             element 2j+1 the low nibble; an odd n leaves the last low
 *             nibble 0. A code is the index of an NF4 level (0..15, ascending;
 *             7 is the exact 0.0 level).
 *   absmax_q  nb int8 codes in [-127, 127] of the block absmax constants.
 *   dq_scale  nd fp32: per DQ block, the largest |absmax - mean|.
 *   dq_mean   1 fp32 (device): the mean of the nb absmax constants.
 *   absmax    formats without DQ only: nb fp32 block absmax constants (then
 *             absmax_q, dq_scale and dq_mean are unused and may be NULL; with
 *             DQ, absmax is unused and may be NULL).
 * Reconstruction of element i in block b = i/64, DQ block d = b/256:
 *   k_d = fp32(dq_scale[d] / 127); c_b = fp32(fp32(absmax_q[b] * k_d) + mean);
 *   (without DQ: c_b = absmax[b])
 *   w_i = fp32(level[code_i] * c_b), all round-to-nearest-even, no FMA.
 * A zero-initialized struct with its buffers set is NF4 + DQ.
 */
typedef struct {
  int64_t rows, cols;
  uint8_t *codes;
  int8_t *absmax_q;
  float *dq_scale;
  float *dq_mean;
  float *absmax;
  int32_t format;
} qlora_nf4_weight;

/* Bytes of the stored format: ceil(n/2) + nb + 4*nd + 4. Returns 0 if
 * rows or cols <= 0. Host-only, touches no device. */
size_t qlora_nf4_storage_bytes(int64_t rows, int64_t cols);

/* The library's 16 NF4 levels (fp32, ascending) written to out[16]. The
 * levels are normal quantiles at equally spaced probabilities with an exact
 * zero, scaled to [-1, 1] (Guanaco topic page, "Technical Innovations:
 * NormalFloat4"; QLoRA review, finding on paper p.5 Section 3). Host-only.
 * Returns QLORA_OK or QLORA_ERR_NULL. */
int qlora_nf4_codebook(float *out);

/* Bytes of the stored format `format`: as qlora_nf4_storage_bytes with DQ,
 * ceil(n/2) + 4*nb without. Returns 0 for an invalid shape or format.
 * Host-only. */
size_t qlora_weight_storage_bytes(int64_t rows, int64_t cols, int format);

/* The 16 levels of `format` (fp32, ascending by code) written to out[16]
 * (NF4 as qlora_nf4_codebook, or the FP4 levels described at qlora_format).
 * Host-only. Returns QLORA_OK, QLORA_ERR_NULL or QLORA_ERR_FORMAT. */
int qlora_format_levels(int format, float *out);

/* Workspace bytes needed by qlora_nf4_quantize for this shape (0 if the shape
 * is invalid). Formats without DQ use no workspace. */
size_t qlora_nf4_quantize_workspace_bytes(int64_t rows, int64_t cols);

/*
 * Quantize W [rows, cols] (fp32 or bf16, device) into `out` in out->format
 * (NF4 + DQ by default), whose rows/cols must equal the arguments and whose
 * buffers for that format must be allocated by the caller with the sizes
 * given above.
 * Blocks of 64 consecutive flattened elements; absmax a_b = max|x|; each
 * element is coded as the level nearest to fp32(x / a_b) (ties to the lower
 * level; a zero block gets code 7 and a_b = 0). The constants a_b are then
 * double-quantized: mean over all nb constants (fp64 binary-tree sum,
 * adjacent pairs, leaves in index order, zero padded to a power of two, then
 * fp32(sum/nb)); per 256-block scale s = max|fp32(a - mean)|; code
 * q = clamp(rint(fp32(fp32((a - mean)/s) * 127)), -127, 127), 0 if s = 0.
 * (QLoRA vs ChatGPT page, capabilities "NF4 4-bit quantization" and "double
 * quantization".) Without DQ the fp32 a_b are stored as they are; with FP4
 * levels "level" means the FP4 table. Results are bit-identical to that
 * definition.
 * ws: device workspace of at least qlora_nf4_quantize_workspace_bytes() with
 * DQ; unused (may be NULL) without.
 */
int qlora_nf4_quantize(const void *W, int w_dtype, int64_t rows, int64_t cols,
                       const qlora_nf4_weight *out, void *ws, size_t ws_bytes,
                       void *stream);

/*
 * Dequantize `q` to out [rows, cols] (device) as fp32 (bit-exact
 * reconstruction above) or bf16 (round-to-nearest-even of that fp32).
 * Block-wise dequantization: QLoRA vs ChatGPT page, capability "training
 * pipeline". No workspace.
 */
int qlora_nf4_dequantize(const qlora_nf4_weight *q, void *out, int out_dtype, void *stream);

/* Workspace bytes needed by qlora_linear_fwd and qlora_linear_bwd for these
 * sizes (the larger of the two; 0 if the sizes are invalid).
 * The first QLORA_LINEAR_SYNC_BYTES of a linear workspace are
 * synchronization words (arrival counters and publication flags of the
 * single-launch skinny-M forward). They must be zero when the workspace is
 * first passed to the library (allocate it zero-filled, or clear it once);
 * every call returns them to zero by the time it completes, so a workspace
 * can be reused for any sizes and for both calls without clearing it again.
 * One workspace must not be used by two calls that run concurrently. */
#define QLORA_LINEAR_SYNC_BYTES (256 * 1024)
size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r);

/*
 * QLoRA linear forward (QLoRA vs ChatGPT page, capabilities "LoRA on the
 * quantized base" and "training pipeline"):
 *     Y = X W^T + scale * (X A^T) B^T
 * with W the 4-bit weight [N, K] (any qlora_format) dequantized block by
 * block on the fly.
 *   X      bf16 [M, K] (device)
 *   W      weight with rows = N, cols = K; N and K must be multiples
 *          of 64 and at most 2^23 (8388608): the large-tile kernels address
 *          a 256-row operand tile with 32-bit byte offsets
 *   A      fp32 [r, K], B fp32 [N, r] (device); r = 0 with A = B = NULL
 *          means no adapter; 0 <= r <= 256
 *   scale  the LoRA scale s (alpha / r in the usual convention)
 *   Y      bf16 [M, N] (device), overwritten
 * Products run on bf16 matrix cores with fp32 accumulation; A, B and the
 * adapter activations enter them rounded to bf16. For M > 32 the base enters
 * as bf16(w_i); for M <= 32 (the decode path) it enters as bf16(level) and
 * the fp32 block scale c_b multiplies each block's partial product. M >= 1.
 * When the 256 x 256 output tiles of M > 32 fill less than half of the GPU,
 * the reduction over K is split into fp32 partials in the workspace, summed
 * in a fixed order before the rounding to bf16 (results stay deterministic).
 * The decode path is one kernel launch; its workgroups exchange partial sums
 * through the workspace and wait for one another with bounded spins (see
 * QLORA_LINEAR_SYNC_BYTES for the workspace's leading words).
 */
int qlora_linear_fwd(const void *X, int64_t M, const qlora_nf4_weight *W,
                     const float *A, const float *B, int32_t r, float scale,
                     void *Y, void *ws, size_t ws_bytes, void *stream);

/*
 * QLoRA linear backward with the base frozen (gradients for the adapter
 * and the input only; QLoRA vs ChatGPT page, capability "training
 * pipeline"):
 *     dH = scale * dY B                  [M, r]
 *     dX = dY W + dH A                   bf16 [M, K]
 *     dA = dH^T X                        fp32 [r, K]
 *     dB = scale * dY^T (X A^T)          fp32 [N, r]
 * Arguments as in qlora_linear_fwd; dY is bf16 [M, N]. With r = 0, dA and
 * dB must be NULL and only dX is computed.
 */
int qlora_linear_bwd(const void *dY, const void *X, int64_t M, const qlora_nf4_weight *W,
                     const float *A, const float *B, int32_t r, float scale,
                     void *dX, float *dA, float *dB, void *ws, size_t ws_bytes,
                     void *stream);

/*
 * qlora_linear_fwd that also keeps the adapter activations for the backward,
 * as a training step saves its activations (QLoRA vs ChatGPT page,
 * capability "training pipeline"):
 *   Hs     bf16 [M, r] (device, 16-byte aligned, overwritten) = bf16(scale *
 *          X A^T), the rounded value the forward multiplies by B^T
 * r must be at least 1. Other arguments, results and errors as
 * qlora_linear_fwd (Y is bit-identical to its Y).
 */
int qlora_linear_fwd_save(const void *X, int64_t M, const qlora_nf4_weight *W,
                          const float *A, const float *B, int32_t r, float scale,
                          void *Y, void *Hs, void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_linear_bwd with the adapter activations Hs of qlora_linear_fwd_save
 * (same X, A and scale; bf16 [M, r], device, read only): the backward then
 * does not read X to form them again (X is still read for dA). Results as
 * qlora_linear_bwd up to the order of fp32 sums in H (the forward and the
 * backward split the reduction over K differently); with the Hs of the same
 * forward the call is deterministic. r must be at least 1.
 */
int qlora_linear_bwd_saved(const void *dY, const void *X, const void *Hs, int64_t M,
                           const qlora_nf4_weight *W, const float *A, const float *B,
                           int32_t r, float scale, void *dX, float *dA, float *dB,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The same kernels and results as
 * qlora_linear_fwd; the library uses a scratch array of 64 MiB in device
 * memory that each GPU holds from library load until the process ends, and
 * the call allocates nothing. Sizes whose forward needs more scratch than
 * that fail with QLORA_ERR_WORKSPACE before anything is launched (every
 * M <= 32 call of the 7B and 65B shapes fits, and M = 4096 at 4096 x 4096).
 * Where qlora_linear_fwd splits the GEMM's reduction into fp32 partials (few
 * output tiles, M up to about 2048) and they would not fit, this call runs
 * the reduction in one pass: Y then differs from qlora_linear_fwd's in the
 * order of the fp32 sums only.
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 * (two streams, two threads) race and must not be issued; calls ordered on
 * one stream are safe. Arguments and errors as qlora_linear_fwd.
 */
int qlora_linear_fwd_noalloc(const void *X, int64_t M, const qlora_nf4_weight *W,
                             const float *A, const float *B, int32_t r, float scale,
                             void *Y, void *stream);

/* Workspace bytes needed by qlora_nf4_merge (0 if the sizes are invalid). */
size_t qlora_nf4_merge_workspace_bytes(int64_t rows, int64_t cols, int32_t r);

/*
 * Merge a LoRA adapter into the quantized base and quantize the result again
 * (QLoRA vs ChatGPT page, capability on adapter composition: adapters are
 * merged into the base weights to give a standalone model):
 *     W'[n][k] = fp32(w-hat[n][k] + fp64(scale * sum_j B[n][j] A[j][k]))
 * with w-hat the fp32 dequantized W (any qlora_format), the rank sum in fp64
 * over j ascending (each fp32 product is exact in fp64), one fp64 multiply by
 * scale, one fp64 add and one rounding to fp32; then W' is quantized into
 * `out` exactly as qlora_nf4_quantize does, in out->format. Results are
 * bit-identical to that definition.
 *   W      the base, rows = N, cols = K (any shape the weight allows)
 *   A      fp32 [r, K], B fp32 [N, r] (device); r = 0 with A = B = NULL
 *          requantizes w-hat (for instance into another format); 0 <= r <= 256
 *   out    same rows/cols as W, any format, buffers allocated by the caller;
 *          it may be W itself (W is read completely before out is written)
 *   ws     device workspace of at least qlora_nf4_merge_workspace_bytes()
 * A weighted ensemble of adapters is one call with the adapters concatenated
 * along r and each weight folded into its columns of B.
 */
int qlora_nf4_merge(const qlora_nf4_weight *W, const float *A, const float *B, int32_t r,
                    float scale, const qlora_nf4_weight *out, void *ws, size_t ws_bytes,
                    void *stream);

/* AdamW hyperparameters and the step count t >= 1 of this update (the first
 * update is t = 1). The library forms the bias corrections
 * bc1 = fp32(1 - beta1^t) and bc2 = fp32(1 - beta2^t) from the fp32 betas,
 * the power and the difference in fp64, rounded once. */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int64_t step;
} qlora_adamw_hparams;

/* Workspace bytes of qlora_adamw_step: 0 with the state in device memory,
 * two staging arrays of up to 4 Mi floats each with the state on the host
 * (0 also if n is invalid). */
size_t qlora_adamw_workspace_bytes(int64_t n, int state_on_host);

/*
 * One AdamW step of n adapter parameters (Guanaco topic page, "Technical
 * Innovations: Paged Optimizers", and QLoRA vs ChatGPT page, capability on
 * paged optimizers: the optimizer state, momentum and variance, is paged
 * between GPU and host memory). Per element, all fp32, each operation
 * rounded to nearest even, no fused multiply-add (c1 = 1 - beta1 and
 * c2 = 1 - beta2 in fp32):
 *     m' = b1 m + c1 g,  v' = b2 v + c2 (g g)
 *     p' = p - lr ((m' / bc1) / (sqrt(v' / bc2) + eps) + wd p)
 * with bc1, bc2 the bias corrections of hp->step (see qlora_adamw_hparams).
 * Results are bit-identical to that definition wherever the state lives.
 *   param, grad   fp32 [n] (device); param and the state are updated in place
 *   m, v          fp32 [n]: device memory (state_on_host = 0) or pinned host
 *                 memory from hipHostMalloc (state_on_host = 1), which the
 *                 call pages through the workspace in chunks, copies ordered
 *                 on `stream`; the host arrays may be read again only after
 *                 the stream has reached this call's end
 *   ws            device workspace of qlora_adamw_workspace_bytes() bytes
 *                 (may be NULL when that is 0)
 * Errors: NULL pointers, n <= 0, misaligned pointers, step < 1, beta
 * outside [0, 1), eps < 0, a short workspace.
 */
int qlora_adamw_step(float *param, const float *grad, float *m, float *v, int64_t n,
                     const qlora_adamw_hparams *hp, int state_on_host, void *ws, size_t ws_bytes,
                     void *stream);

/*
 * Opt-in kernel timing for benchmarks. While enabled, each call records a
 * pair of HIP events on its stream around its dominant kernel:
 *   QLORA_PROF_FWD_GEMM     the fused dequant-GEMM of qlora_linear_fwd
 *   QLORA_PROF_BWD_DX       the transposed dequant-GEMM (dX) of qlora_linear_bwd
 *   QLORA_PROF_QUANTIZE     the absmax + NF4 code kernel of qlora_nf4_quantize
 *   QLORA_PROF_DEQUANTIZE   the kernel of qlora_nf4_dequantize
 * qlora_profile_read waits for the recorded events of `kind` and returns the
 * summed elapsed milliseconds and the number of launches; qlora_profile_reset
 * releases them. Not part of the method: instrumentation only.
 */
#define QLORA_PROF_FWD_GEMM 0
#define QLORA_PROF_BWD_DX 1
#define QLORA_PROF_QUANTIZE 2
#define QLORA_PROF_DEQUANTIZE 3
int qlora_profile_enable(int on);
int qlora_profile_read(int kind, double *total_ms, int64_t *launches);
int qlora_profile_reset(void);

/* Message for the last non-OK status returned on the calling thread
 * ("" if none). The pointer stays valid until the thread's next call. */
const char *qlora_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
