/*
 * convrot.h -- C ABI of libconvrot.so, the ConvRot W8A8 rotated-INT8 linear layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (sources cited by page title and section):
 *   - "LoRA Training Guide for MOSS-Image", section 7.1 "VRAM Usage Optimization",
 *     subsection "ConvRot INT8": frozen base weights are rotated by a
 *     block-diagonal Hadamard matrix and quantized per channel (per output row) to
 *     int8; the forward rotates the activations online, quantizes them row-wise on
 *     the fly, runs the int8 matmul and dequantizes; the input gradient goes either
 *     through a transient bf16 dequantization (default) or through the int8 GEMM.
 *   - sd-scripts pull request 2461 (MOSS-Image ConvRot INT8), Summary, kernels and
 *     utils bullets: block-diagonal Hadamard rotation, row-wise int8 quantization,
 *     fused int8 GEMM with online rotation + dynamic per-row quantization +
 *     dequantization epilogue; frozen base whose backward returns grad_x only;
 *     row-chunked quantization of the token embedding and a quantized embedding
 *     whose lookup dequantizes the rows and applies the inverse rotation.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to caller-owned memory, row-major and
 *     contiguous, 16-byte aligned (the lookup's oob_count: 4-byte aligned), bias
 *     included when given; a misaligned pointer is CONVROT_EINVAL.  bf16 values
 *     are passed as uint16_t bit patterns.  Scales are fp32 and are never cast.
 *   - Size limits: every row, column, token or id count is at most 2^31 - 1 and
 *     every tensor holds at most 2^40 elements (CONVROT_ESHAPE otherwise).
 *   - The rotation R = diag(H_128 / sqrt(128)) acts along the contraction axis;
 *     H_128 is the Sylvester Hadamard matrix in natural order.  block must be 128;
 *     the contraction length (K, or D for the embedding) must be a multiple of 128.
 *   - Work is enqueued on `stream` in stream order; no entry point synchronizes the
 *     host, allocates memory, or keeps a pointer after it returns.  Calls on
 *     different streams that share output buffers race.
 *   - Outputs must not alias inputs.
 *   - The batch size may be 0 (M rows of activations or gradients, the rows of a
 *     weight, T ids): the call then checks its other sizes, enqueues nothing and
 *     returns CONVROT_OK without reading any pointer (they may be NULL).  Every
 *     other size must be positive.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     argument error (CONVROT_EINVAL, _ESHAPE, _EWORKSPACE, _EDEVICE) nothing is
 *     launched.  CONVROT_EHIP reports a failed HIP call or launch; launches of
 *     the same call made before it (e.g. earlier row chunks) stay enqueued, and
 *     the outputs are then undefined.  Faults inside kernels surface
 *     asynchronously on the stream, as for any HIP launch.
 */
#ifndef CONVROT_H_
#define CONVROT_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define CONVROT_OK 0
#define CONVROT_EINVAL (-1)     /* null pointer, negative or zero size, misaligned pointer */
#define CONVROT_ESHAPE (-2)     /* block != 128, K or D not a multiple of 128, size over a limit */
#define CONVROT_EWORKSPACE (-3) /* workspace too small */
#define CONVROT_EHIP (-4)       /* a HIP call or launch failed */
#define CONVROT_EDEVICE (-5)    /* current device is not gfx950 */
#define CONVROT_ESCRATCH (-6)   /* the call needs more than the allocation-free scratch */

/* Backward modes of convrot_linear_bwd_dx. */
#define CONVROT_BWD_BF16 0 /* transient bf16 dequantization, then a bf16 GEMM */
#define CONVROT_BWD_INT8 1 /* per-row int8 quantization of dY (s_w folded in), int8 GEMM */

/* Operations for convrot_workspace_bytes. */
#define CONVROT_OP_LINEAR_FWD 0
#define CONVROT_OP_LINEAR_BWD_DX 1
#define CONVROT_OP_LINEAR_FWD_LORA 2  /* mode = LoRA rank */

/* Largest supported contraction length of the row quantizer (32768 = 256 blocks). */
#define CONVROT_MAX_ROW_LEN 32768

/*
 * Load-time weight quantization ("ConvRot INT8" in the training guide section 7.1;
 * row-wise quantization and row-chunked embedding quantization in the pull
 * request's Summary).  For every row of w [rows, cols]: rotate r = w_row * R
 * (r = fl32(fl64(sum) * c), c = 1/sqrt(128) in fp64; the binary64 sum is exact
 * while a 128-block's magnitude spread stays under about 2^38),
 * a = max |r|, scale = fl32(a / 127), codes = round-half-even(fl32(r / scale))
 * clamped to [-127, 127].  A row whose scale is 0 (all zero, or a maximum below
 * 127 * 2^-150, where a / 127 underflows) gets codes 0.  A row with a NaN or
 * infinite r (a non-finite input, or an fp32 overflow of the rotated value) gets
 * scale NaN (0x7fc00000) and codes 0, so it dequantizes to NaN; the forward's
 * activation quantizer and the int8 input gradient's dY quantizer apply the
 * same rules per row.
 *   w      bf16 [rows, cols], cols % 128 == 0, cols <= CONVROT_MAX_ROW_LEN
 *   block  must be 128
 *   chunk_rows  rows per launch (0 = all rows at once); results do not depend on it
 *   q      int8 [rows, cols] out;  scale fp32 [rows] out
 */
int convrot_quantize_weight(const uint16_t* w, int64_t rows, int64_t cols, int32_t block,
                            int64_t chunk_rows, int8_t* q, float* scale, hipStream_t stream);

/*
 * Forward of the ConvRot linear (the fused int8 GEMM of the pull request's
 * Summary): y = bf16( fl32(acc) * s_x[m] * s_w[n] (+ bias[n]) ), evaluated in fp32 as
 * (fl32(acc) * s_w[n]) * s_x[m] (the frozen weight's scale first, so that no
 * activation scale makes an intermediate overflow where y does not), with
 * acc[m][n] = sum_k q_x[m][k] * q_w[n][k] (int32, exact), where (q_x, s_x) is the
 * rotated per-row quantization of x computed on the fly.  Since R is orthogonal,
 * y approximates x * W^T in the unrotated basis.
 *   x     bf16 [M, K] (activations keep their own dtype; never cast to int8)
 *   qw    int8 [N, K], sw fp32 [N]  (from convrot_quantize_weight)
 *   bias  bf16 [N] or NULL
 *   y     bf16 [M, N] out
 *   workspace  >= convrot_workspace_bytes(CONVROT_OP_LINEAR_FWD, M, N, K, 0) bytes
 *              of device memory, 256-byte aligned: q_x and s_x, plus int32 partial
 *              sums when the contraction is split along K (few 256 x 256 output
 *              tiles, or more than 32 rows at K = 8192 on the few-row path).
 *              Which kernels run depends on M, N and K (one tiled GEMM, a
 *              few-row kernel for M <= 128 or for N <= 128, or a split along K);
 *              y is the same bit for bit on every path.  For at most
 *              8 / ceil(K / 2048) rows (K <= 8192, N <= 8192) the forward is one
 *              launch that keeps q_x and s_x on chip and leaves the workspace
 *              untouched; its contents after a call are unspecified either way.
 */
int convrot_linear_fwd(const uint16_t* x, int64_t M, int64_t K, const int8_t* qw,
                       const float* sw, int64_t N, const uint16_t* bias, uint16_t* y,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory or
 * hand over a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same computation, kernels and result as
 * convrot_linear_fwd (bit for bit), with q_x, s_x and any split-K partials held
 * in a static device array of the library instead of a workspace.
 *   - The array holds CONVROT_NOALLOC_SCRATCH_BYTES (96 MiB) on each GPU the
 *     library runs on, from the first call on that GPU until the process ends.
 *     A call needing more (convrot_workspace_bytes(CONVROT_OP_LINEAR_FWD, M, N,
 *     K, 0) > CONVROT_NOALLOC_SCRATCH_BYTES; e.g. M * K above ~100 M) returns
 *     CONVROT_ESCRATCH and enqueues nothing.
 *   - Every call on a GPU shares that GPU's array: calls that overlap in time
 *     on one GPU (different streams, or host threads) race and give undefined
 *     outputs.  Calls in one stream are ordered and safe.
 *   - The call itself allocates nothing; on the first call on a device it looks
 *     up the array's device address (hipGetSymbolAddress) and keeps it.
 * Other arguments, errors and ownership as convrot_linear_fwd.
 */
#define CONVROT_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int convrot_linear_fwd_noalloc(const uint16_t* x, int64_t M, int64_t K, const int8_t* qw,
                               const float* sw, int64_t N, const uint16_t* bias, uint16_t* y,
                               hipStream_t stream);

/*
 * Forward with a LoRA branch.  The quantized layers stay LoRA-trainable and the
 * LoRA branch receives the unrotated input (training guide section 7.1, ConvRot
 * INT8 scope bullet):
 *   xa = bf16( x * A^T )                       (as a bf16 Linear; fp32 accumulation)
 *   y  = bf16( fl32(acc) * s_x[m] * s_w[n] (+ bias[n]) + lora_scale * (xa[m] . B[n]) ),
 *        the product evaluated as in convrot_linear_fwd
 * with the base terms exactly as in convrot_linear_fwd and the LoRA term added in
 * fp32 before the single bf16 rounding.
 *   lora_a  bf16 [R, K] (down projection);  lora_b bf16 [N, R] (up projection)
 *   R       16 or 32 (otherwise CONVROT_ESHAPE)
 *   lora_scale  multiplier * alpha / R, applied to the up projection
 *   workspace  >= convrot_workspace_bytes(CONVROT_OP_LINEAR_FWD_LORA, M, N, K, R)
 * Other arguments, errors and ownership as convrot_linear_fwd.
 */
int convrot_linear_fwd_lora(const uint16_t* x, int64_t M, int64_t K, const int8_t* qw,
                            const float* sw, int64_t N, const uint16_t* bias,
                            const uint16_t* lora_a, const uint16_t* lora_b, int32_t R,
                            float lora_scale, uint16_t* y, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Input gradient of the frozen base (the pull request's utils bullet: only
 * grad_x, bf16 transient dequant or the int8 GEMM; the guide's section 7.1 flag
 * description).  dX approximates dY * W_hat, W_hat = (s_w * q_w) * R.
 *   mode CONVROT_BWD_BF16: W_hat^T is materialized in bf16 in the workspace, then a
 *        bf16 MFMA GEMM with fp32 accumulation.
 *   mode CONVROT_BWD_INT8: g = fl32(dY) * s_w[n] (fp32), per-row int8 quantization
 *        of g (no rotation) -> (q_g, s_g); acc2[m][k] = sum_n q_g[m][n] q_w[n][k];
 *        dX = bf16( inverse-rotate( fl32(acc2) * s_g[m] ) ).
 *   dy  bf16 [M, N];  qw int8 [N, K];  sw fp32 [N];  dx bf16 [M, K] out
 *   workspace  >= convrot_workspace_bytes(CONVROT_OP_LINEAR_BWD_DX, M, N, K, mode)
 */
int convrot_linear_bwd_dx(const uint16_t* dy, int64_t M, int64_t N, const int8_t* qw,
                          const float* sw, int64_t K, int32_t mode, uint16_t* dx,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Quantized embedding lookup (the pull request's utils bullet: rows stored in the
 * rotated basis; the lookup dequantizes and applies the inverse rotation):
 * out[t] = bf16( (s_E[id] * q_E[id]) * R ).  An id outside [0, V) produces a zero
 * row and, if oob_count is non-NULL, atomically increments *oob_count (device
 * int32, 4-byte aligned, not cleared by the call).
 *   ids int32 [T];  qe int8 [V, D];  se fp32 [V];  out bf16 [T, D]; D % 128 == 0
 */
int convrot_embedding_lookup(const int32_t* ids, int64_t T, const int8_t* qe, const float* se,
                             int64_t V, int64_t D, uint16_t* out, int32_t* oob_count,
                             hipStream_t stream);

/* Workspace bytes needed by an operation (0 on invalid sizes or sizes over the
 * limits, and for an empty batch, which needs none). */
size_t convrot_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t mode);

/* Human-readable text of a status code (static storage). */
const char* convrot_status_string(int status);

/* ---------------------------------------------------------------------------
 * Building blocks of the entry points above, exported so that tests can check the
 * exact intermediates (codes, scales, int32 accumulators) and benchmarks can time
 * each kernel.  Same kernels as the composite calls.
 * ------------------------------------------------------------------------- */

/* Activation rotation + dynamic per-row quantization (first stage of the
 * forward; same arithmetic as convrot_quantize_weight). */
int convrot_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* qx, float* sx,
                         hipStream_t stream);

/* int8 GEMM with the dequantizing epilogue (second stage of the forward):
 * y = bf16( fl32(sum_k qx[m][k] qw[n][k]) * sx[m] * sw[n] (+ bias[n]) ). */
int convrot_gemm_i8_bf16(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw,
                         int64_t M, int64_t N, int64_t K, const uint16_t* bias, uint16_t* y,
                         hipStream_t stream);

/* Raw int32 contraction.  b_layout 0: acc[m][n] = sum_k a[m][k] b[n][k] with
 * a [M, K], b [N, K] (forward).  b_layout 1: acc[m][n] = sum_k a[m][k] b[k][n] with
 * a [M, K], b [K, N] (contraction along the rows of b, as in the int8 input
 * gradient; K % 128 == 0 and N % 128 == 0 required). */
int convrot_gemm_i8_i32(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K,
                        int32_t b_layout, int32_t* acc, hipStream_t stream);

/* First stage of the int8 input gradient: q_g, s_g from dY and s_w. */
int convrot_bwd_quant_dy(const uint16_t* dy, int64_t M, int64_t N, const float* sw, int8_t* qg,
                         float* sg, hipStream_t stream);

/* Transient dequantization of the bf16 input gradient: what_t [K, N] bf16 =
 * transpose of W_hat = bf16( (s_w * q_w) * R ). */
int convrot_dequant_weight_t(const int8_t* qw, const float* sw, int64_t N, int64_t K,
                             uint16_t* what_t, hipStream_t stream);

/* First stage of the LoRA forward: xa [M, R] bf16 = bf16( x [M, K] * lora_a [R, K]^T )
 * with fp32 accumulation.  R 16 or 32, K % 128 == 0. */
int convrot_lora_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* lora_a,
                      int32_t R, uint16_t* xa, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H_ */
