/*
 * dlfusion.h - C ABI of the fused Conv/MatMul -> BatchNorm -> activation
 * operator for AMD Instinct MI355X (gfx950).
 *
 * The library computes, for one layer,
 *     out = act( conv(x, W') + b' [+ residual] )           (bf16 / fp32)
 *     out = Q( relu( acc(xq, Wq) * alpha + beta' ) / s_y )  (fp8 e4m3)
 * in a single kernel whose epilogue runs on the accumulator registers, so the
 * pre-activation tensors never reach HBM.  BatchNorm is folded into the
 * weights on the host beforehand (dlf_fold_bn, dlf_bn_scale_shift).  An
 * unfused chain of separate kernels (dlf_conv_plain ... dlf_quant_apply) is
 * kept only for comparing HBM traffic and timings against the fused kernel.
 *
 * Sources (web pages; the section named is where each definition appears):
 *  [OPPL] "OpenPPL算子融合深度解析：从图优化到推理性能提升" (OpenPPL operator
 *         fusion deep dive), codechina.net.
 *  [INFR] discosf.com inference-fusion practice article (page titled
 *         "企业官网建设流程全解析").
 *  [CANN] aitangshan.cn graph-autofusion (CANN) article.
 *  [RFC]  "RFC：自动融合: 扩展统一 Pattern Matcher 覆盖量化融合与 GMM/MM+激活",
 *         MindIE-SD issue 298.
 *  [FRT]  "FlashRT 跨层融合深度解析", sheratonhq.com.
 *
 * Conventions shared by every entry point
 *  - Plain C types only.  Device pointers are HIP device memory owned by the
 *    caller; the library allocates no device memory and keeps no pointer after
 *    it returns.  Host pointers (fold functions) are plain host memory.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    Device work is enqueued asynchronously on it; nothing synchronises.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - Every argument is validated on the host before any HIP call; a failed
 *    check returns a negative dlf_status and launches nothing.  The reason is
 *    kept in a thread-local string returned by dlf_last_error().
 *  - DLF_ERR_UNSUPPORTED means "this combination has no fused kernel": the
 *    caller runs the unfused chain instead.  Nothing is ever approximated
 *    silently ([OPPL] §4.2 falls back to separate ops when a fused form does
 *    not apply; [RFC] §3.7 falls back to the original graph on a mismatch).
 *  - Device pointers must be 16-byte aligned (vector loads); bf16 GEMM inputs
 *    need k to be a multiple of 8, fp8 inputs a multiple of 16.  A bf16
 *    convolution takes any c_in (c_in % 8 != 0, such as a 3-channel image,
 *    gathers its operands value by value: slower, for stems).  Zero-sized
 *    outputs are valid and launch nothing.
 *  - The output must not overlap any input (DLF_ERR_ALIAS): every input
 *    element is read by many output tiles.
 *  - Thread safety: no global mutable state besides the thread-local error and
 *    the tuning switches, which are read once when the library loads (see
 *    dlf_tuning_reload).
 */
#ifndef DLFUSION_H
#define DLFUSION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are int-sized.  A C++ translation unit gives them int as their fixed
 * underlying type, so that every int a C caller passes is a value of the type (an unknown code
 * is then a checked error, never undefined behaviour). */
#ifdef __cplusplus
#define DLF_ENUM enum : int
#else
#define DLF_ENUM enum
#endif

typedef DLF_ENUM {
    DLF_OK = 0,
    DLF_ERR_INVALID_ARG = -1,   /* null / negative / non-finite / misaligned argument */
    DLF_ERR_UNSUPPORTED = -2,   /* no fused kernel for this combination: run the unfused chain */
    DLF_ERR_HIP = -3,           /* a HIP runtime call or kernel launch failed */
    DLF_ERR_ALIAS = -4          /* the output overlaps an input */
} dlf_status;

typedef DLF_ENUM {
    DLF_F32 = 0,                /* IEEE binary32 */
    DLF_BF16 = 1,               /* bfloat16, stored as uint16 bit patterns */
    DLF_FP8_E4M3 = 2            /* OCP e4m3fn codes (uint8): max 448, no inf, S.1111.111 = NaN */
} dlf_dtype;

/* Activation of the epilogue; numbering as the epilogue's activation field in
 * [OPPL] §4.3 (0 none, 1 ReLU, 2 GELU).  GELU is the tanh form
 * 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).  3 is the exact GELU
 * v Phi(v) = 0.5 v (1 + erf(v / sqrt(2))), the erf type beside tanh in [RFC]
 * §2.1 and §2.4.  Every activation is available to every fused path; on the fp8
 * GEMM the GELU forms give the quantised MatMul + GELU of [RFC] §2.1. */
typedef DLF_ENUM {
    DLF_ACT_NONE = 0,
    DLF_ACT_RELU = 1,
    DLF_ACT_GELU_TANH = 2,
    DLF_ACT_GELU_ERF = 3
} dlf_act;

/* Gate of a gated projection (dlf_gemm_fused_gated): out = gate(g) * u.
 * SILU gives SwiGLU (silu(g) = g / (1 + e^-g); [RFC] §2.2 GMM + SwiGLU, §2.3
 * the gated Linear form); the GELU forms give GELU x Mul ([RFC] §2.4,
 * gelu(x) * y). */
typedef DLF_ENUM {
    DLF_GATE_SILU = 0,
    DLF_GATE_GELU_TANH = 1,
    DLF_GATE_GELU_ERF = 2
} dlf_gate;

/* A 2-D convolution layer.  x is NHWC [n][h][w][c_in]; weights are OHWI
 * [c_out][kh][kw][c_in] (the GEMM view: B = [c_out][K], K = kh*kw*c_in,
 * k = (r*kw + s)*c_in + ci); y (and residual) are NHWC [n][ho][wo][c_out] with
 * ho = (h + 2 pad_h - kh)/stride_h + 1, wo likewise.  Zero padding, dilation 1,
 * one group.  [INFR] §3.3 gives the kernel arguments (C_in, C_out, H, W, KH,
 * KW, stride, pad) and the zero-padding rule; [OPPL] §3.4 motivates NHWC. */
typedef struct {
    int64_t n, h, w, c_in, c_out, kh, kw;
    int32_t stride_h, stride_w, pad_h, pad_w;
    dlf_dtype dtype;            /* storage type of x, w, residual and y */
    dlf_act act;
} dlf_conv_desc;

/* A matrix product C[m][n] = A[m][k] . B[n][k]^T (a 1x1 convolution over m
 * tokens; B in the [out][in] layout of a linear layer). */
typedef struct {
    int64_t m, n, k;
    dlf_dtype in_dtype;         /* type of A and B */
    dlf_dtype out_dtype;        /* type of C (and residual) */
    dlf_act act;
    float out_inv_scale;        /* fp8 output only: fp32(1/s_y) of the static output scale */
} dlf_gemm_desc;

/* ---------------------------------------------------------------------- */
/* Host-side folding (once per layer, at load time)                        */
/* ---------------------------------------------------------------------- */

/* Fold an inference BatchNorm into the preceding convolution's weights and
 * bias ([OPPL] §3.1; derivation in [INFR] §2.1):
 *     s[c]   = gamma[c] / sqrt(var[c] + eps)
 *     W'[c,:] = W[c,:] * s[c]
 *     b'[c]  = (b[c] - mean[c]) * s[c] + beta[c],   b = 0 when conv_bias is NULL
 * A bias is always produced, so a conv without one gains one ([OPPL] §3.1).
 * eps is used exactly as given; nothing is approximated ([OPPL] §3.1, [INFR]
 * §2.1 and §4.1 on what a dropped eps does to low-variance channels).  The
 * bias is computed from the original W and b, never from W' ([INFR] §2.1).
 * All arithmetic is binary64; each W' is rounded once (round to nearest
 * even) to w_out_dtype, avoiding the double rounding of [OPPL] §6.2.
 *   w        host, [cout][k] fp32 (OHWI flattened, k = kh*kw*c_in)
 *   conv_bias host, [cout] fp32 or NULL
 *   gamma, beta, mean, var  host, [cout] fp32
 *   eps      finite, >= 0; var[c] + eps must be > 0 for every channel
 *   w_out_dtype  DLF_F32 or DLF_BF16 (else DLF_ERR_UNSUPPORTED)
 *   w_out    host, [cout][k] in w_out_dtype (uint16 bit patterns for bf16)
 *   bias_out host, [cout] fp32, always written
 * Synchronous; touches no GPU.  May be called with cout == 0 or k == 0. */
dlf_status dlf_fold_bn(int64_t cout, int64_t k, const float *w, const float *conv_bias,
                       const float *gamma, const float *beta, const float *mean,
                       const float *var, double eps, dlf_dtype w_out_dtype,
                       void *w_out, float *bias_out);

/* Per-channel scale and shift of a BatchNorm kept out of the weights, for the
 * fp8 path, where a per-channel factor inside the weights would change their
 * per-tensor amax and thus their scale ([RFC] §3.4 takes the input and weight
 * scales from the graph; [FRT] §3 folds norm parameters at load time):
 *     s[c] = gamma[c] / sqrt(var[c] + eps)
 *     scale_out[c] = fp32( pre_scale * s[c] )                 (alpha)
 *     shift_out[c] = fp32( (b[c] - mean[c]) * s[c] + beta[c] )  (beta')
 * so that  BN(acc * pre_scale + b) = acc * alpha + beta'.  pre_scale is the
 * product of the static input and weight scales s_x * s_w (1 for none).
 * Binary64 throughout, one rounding per output.  Host memory, synchronous. */
dlf_status dlf_bn_scale_shift(int64_t cout, const float *conv_bias, const float *gamma,
                              const float *beta, const float *mean, const float *var,
                              double eps, double pre_scale, float *scale_out,
                              float *shift_out);

/* ---------------------------------------------------------------------- */
/* Fused kernels (the hot path)                                            */
/* ---------------------------------------------------------------------- */

/* Fused convolution with a register epilogue ([OPPL] §4.3: conv main loop as
 * an implicit GEMM plus an epilogue applied in the order bias -> residual ->
 * activation before the single store; [OPPL] §2.1 and §3.3):
 *     y = act( conv(x, w) + bias[c] + residual )
 * w and bias are the folded W' and b' from dlf_fold_bn.  Accumulation is fp32
 * ([OPPL] §4.2 and §6.2, [INFR] §4.1); the output is rounded once (RNE).
 * Each element of y is written to device memory exactly once.
 *   d        host descriptor; dtype DLF_F32 (fp32 FMA kernel) or DLF_BF16
 *            (bf16 MFMA implicit GEMM, any c_in); DLF_FP8_E4M3 ->
 *            DLF_ERR_UNSUPPORTED
 *   x, w     device, layouts as in dlf_conv_desc, type d->dtype
 *   bias     device [c_out] fp32, or NULL (no bias)
 *   residual device, same shape and type as y, or NULL ([OPPL] §4.2: only a
 *            dense same-shape tensor is absorbed)
 *   y        device output
 *   stream   hipStream_t or NULL */
dlf_status dlf_conv_fused(const dlf_conv_desc *d, const void *x, const void *w,
                          const float *bias, const void *residual, void *y, void *stream);

/* Fused matrix product with the same register epilogue, per output column n:
 *     v = acc * col_scale[n] + col_shift[n]  [+ residual]; v = act(v)
 *     bf16 out:  C = bf16(v)
 *     fp8 out:   C = Q( fp32(v * out_inv_scale) )  (static per-tensor scale)
 * Q rounds to the nearest e4m3 value, ties to even, and saturates at +-448
 * (the quantisation-aware clamp of [OPPL] §6.4; the static-scale fp8 epilogue
 * of [FRT] §3 and §6; quantised MatMul + activation of [RFC] §3.4).
 * Supported: in_dtype BF16 -> out BF16 (any act, optional bf16 residual);
 *            in_dtype FP8_E4M3 -> out FP8_E4M3 or BF16 (any act, no
 *            residual; with a GELU: quantised MatMul + GELU, [RFC] §2.1).
 *            Everything else -> DLF_ERR_UNSUPPORTED.
 *   a        device [m][k]; b device [n][k] (k % 8 == 0 bf16, % 16 == 0 fp8)
 *   col_scale device [n] fp32 or NULL (= 1); col_shift device [n] fp32 or
 *            NULL (= 0): the bias, or the folded BN scale/shift (alpha, beta')
 *   residual device [m][n] in out_dtype (bf16 only) or NULL
 *   c        device [m][n] in out_dtype */
dlf_status dlf_gemm_fused(const dlf_gemm_desc *d, const void *a, const void *b,
                          const float *col_scale, const float *col_shift,
                          const void *residual, void *c, void *stream);

/* The GEMM of dlf_gemm_fused over weights concatenated along n at load, stored
 * split by columns: one launch computes Q, K and V (or any equal column
 * blocks) and writes each block to its own tensor.  [OPPL] §3.2: the Q, K and
 * V projections become one GEMM over [W_q; W_k; W_v] ([3h, h]) whose result is
 * cut into Q, K and V, by a split kernel or by offsets; here the epilogue's
 * store does the cut, so the [m][3h] result never exists in memory.
 *   columns [p n/parts, (p+1) n/parts) -> outs[p], a row-major [m][n/parts]
 *   tensor of d->out_dtype; outs is a HOST array of `parts` device pointers.
 * Same operands, scale/shift, activation and dtypes as dlf_gemm_fused; no
 * residual.  INVALID_ARG: parts < 1, outs or an outs[p] NULL or not 16-byte
 * aligned, n not divisible by parts.  UNSUPPORTED: parts > 4, a part's row not
 * a whole number of 16-byte chunks (n/parts % 8 for bf16, % 16 for fp8 output),
 * and every case dlf_gemm_fused refuses.  ALIAS: a part overlaps an input or
 * another part. */
dlf_status dlf_gemm_fused_split(const dlf_gemm_desc *d, const void *a, const void *b,
                                const float *col_scale, const float *col_shift,
                                int32_t parts, void *const *outs, void *stream);

/* Gated projection: one GEMM over gate and up weights interleaved by rows at
 * load, with a gated register epilogue, so neither projection reaches memory:
 *     b row 2j = gate weight j, row 2j+1 = up weight j (d->n = 2 x outputs);
 *     g = acc[2j] * col_scale[2j] + col_shift[2j]   (likewise u from 2j+1)
 *     c[m][j] = bf16( gate(g) * u ),  c is [m][n/2].
 * col_scale / col_shift are [n], interleaved like b (NULL = 1 / 0).  [RFC]
 * §2.2 - §2.4 list GMM + SwiGLU, the gated Linear and gelu(x) * y among the
 * fusion targets; the interleave keeps each (gate, up) pair in one lane's
 * registers.  bf16 operands and output; d->act must be NONE (the gate is the
 * activation); no residual.
 * INVALID_ARG: unknown gate, act != NONE, odd n, NULL / misaligned pointers.
 * UNSUPPORTED: other dtypes, k % 8 != 0.  ALIAS: c overlaps an input. */
dlf_status dlf_gemm_fused_gated(const dlf_gemm_desc *d, const void *a, const void *b,
                                const float *col_scale, const float *col_shift,
                                dlf_gate gate, void *c, void *stream);

/* ---------------------------------------------------------------------- */
/* Unfused comparison chain: one kernel per op, every intermediate goes     */
/* through device memory ([OPPL] §2.1, §3.3; [CANN] MatMul->BiasAdd->ReLU   */
/* costs three HBM round trips where the fused form costs one).             */
/* ---------------------------------------------------------------------- */

/* y = conv(x, w) + conv_bias (no BN, no activation), rounded once to d->dtype.
 * Same layouts, dtypes and checks as dlf_conv_fused; d->act must be NONE. */
dlf_status dlf_conv_plain(const dlf_conv_desc *d, const void *x, const void *w,
                          const float *conv_bias, void *y, void *stream);

/* y = A . B^T, no epilogue.  bf16 in -> d->out_dtype BF16 (rounded once);
 * fp8 in -> d->out_dtype F32 with y = fp32(acc * dequant), dequant = s_x*s_w.
 * d->act must be NONE. */
dlf_status dlf_gemm_plain(const dlf_gemm_desc *d, const void *a, const void *b,
                          float dequant, void *y, void *stream);

/* Inference BatchNorm as its own pass over [rows][c] (channel innermost):
 *     z = gamma (y - mean) / sqrt(var + eps) + beta        ([OPPL] §3.1)
 * computed in fp32; dt is DLF_F32 or DLF_BF16 for both y and z; BN params are
 * device [c] fp32. */
dlf_status dlf_bn_apply(int64_t rows, int64_t c, dlf_dtype dt, const void *y,
                        const float *gamma, const float *beta, const float *mean,
                        const float *var, double eps, void *z, void *stream);

/* z = y * scale[ch] + shift[ch] over [rows][c]; scale NULL means 1 (a
 * BiasAdd).  dt DLF_F32 or DLF_BF16; scale/shift device fp32 [c]. */
dlf_status dlf_scale_shift_apply(int64_t rows, int64_t c, dlf_dtype dt, const void *y,
                                 const float *scale, const float *shift, void *z,
                                 void *stream);

/* out = a + b elementwise (the residual Add as its own kernel, [OPPL] §3.3).
 * dt DLF_F32 or DLF_BF16. */
dlf_status dlf_add(int64_t count, dlf_dtype dt, const void *a, const void *b, void *out,
                   void *stream);

/* out = act(in) elementwise; dt DLF_F32 or DLF_BF16.  in == out is allowed
 * (the only entry point that may work in place). */
dlf_status dlf_act_apply(int64_t count, dlf_dtype dt, dlf_act act, const void *in, void *out,
                         void *stream);

/* codes = Q( fp32(in * inv_scale) ): the same e4m3 quantiser the fused fp8
 * epilogue uses, as its own pass (static per-tensor scale, [FRT] §3). */
dlf_status dlf_quant_apply(int64_t count, const float *in, float inv_scale, uint8_t *codes,
                           void *stream);

/* ---------------------------------------------------------------------- */
/* Feed-forward block in one kernel: FC1 -> activation -> FC2               */
/* ---------------------------------------------------------------------- */

/* A transformer feed-forward block ([OPPL] §3.2: the two fully connected
 * layers and the activation between them fused into one kernel, the
 * activated intermediate kept on chip; the block's residual add rides in the
 * second layer's epilogue, [OPPL] §3.3):
 *     y = act(x W1^T + b1) W2^T + b2 [+ residual]
 * x, residual, y: [m][d_model]; W1: [d_ff][d_model]; W2: [d_model][d_ff]
 * (the [out][in] layout of a linear layer); biases fp32. */
typedef struct {
    int64_t m, d_model, d_ff;
    dlf_dtype dtype;            /* DLF_BF16 (else DLF_ERR_UNSUPPORTED) */
    dlf_act act;
} dlf_ffn_desc;

/* Load-time packing of one weight matrix W [rows][k] (bf16 bit patterns) into
 * the order the fused kernel streams it: for each block of 32 rows rb and
 * each 16-wide k step s, 64 runs of 8 values,
 *     packed[((rb * (k/16) + s) * 64 + l) * 8 + e]
 *         = W[32 rb + l % 32][16 s + 8 (l / 32) + e],
 * i.e. one MFMA operand fragment of a wave per contiguous kilobyte.  Host
 * memory, synchronous; rows % 32 == 0 and k % 16 == 0 (else
 * DLF_ERR_INVALID_ARG); packed must not overlap w (DLF_ERR_ALIAS). */
dlf_status dlf_ffn_pack(int64_t rows, int64_t k, const uint16_t *w, uint16_t *packed);

/* The fused block.  A workgroup owns 32 tokens and all d_model outputs: it
 * walks d_ff in chunks of 256, computes each chunk of act(x W1^T + b1) into
 * LDS (rounded to bf16, the operand type of the second product) and
 * accumulates the chunk's contribution to y in fp32 registers; y is rounded
 * once (RNE) and written once.
 *   d          host; d_model in {256, 512, 768, 1024}, d_ff a positive
 *              multiple of 256 (else DLF_ERR_UNSUPPORTED: run the two GEMMs)
 *   x          device [m][d_model] bf16
 *   w1_packed  device, dlf_ffn_pack of W1 (rows d_ff, k d_model)
 *   b1         device [d_ff] fp32 or NULL
 *   w2_packed  device, dlf_ffn_pack of W2 (rows d_model, k d_ff)
 *   b2         device [d_model] fp32 or NULL
 *   residual   device [m][d_model] bf16 or NULL
 *   y          device [m][d_model] bf16, not overlapping any input
 *   stream     hipStream_t or NULL */
dlf_status dlf_ffn_fused(const dlf_ffn_desc *d, const void *x, const void *w1_packed,
                         const float *b1, const void *w2_packed, const float *b2,
                         const void *residual, void *y, void *stream);

/* Bytes of device workspace dlf_ffn_fused_ws needs for d (0 where it does
 * not split), written to *bytes.  The same descriptor checks and statuses as
 * dlf_ffn_fused; bytes NULL: DLF_ERR_INVALID_ARG.  Host only. */
dlf_status dlf_ffn_workspace_bytes(const dlf_ffn_desc *d, size_t *bytes);

/* dlf_ffn_fused with a caller-owned workspace, which lets the block split d_ff
 * where one workgroup per 32 or 64 tokens would stream the weights through
 * too few CUs (fewer than 160 token blocks, d_model <= 768, d_ff >= 512): S
 * workgroups share a token block, each over 1/S of d_ff, and write fp32
 * partial sums of act(x W1^T + b1) W2^T to the workspace ([S][m][d_model]); a
 * second kernel adds them, b2 and the residual and rounds y once (RNE).  The
 * same result up to the order of the fp32 sums.
 *   workspace        device, 16-byte aligned, at least dlf_ffn_workspace_bytes(d)
 *                    bytes (else DLF_ERR_INVALID_ARG), overlapping no operand
 *                    (DLF_ERR_ALIAS); may be NULL where that size is 0.  Its
 *                    contents are scratch: calls that share one on overlapping
 *                    streams race.
 * Every other argument, check and status as dlf_ffn_fused. */
dlf_status dlf_ffn_fused_ws(const dlf_ffn_desc *d, const void *x, const void *w1_packed,
                            const float *b1, const void *w2_packed, const float *b2,
                            const void *residual, void *y, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Bytes of the static device scratch behind dlf_ffn_fused_noalloc (32 MiB). */
#define DLF_FFN_NOALLOC_SCRATCH_BYTES (32u << 20)

/* dlf_ffn_fused_ws for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The d_ff split's partial sums go to a static device array of
 * DLF_FFN_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on until the process ends; the call itself allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).
 *   - A block whose split needs more than DLF_FFN_NOALLOC_SCRATCH_BYTES
 *     (dlf_ffn_workspace_bytes(d) tells) is rejected with
 *     DLF_ERR_INVALID_ARG before anything is launched; use dlf_ffn_fused_ws.
 *   - Every call on one device shares that device's array: calls that may
 *     overlap on one device (concurrent streams, several host threads) race.
 *     Its contents persist between calls; none is read before it is written.
 *   - The first call on a device looks the array's address up (a HIP runtime
 *     query, not an allocation); later calls reuse it.
 * Every other argument, check, status and the result as dlf_ffn_fused_ws. */
dlf_status dlf_ffn_fused_noalloc(const dlf_ffn_desc *d, const void *x, const void *w1_packed,
                                 const float *b1, const void *w2_packed, const float *b2,
                                 const void *residual, void *y, void *stream);

/* ---------------------------------------------------------------------- */
/* Host fusion pass: which chains of a graph become one fused launch        */
/* ---------------------------------------------------------------------- */

/* Operation of a graph node.  The pass fuses a contraction (CONV, MATMUL,
 * MATMUL_FP8) with the epilogue ops that follow it; every other op is kept. */
typedef DLF_ENUM {
    DLF_OP_INPUT = 0,           /* a tensor that no node computes */
    DLF_OP_CONV = 1,
    DLF_OP_MATMUL = 2,
    DLF_OP_MATMUL_FP8 = 3,      /* fp8 codes in, dequantised fp32 out */
    DLF_OP_BIAS_ADD = 4,
    DLF_OP_BATCHNORM = 5,
    DLF_OP_ADD = 6,             /* elementwise, two inputs */
    DLF_OP_RELU = 7,
    DLF_OP_GELU_TANH = 8,
    DLF_OP_GELU_ERF = 9,
    DLF_OP_QUANT = 10,          /* static e4m3 quantisation */
    DLF_OP_OTHER = 11           /* anything else (Reshape, Transpose, ...): never fused */
} dlf_op;

#define DLF_NODE_OUTPUT 1u      /* the node's tensor is a graph output and must reach memory */
#define DLF_NODE_TRAINING 2u    /* a BatchNorm in training mode (never folded) */

/* One node of a graph in topological order.  inputs[j] < the node's own
 * index.  shape is the output shape (rank 0..4, extents >= 0); dtype its
 * storage type; flops the node's arithmetic as the caller counts it (2MNK for
 * a contraction, a few per element for the rest). */
typedef struct {
    int32_t op;                 /* dlf_op */
    int32_t n_inputs;           /* 0, 1 or 2 */
    int32_t inputs[2];
    int32_t dtype;              /* dlf_dtype */
    uint32_t flags;             /* DLF_NODE_* */
    int32_t rank;
    int32_t reserved;           /* 0 */
    int64_t shape[4];
    int64_t flops;
} dlf_graph_node;

/* One fused group: nodes[0] is the contraction, then its epilogue ops in
 * chain order (at most bias/BN, Add, activation, quantisation). */
typedef struct {
    int32_t count;              /* 2..5 */
    int32_t nodes[5];
    int64_t saved_bytes;        /* HBM bytes the fusion avoids */
    double net_benefit;         /* saved_bytes - overhead, in bytes */
} dlf_fusion_group;

/* Plan the fusions of a graph with the three stages of the CANN
 * graph-autofusion article ([CANN]):
 *  1. pattern matching: from every contraction, follow the chain
 *       contraction [bias_add | batchnorm] [add] [activation] [quant]
 *     (the fused epilogue's order, [OPPL] §4.3; quant only after MATMUL_FP8,
 *     which takes no Add).  A value may flow on only when it has exactly one
 *     reader and is not a graph output ([OPPL] §4.1, §4.2); a BatchNorm must
 *     be in inference mode ([OPPL] §4.1); the other operand of the Add must
 *     have the chain's shape and dtype (no broadcast, [OPPL] §4.2); every op
 *     keeps the contraction's output shape and dtype.  Every prefix of two or
 *     more ops is a candidate.
 *  2. benefit: saved_bytes = 2 x the bytes of every tensor inside the chain
 *     (each would be written once and read back once); overhead =
 *     overhead_frac x (sum of the group's flops) / ridge, the bytes the HBM
 *     moves while the chip does that fraction of the group's arithmetic
 *     (ridge = peak flop/s over peak bytes/s); net = saved - overhead in
 *     binary64.  Candidates with net <= 0 are dropped.
 *  3. conflict resolution: greedy by net benefit, largest first (ties: the
 *     lower first node, then the longer chain); a candidate sharing an op with
 *     one already taken is dropped.
 * Groups are written in order of their first node.
 *   nodes        host, [n_nodes] (NULL when n_nodes == 0)
 *   ridge        > 0 and finite (MI355X bf16: 2516.6e12 / 8e12)
 *   overhead_frac  >= 0 and finite (the article's 0.05)
 *   groups       host, [capacity]; may be NULL when capacity == 0
 *   n_groups     host, receives the number of groups
 * Returns DLF_ERR_INVALID_ARG for a malformed graph (bad op, dtype, rank,
 * negative extent or flops, an input index not below the node's own) and
 * when capacity is too small (then *n_groups holds the number needed and no
 * group is written).  Synchronous; touches no GPU. */
dlf_status dlf_fusion_plan(const dlf_graph_node *nodes, int32_t n_nodes, double ridge,
                           double overhead_frac, dlf_fusion_group *groups, int32_t capacity,
                           int32_t *n_groups);

/* ---------------------------------------------------------------------- */
/* Status                                                                   */
/* ---------------------------------------------------------------------- */

/* Static name of a status code. */
const char *dlf_status_string(dlf_status s);

/* Detail of the last non-OK status returned on this thread ("" if none).
 * The pointer stays valid until the next library call on this thread. */
const char *dlf_last_error(void);

/* ---------------------------------------------------------------------- */
/* Tuning switches                                                          */
/* ---------------------------------------------------------------------- */

/* Kernel routes and tiles can be forced for tuning and tests through the
 * environment: DLF_TILE (an MFMA tile index), DLF_GEMM (tiled | stream),
 * DLF_CONV (generic | stream), DLF_STREAM_NB (128 | 256 | 384), DLF_FFN_TOK
 * (32 | 64) and DLF_FFN_SPLIT (d_ff parts; 0 or 1: none).  Forcing a route
 * never changes a result beyond the order of fp32 sums.  The library reads
 * them once when it is loaded; dlf_tuning_reload() reads them again.  Host
 * only; it must not run concurrently with another library call. */
void dlf_tuning_reload(void);

/* ---------------------------------------------------------------------- */
/* Measurement aid                                                          */
/* ---------------------------------------------------------------------- */

/* Shader-clock probe for a clock-derived matrix-core peak (the pages ask for
 * each fused kernel's throughput against the hardware's limits: [OPPL] §5.2
 * measures per-kernel DRAM throughput, [INFR] §1.2 places a fused op on the
 * roofline).  Launches `workgroups` workgroups of four waves; each runs
 * `iters` steps of four independent bf16 32x32x16 MFMAs and writes, for
 * workgroup b,
 *     stamps[4b + 0], stamps[4b + 1]  shader-clock counter before, after
 *     stamps[4b + 2], stamps[4b + 3]  100 MHz constant counter before, after
 * so that (s1 - s0) / (r1 - r0) * 100 MHz is the shader clock the chip held
 * while its matrix pipes were busy.
 *   workgroups  1 .. 65536; iters >= 1 (else DLF_ERR_INVALID_ARG)
 *   stamps      device, 16-byte aligned, 4 * workgroups uint64 values
 *   stream      hipStream_t or NULL; asynchronous like every launch */
dlf_status dlf_clock_probe(int32_t workgroups, int32_t iters, uint64_t *stamps, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DLFUSION_H */
