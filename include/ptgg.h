/*
 * ptgg.h -- C ABI of the MoE expert grouped GEMM library for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation: the tokens routed to the experts of a Mixture-of-Experts
 * layer arrive sorted by expert, so expert g owns a contiguous run of
 * group_lens[g] rows of the activation matrix, and every expert multiplies
 * its own rows by its own weight matrix.  All experts are issued as ONE
 * kernel over the ragged batch instead of one small GEMM per expert (blog
 * "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
 * Primus", section "Expert parallelism: DeepEP and the grouped GEMM", and
 * its optimisation-ladder table, rung "Turbo grouped GEMM").
 *
 * Conventions shared by every entry point
 *  - Pointers named a, b, dy, out, dx, main_grad, q, scales, group_lens,
 *    group_offs and workspace are DEVICE pointers on the current HIP device.
 *    The library never dereferences them on the host, never allocates, never
 *    frees and never synchronises; the caller owns every buffer and keeps it
 *    alive until the work queued on `stream` has finished.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is only enqueued; calls return immediately.
 *  - Row ranges: expert g owns rows [offs[g], offs[g] + group_lens[g]) of the
 *    row-indexed operands, where offs = group_offs (int64[G+1]) when given,
 *    else the exclusive prefix sum of group_lens computed on the device.
 *    With group_offs the ranges must come in expert order without
 *    overlapping (offs[g] + lens[g] <= offs[g + 1], offs[G] <= M); rows
 *    between them belong to no expert.
 *    group_lens are int64, >= 0, and come from the router on the device; the
 *    host never reads them.  Experts with zero rows are allowed anywhere.
 *    Device code clamps every range into [0, M], so malformed lengths never
 *    cause an out-of-bounds access; it records them instead in the optional
 *    error word (see pt_read_error_flags).
 *  - Element types (pt_dtype):
 *      PT_BF16         bfloat16, row-major.
 *      PT_MXFP8_E4M3   OCP-MX: one E4M3 byte per element + one E8M0 scale
 *                      byte per 32 consecutive elements along the reduction
 *                      dimension K.
 *      PT_MXFP4_E2M1   OCP-MX: E2M1 codes packed two per byte (even element
 *                      in the low nibble, the float4_e2m1fn_x2 layout named
 *                      in the PR page "[Megatron-LM] feat: add grouped gemm
 *                      fp4 support, skip cache trans weight and santize
 *                      code", section "Changes") + one E8M0 scale per 32.
 *    For MX operands the scales form a row-major [rows, K/32] byte matrix.
 *  - Size limits: the kernels address operands with 32-bit byte offsets, so
 *    each of A (or dY), one expert's weight matrix, and the whole scale
 *    tensors must stay below 2 GiB; larger problems get PT_ERR_UNSUPPORTED
 *    (split them along M or N).
 *  - Accumulation is in fp32 on the matrix cores; outputs are rounded once
 *    (bf16 round-to-nearest-even, or fp32 for main_grad).
 *  - Return value: a pt_status.  On any error nothing is launched.
 */
#ifndef PTGG_H
#define PTGG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PT_OK = 0,
    PT_ERR_INVALID_ARG = 1,  /* NULL required pointer, negative or inconsistent size */
    PT_ERR_UNSUPPORTED = 2,  /* dtype/layout/epilogue combination, too many experts, not gfx950 */
    PT_ERR_MISALIGNED = 3,   /* pointer or leading dimension not 16-byte aligned */
    PT_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required */
    PT_ERR_HIP = 5           /* a HIP runtime call failed */
} pt_status;

typedef enum {
    PT_BF16 = 0,
    PT_MXFP8_E4M3 = 1,
    PT_MXFP4_E2M1 = 2,
    PT_FP8_E4M3 = 3,         /* E4M3 codes with one fp32 scale per tensor (current
                                scaling, pt_fp8_quantize): the scale arguments point
                                to fp32 factors, one for A and one per expert for B */
    PT_FP8_E4M3_ROWWISE = 4  /* E4M3 codes with one fp32 scale per row of A [M] and per
                                row of B [G, N] (pt_fp8_quantize_rows) */
} pt_dtype;

typedef enum {
    PT_EPI_NONE = 0,         /* out = bf16(C), [M, N]                               */
    PT_EPI_SWIGLU = 1,       /* out = bf16(silu(C[:, :N/2]) * C[:, N/2:]), [M, N/2] */
    PT_EPI_SWIGLU_MXFP4 = 2  /* SWIGLU's bf16 value, then MXFP4-quantised along its
                                columns: out = codes [M, N/4] bytes,
                                out_scale = E8M0 [M, N/64]                         */
} pt_epilogue;

typedef enum {
    PT_OP_FWD = 0,
    PT_OP_DGRAD = 1,
    PT_OP_WGRAD = 2,
    PT_OP_DGRAD_SWIGLU = 3   /* pt_grouped_gemm_dgrad_swiglu (for pt_gemm_config_of) */
} pt_op;

/* Largest expert count one call accepts. */
#define PT_MAX_GROUPS 1024

/*
 * Grouped forward: for every expert g and each of its rows r,
 *     C[r, :] = A[r, :] . B_g            (B_g is K x N)
 * followed by the epilogue.  This is the FC1/FC2 expert GEMM; the SwiGLU
 * epilogue takes the FC1 output as [gate | up] halves, gate first, since the
 * FC1 weight stacks gate and up projections (blog "Enabling DeepSeek-V4-Flash
 * Training on AMD Instinct MI355X GPUs with Primus", section "MegaMoE: fusing
 * communication into the grouped GEMM", weight w1 [g, 2I, H] "gate + up", with
 * SwiGLU between the two grouped GEMMs; Primus-Turbo README, "What's New":
 * expert MLP with SwiGLU folded into the grouped GEMM).
 *
 *  a          [M, K]   activations (bf16 / E4M3 bytes / packed E2M1 [M, K/2])
 *  a_scale    [M, K/32] E8M0, MX only (else NULL)
 *  b          trans_b = 0: [G, K, N] (bf16 only); trans_b = 1: [G, N, K], the
 *             [experts, out, in] weight layout (required for MX)
 *  b_scale    [G, N, K/32] E8M0, MX only
 *  out        see pt_epilogue; rows outside every expert are not written
 *  out_scale  [M, N/64] E8M0 for PT_EPI_SWIGLU_MXFP4, else NULL
 *  Requirements: K % 8 == 0 (bf16) or K % 32 == 0 (MX); N % 8 == 0 (bf16
 *  with trans_b = 0, and MX); N % 16 == 0 for SWIGLU, N % 64 == 0 for
 *  SWIGLU_MXFP4;
 *  a_scale and b_scale 4-byte aligned (else PT_ERR_MISALIGNED).
 *  PT_FP8_E4M3 (FP8 with current scaling: the grouped linear's FP8 path
 *  calls the grouped FP8 GEMM, PR page "[Megatron-LM] feat: add grouped gemm
 *  fp4 support, ...", Copilot overview, and its "Changes" treat current
 *  scaling as an FP8 recipe): a [M, K] and b [G, N, K] E4M3 codes (trans_b = 1), a_scale one
 *  fp32 factor and b_scale [G] fp32 factors (the `dequant` outputs of
 *  pt_fp8_quantize), read as const float *; then
 *      C[r, :] = (sum_k a[r, k] * b_g[:, k]) * a_scale[0] * b_scale[g]
 *  with exact code products, an fp32 sum and one fp32 product of the two
 *  factors, before the epilogue.  Requirements as for MXFP8.
 *  PT_FP8_E4M3_ROWWISE: the same with a_scale [M] fp32 (one factor per row
 *  of A) and b_scale [G, N] fp32 (one per row of each expert's B, i.e. per
 *  output column): C[r, n] = (sum_k a[r, k] * b_g[n, k]) * (a_scale[r] *
 *  b_scale[g, n]), the two factors multiplied in fp32 first.
 *  swiglu_limit  the clamped SwiGLU of the SWIGLU epilogues (the DeepSeek-V4
 *             blog lists a swiglu_limit knob, 10.0 for V4-Flash, "clamped
 *             SwiGLU" for FP8 and FP4 stability, without a formula; the
 *             reading taken): with L = swiglu_limit > 0 and finite, the
 *             epilogue computes silu(min(g, L)) * min(max(u, -L), L).  0 or
 *             infinity: the plain SwiGLU; NaN: PT_ERR_INVALID_ARG.  Ignored
 *             by PT_EPI_NONE.
 *  workspace  optional (may be NULL): the error word and tile queues, see
 *             pt_grouped_gemm_workspace_size.
 */
int pt_grouped_gemm_fwd(const void *a, const uint8_t *a_scale,
                        const void *b, const uint8_t *b_scale,
                        void *out, uint8_t *out_scale,
                        const int64_t *group_lens, const int64_t *group_offs,
                        int64_t G, int64_t M, int64_t N, int64_t K,
                        int dtype, int trans_b, int epilogue, float swiglu_limit,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * pt_grouped_gemm_fwd for the MX and FP8 dtypes with code rows of A [M, ...]
 * and of B [G, N, ...] stored code_pitch bytes apart (as
 * pt_mx_quantize_pitched writes them) instead of packed; trans_b is 1 (the
 * weights' codes are reduction-contiguous).  Same operation and passages as
 * pt_grouped_gemm_fwd, and bit-identical results for the same codes: only
 * where each code row starts changes.  A row pitch that is a multiple of
 * 128 bytes starts every row on a cache line, so the kernel's 128-byte
 * reduction stages read whole lines (a 2880-byte pitch starts every other row
 * half-way into one).  The bytes past a row's codes are never read.
 *  dtype      PT_MXFP8_E4M3, PT_MXFP4_E2M1, PT_FP8_E4M3 or PT_FP8_E4M3_ROWWISE;
 *             PT_BF16 gives PT_ERR_UNSUPPORTED.
 *  code_pitch bytes between code rows of both A and B: at least K (E4M3) or
 *             K/2 (E2M1) and a multiple of 16, else PT_ERR_INVALID_ARG.  a
 *             holds (M - 1) * code_pitch + the row's code bytes, b
 *             (G * N - 1) * code_pitch + the row's code bytes.  Scales as
 *             pt_grouped_gemm_fwd (packed).
 *  Runs on the 256 x 256 kernel only: MXFP4 with K % 256 != 0 also needs
 *  the workspace's stage-major scale copies (else PT_ERR_UNSUPPORTED), and
 *  configurations 2 and 3 of pt_set_gemm_config fall back to 0 and 1.
 *  Other arguments, requirements and errors as pt_grouped_gemm_fwd.
 */
int pt_grouped_gemm_fwd_pitched(const void *a, const uint8_t *a_scale,
                                const void *b, const uint8_t *b_scale,
                                void *out, uint8_t *out_scale,
                                const int64_t *group_lens, const int64_t *group_offs,
                                int64_t G, int64_t M, int64_t N, int64_t K,
                                int dtype, int epilogue, float swiglu_limit, int64_t code_pitch,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * pt_grouped_gemm_fwd without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and
 * requirements as pt_grouped_gemm_fwd, bit for bit; the scratch that the
 * workspace would carry -- the error word and the eight tile-queue counters,
 * 1280 bytes whatever the problem size -- lives in a static device array of
 * the library (4 KiB, one copy per GPU, held until the process ends), so no
 * size can exceed it.  The call allocates nothing and never times kernel
 * configurations (under PT_CONFIG_TUNE it takes a tuned choice of its
 * class, else the rules' choice).  The MX forwards run on row-major scales
 * (no stage-major scale copies, which need a workspace).  The counters are
 * zeroed on `stream` at every call; the device error bits are not reported.
 * Every call on one GPU shares that array: calls that may overlap on one GPU
 * (different streams, or different host threads) race and must be
 * serialised by the caller.
 */
int pt_grouped_gemm_fwd_noalloc(const void *a, const uint8_t *a_scale,
                                const void *b, const uint8_t *b_scale,
                                void *out, uint8_t *out_scale,
                                const int64_t *group_lens, const int64_t *group_offs,
                                int64_t G, int64_t M, int64_t N, int64_t K,
                                int dtype, int trans_b, int epilogue, float swiglu_limit,
                                void *stream);

/*
 * Grouped data gradient: for every expert g and each of its rows r,
 *     dX[r, k] = sum_n dY[r, n] * B_g[k, n]
 * (the grouped GEMM's backward flow, PR page "[Megatron-LM] feat: add grouped
 * gemm fp4 support, ...", Copilot overview: the grouped linear returns to the
 * standard grouped GEMM backward).
 *  BF16: dy [M, N] bf16;  b as in pt_grouped_gemm_fwd (trans_b selects
 *  [G,K,N] or [G,N,K]);  the scale arguments NULL.  Requirements: N % 8 == 0
 *  and K % 8 == 0.
 *  MX (PT_MXFP8_E4M3, PT_MXFP4_E2M1): dy [M, N] codes with dy_scale
 *  [M, N/32] (pt_mx_quantize of dY); b the weight's transposed cache
 *  [G, K, N] codes with b_scale [G, K, N/32] (pt_mx_quantize_t of a [G, N, K]
 *  weight, or pt_mx_quantize of a [G, K, N] one), so trans_b must be 0;
 *  the products are exact and the sums fp32, as in the MX forward.
 *  FP8 (PT_FP8_E4M3): dy [M, N] codes with its one fp32 factor
 *  (pt_fp8_quantize of dY, batch 1) as dy_scale; b the transposed weight
 *  [G, K, N] as E4M3 codes with one fp32 factor per expert (pt_fp8_quantize,
 *  batch G, of the transposed weight, whose amax is the forward weight's) as
 *  b_scale.  PT_FP8_E4M3_ROWWISE: factors per row of dY [M] and per row of
 *  the transposed weight [G, K] (pt_fp8_quantize_rows), i.e. per output row
 *  and per output column.  dX = factors times the exact code products
 *  summed in fp32, as in the FP8 forward.
 *  Requirements: N % 32 == 0, K % 8 == 0; scales 4-byte aligned.
 *  dx  [M, K] bf16 in every case.
 */
int pt_grouped_gemm_dgrad(const void *dy, const uint8_t *dy_scale,
                          const void *b, const uint8_t *b_scale, void *dx,
                          const int64_t *group_lens, const int64_t *group_offs,
                          int64_t G, int64_t M, int64_t N, int64_t K,
                          int dtype, int trans_b,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * FC1 with the fused SwiGLU epilogue that also keeps FC1's output for the
 * backward (the training form of the Primus-Turbo README's fused grouped MLP,
 * "What's New": SwiGLU folded into the grouped GEMM; the SwiGLU backward,
 * pt_grouped_gemm_dgrad_swiglu, reads that output):
 *     c[r, :] = bf16(C[r, :])                        [M, N]  (= PT_EPI_NONE's output)
 *     h[r, j] = bf16(silu(C[r, j]) * C[r, N/2 + j])  [M, N/2] (= PT_EPI_SWIGLU's output,
 *               with the same swiglu_limit clamp)
 * both from one pass over the operands, C = A B_g as pt_grouped_gemm_fwd
 * computes it for the dtype (BF16, MXFP8, MXFP4, FP8 with tensor or row
 * factors; the scale arguments, dtype, trans_b, lengths and workspace as
 * there); each output is bit-identical to the call with that single
 * epilogue.  Requirements: N % 16 == 0, K % 8 == 0 and those of the dtype;
 * a, b, h and c 16-byte aligned.  Runs on the 256 x 256 kernels in every
 * configuration, so MXFP4 with K % 256 != 0 needs the workspace that holds
 * the scale copies (else PT_ERR_UNSUPPORTED).
 */
int pt_grouped_gemm_fwd_swiglu_save(const void *a, const uint8_t *a_scale,
                                    const void *b, const uint8_t *b_scale, void *h, void *c,
                                    const int64_t *group_lens, const int64_t *group_offs,
                                    int64_t G, int64_t M, int64_t N, int64_t K, int dtype, int trans_b,
                                    float swiglu_limit, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Grouped data gradient of FC2 with the SwiGLU backward fused into its
 * epilogue.  The forward computes h[r, j] = silu(g) * u from FC1's output
 * C = [gate | up] (g = C[r, j], u = C[r, K + j]) and feeds h to FC2 (blog
 * "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
 * Primus", section "MegaMoE: fusing communication into the grouped GEMM":
 * SwiGLU between the two grouped GEMMs; Primus-Turbo README, "What's New":
 * the expert MLP with SwiGLU folded into the grouped GEMM).  This call
 * takes FC2's output gradient and returns the gradient of C:
 *     dH[r, j] = bf16( sum_n dY[r, n] * B_g[j, n] )      (as pt_grouped_gemm_dgrad)
 *     dC[r, j]     = bf16( dH * u * s * (1 + g * (1 - s)) )
 *     dC[r, K + j] = bf16( dH * g * s ),   s = 1 / (1 + exp(-g))
 * (the derivative of silu(g) * u; dH is rounded to bf16 first, as the
 * unfused dgrad would store it, and the rest runs in fp32).
 *  dtype    PT_BF16: dy [M, N] bf16 (gradient of FC2's output), b FC2's
 *           weight as in pt_grouped_gemm_fwd (trans_b selects [G,K,N] or
 *           [G,N,K]), the scale arguments NULL.
 *           PT_MXFP8_E4M3, PT_MXFP4_E2M1, PT_FP8_E4M3, PT_FP8_E4M3_ROWWISE:
 *           dy, dy_scale, b, b_scale as pt_grouped_gemm_dgrad takes them
 *           for the dtype (dY quantised along N, the weight's transposed
 *           cache [G, K, N], trans_b = 0), so dH is that call's output; the
 *           low-precision training step of the expert MLP (Primus-Turbo
 *           README, "What's New": FP8 / MXFP8 grouped MLP with SwiGLU folded
 *           into the grouped GEMM; the DeepSeek-V4 blog's knob table lists
 *           swiglu_limit for FP8 and FP4 stability).  MXFP4 with N % 256 !=
 *           0 needs the workspace of pt_grouped_gemm_workspace_size
 *           (PT_OP_DGRAD_SWIGLU, ...), else PT_ERR_UNSUPPORTED.
 *  c_saved  [M, 2K] bf16, FC1's output [gate | up] saved by the forward;
 *  dc       [M, 2K] bf16 output; rows outside every expert are not written.
 *  All four 16-byte aligned.  Requirements: N % 8 == 0, K % 8 == 0.
 *  swiglu_limit  the forward's clamp (see pt_grouped_gemm_fwd; 0 or
 *           infinity for none): g and u are clamped as in the forward, and a
 *           clamped input gets no gradient (dC[r, j] = 0 where g > L,
 *           dC[r, K + j] = 0 where |u| > L).
 *  workspace  optional (may be NULL), as for pt_grouped_gemm_dgrad.
 */
int pt_grouped_gemm_dgrad_swiglu(const void *dy, const uint8_t *dy_scale, const void *b, const uint8_t *b_scale,
                                 const void *c_saved, void *dc,
                                 const int64_t *group_lens, const int64_t *group_offs,
                                 int64_t G, int64_t M, int64_t N, int64_t K, int dtype, int trans_b,
                                 float swiglu_limit, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Grouped weight gradient, accumulated into an fp32 main_grad (PR page
 * "[Megatron-LM] feat: add grouped gemm fp4 support, ...", section "Changes":
 * the weight gradient is always accumulated into weight.main_grad and the
 * weight is flagged as having its gradient added):
 *     D_g[k, n] = sum over expert g's rows r of A[r, k] * dY[r, n]
 *     main_grad[g] = (accumulate ? main_grad[g] : 0) + D_g     (fp32, RNE)
 * The reduction length is the expert's own row count.
 *  a  [M, K] bf16;  dy  [M, N] bf16;
 *  main_grad  trans_out = 0: [G, K, N];  trans_out = 1: [G, N, K]  (fp32)
 *  An expert with no rows leaves its main_grad slice untouched when
 *  accumulating and writes zeros when not.
 *  workspace  optional (may be NULL) for BF16, see
 *             pt_grouped_gemm_workspace_size.  With the full size
 *             (pt_grouped_gemm_workspace_size(PT_OP_WGRAD, ...), any dtype)
 *             the reduction over an expert's tokens is split: with
 *             T = ceil(K/256) * ceil(N/256) output tiles per expert and the
 *             chunk length L = max(512, ceil(M * T / 1024)), an expert with
 *             more than L rows is cut into chunks of L consecutive rows
 *             (the last one shorter); chunk 0 is added into main_grad as an
 *             uncut expert is, each later chunk's fp32 partial sum goes to a
 *             workspace slot, and a second pass adds the partials to
 *             main_grad in chunk order:
 *                 main_grad[g] = fp32(... fp32(fp32(main_grad[g] + S_0) + S_1) ... + S_last)
 *             (S_0 itself accumulated onto main_grad[g] in fp32).  The order
 *             is fixed, so results are deterministic, and within fp32
 *             rounding of the uncut sum.  The split engages only where few
 *             output tiles per expert would leave a long expert as a serial
 *             tail.  A smaller workspace runs every expert uncut.
 *  PT_MXFP8_E4M3 / PT_MXFP4_E2M1: a and dy are codes blocked along tokens
 *  within each expert (pt_mx_quantize_tokens): E4M3 [M, K] / [M, N], or
 *  E2M1 [M, K/2] / [M, N/2], with scales [M/32 + G, K] / [M/32 + G, N];
 *  D_g sums the products of their values (each code times its block's
 *  scale) in fp32 on the scaled matrix instructions, the block scales of
 *  both operands applied per 32 tokens.  The workspace is required:
 *  pt_grouped_gemm_workspace_size(PT_OP_WGRAD, ..., dtype) bytes, else
 *  PT_ERR_WORKSPACE.  It receives both operands transposed to channel
 *  rows (each expert's tokens padded with zero codes to whole blocks of
 *  32), their scales, the experts' starts and the split reduction's
 *  slots; the split's chunk length is L rounded up to a multiple of 256
 *  tokens.
 *  PT_FP8_E4M3: a [M, K] and dy [M, N] E4M3 codes with one fp32 factor
 *  each (a_scale, dy_scale: pt_fp8_quantize, batch 1);
 *      main_grad[g] = (accumulate ? main_grad[g] : 0) + fp32(d_a * d_dy) * S_g
 *  with S_g the fp32 sum of the exact code products (the whole expert's:
 *  no split along tokens), one fused multiply-add per element.  The
 *  workspace is required: both operands' codes transposed to channel rows
 *  as for MXFP8 (no scales) and the experts' starts (the size that
 *  pt_grouped_gemm_workspace_size(PT_OP_WGRAD, ..., PT_FP8_E4M3) gives is
 *  256 bytes more, for pt_grouped_gemm_wgrad_quantize's amax words and
 *  factors; this call needs only the bytes before them),
 *  else PT_ERR_WORKSPACE.  (Row factors vary along the reduction, so
 *  PT_FP8_E4M3_ROWWISE has no weight gradient: PT_ERR_UNSUPPORTED.)
 *  Requirements: K % 8 == 0, N % 8 == 0; dtype PT_BF16, PT_MXFP8_E4M3,
 *  PT_MXFP4_E2M1 or PT_FP8_E4M3.
 */
int pt_grouped_gemm_wgrad(const void *a, const uint8_t *a_scale,
                          const void *dy, const uint8_t *dy_scale,
                          float *main_grad,
                          const int64_t *group_lens, const int64_t *group_offs,
                          int64_t G, int64_t M, int64_t N, int64_t K,
                          int dtype, int trans_out, int accumulate,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * The low-precision weight gradient from the bf16 gradients themselves
 * (Primus-Turbo README, "What's New": MXFP8 grouped MLP backward and FP8
 * grouped GEMM; PR page "[Megatron-LM] feat: add grouped gemm fp4 support,
 * ...", "Changes": the gradient added into weight.main_grad).  a [M, K] and
 * dy [M, N] are bf16, rows grouped by expert as for pt_grouped_gemm_wgrad.
 *  PT_MXFP8_E4M3 / PT_MXFP4_E2M1: both are quantised along tokens within
 *  each expert (blocks of 32 rows, the rule of pt_mx_quantize_tokens)
 *  straight into the workspace's transposed operand layout, then the MX
 *  weight gradient runs: main_grad comes out bit-identical to
 *  pt_mx_quantize_tokens on a and on dy followed by pt_grouped_gemm_wgrad
 *  with that dtype and workspace.
 *  PT_FP8_E4M3: each tensor's amax, then its codes with one factor per
 *  tensor (the rule of pt_fp8_quantize, batch 1, over all M rows) straight
 *  into the transposed layout: bit-identical to pt_fp8_quantize on a and
 *  on dy followed by pt_grouped_gemm_wgrad with PT_FP8_E4M3.
 * The [M, K] and [M, N] codes are neither written nor read back.  Same
 * arguments, layouts (trans_out), accumulate rule, split reduction and
 * errors as pt_grouped_gemm_wgrad; the workspace is required,
 * pt_grouped_gemm_workspace_size(PT_OP_WGRAD, ..., dtype) bytes, else
 * PT_ERR_WORKSPACE.  a, dy and main_grad 16-byte aligned (else
 * PT_ERR_MISALIGNED).  Requirements: K % 8 == 0, N % 8 == 0; another dtype
 * returns PT_ERR_UNSUPPORTED.
 */
int pt_grouped_gemm_wgrad_quantize(const void *a, const void *dy, float *main_grad,
                                   const int64_t *group_lens, const int64_t *group_offs,
                                   int64_t G, int64_t M, int64_t N, int64_t K,
                                   int dtype, int trans_out, int accumulate,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * OCP-MX quantisation of a bf16 matrix x [rows, cols], one block per 32
 * consecutive elements along one axis:
 *   E = clamp(floor(log2(max|v|)) - emax + 127, 0, 254)   (E = 0 for an
 *       all-zero block; emax = 8 for E4M3, 2 for E2M1)
 *   code_i = nearest element-format value to v_i / 2^(E-127), ties to even,
 *            magnitudes beyond the format's maximum saturate, sign kept.
 * (MX weight buffers of the PR page "[Megatron-LM] feat: add grouped gemm fp4
 * support, ...", section "Changes"; the Primus-Turbo README lists MXFP8 and
 * MXFP4 grouped GEMMs under "What's New".)
 *  axis = 1: blocks of 32 consecutive columns of a row (the forward's
 *          reduction-contiguous operands).
 *    q       E4M3: [rows, cols] bytes;  E2M1: [rows, cols/2] bytes (even
 *            column in the low nibble)
 *    scales  [rows, cols/32] E8M0 bytes
 *    Requirements: cols % 32 == 0.
 *  axis = 0: blocks of 32 consecutive rows of a column.
 *    q       E4M3: [rows, cols] bytes (x's layout);  E2M1: [rows/2, cols]
 *            bytes, rows 2i and 2i + 1 of a column sharing byte (i, c), the
 *            even row in the low nibble (pairs along the blocking axis, as
 *            in the axis-1 layout of the transpose)
 *    scales  [rows/32, cols] E8M0 bytes, 4-byte aligned
 *    Requirements: rows % 32 == 0, cols % 8 == 0.
 *  dtype   PT_MXFP8_E4M3 or PT_MXFP4_E2M1; another axis is PT_ERR_INVALID_ARG.
 *  x and q 16-byte aligned.
 *  NaN/Inf inputs are outside the contract (no fault; results unspecified).
 */
int pt_mx_quantize(const void *x, void *q, uint8_t *scales,
                   int64_t rows, int64_t cols, int dtype, int axis, void *stream);

/*
 * pt_mx_quantize along the columns (axis 1) into code rows q_pitch bytes
 * apart instead of packed: row r's codes are bytes [r * q_pitch, r * q_pitch
 * + cols) of q (E4M3) or [r * q_pitch, r * q_pitch + cols/2) (E2M1), the
 * same bytes pt_mx_quantize writes to its row r; the rest of each row is not
 * written.  scales as pt_mx_quantize (packed [rows, cols/32]).  The operand
 * layout for pt_grouped_gemm_fwd_pitched (same MX rule and passages as
 * pt_mx_quantize; the pitch is a storage choice, not part of the method).
 *  q_pitch  bytes between code rows: at least the row's code bytes and a
 *           multiple of 16, else PT_ERR_INVALID_ARG.  q holds
 *           (rows - 1) * q_pitch + the row's code bytes, 16-byte aligned.
 *  Other requirements and errors as pt_mx_quantize with axis = 1.
 */
int pt_mx_quantize_pitched(const void *x, void *q, uint8_t *scales,
                           int64_t rows, int64_t cols, int dtype, int64_t q_pitch, void *stream);

/*
 * Transposing OCP-MX quantisation, the transposed weight cache of the MX
 * data gradient (PR page "[Megatron-LM] feat: add grouped gemm fp4 support,
 * ...", section "Changes": quantised weight buffers kept next to the
 * weight; the data gradient reduces over the weight's other dimension).
 * For each of `batch` bf16 matrices x_b [rows, cols] (row-major, one after
 * another) it writes the quantisation of x_b^T by the rule of
 * pt_mx_quantize: blocks of 32 consecutive rows of x_b, so
 *  q       E4M3: [batch, cols, rows] bytes;  E2M1: [batch, cols, rows/2]
 *  scales  [batch, cols, rows/32] E8M0 bytes.
 * A forward weight [G, N, K] becomes the [G, K, N] operand, packed and
 * scaled along N, that pt_grouped_gemm_dgrad takes for MX.
 *  dtype   PT_MXFP8_E4M3 or PT_MXFP4_E2M1.  Requirements: rows % 32 == 0,
 *          cols % 8 == 0, batch <= 65535; x and q 16-byte aligned.
 */
int pt_mx_quantize_t(const void *x, void *q, uint8_t *scales,
                     int64_t batch, int64_t rows, int64_t cols, int dtype, void *stream);

/*
 * MX quantisation along tokens for the weight gradient (the MX grouped
 * GEMM's backward flow, PR page "[Megatron-LM] feat: add grouped gemm fp4
 * support, ...", Copilot overview; the Primus-Turbo README's "pad-aware
 * paths" keep quantisation blocks inside one expert): within each expert g,
 * rows [off_g, off_g + len_g) of x [M, cols] (bf16) form blocks of 32
 * consecutive rows, the last one partial when len_g % 32 != 0, so no block
 * straddles two experts.  Each block of each column is quantised by the
 * rule of pt_mx_quantize over the rows it has.
 *  q       E4M3: [M, cols] codes (x's layout); E2M1: [M, cols/2], column
 *          2c in the low nibble of byte c, column 2c + 1 in the high one;
 *  scales  [M/32 + G, cols] E8M0: block j of expert g is row
 *          sum over earlier experts of ceil(len/32), plus j; rows past the
 *          last block are left as they are.
 *  group_offs may be NULL (derived by exclusive scan on the device).
 *  dtype   PT_MXFP8_E4M3 or PT_MXFP4_E2M1.  Requirements: cols % 8 == 0; x, q and scales
 *          16-byte aligned.  workspace optional (the error word).
 */
int pt_mx_quantize_tokens(const void *x, const int64_t *group_lens, const int64_t *group_offs, void *q,
                          uint8_t *scales, int64_t G, int64_t M, int64_t cols, int dtype,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * FP8 E4M3 quantisation with one scale per matrix ("current scaling": the
 * scale comes from the tensor being quantised; PR page "[Megatron-LM] feat:
 * add grouped gemm fp4 support, ...", "Description" and "Changes" name
 * current scaling as an FP8 recipe).  For each of `batch` bf16 matrices x_b of
 * rows * cols values (one after another):
 *   amax[b]    = max |x_b|                                   (fp32, exact)
 *   s_b        = 448 / amax[b] in fp32 (1 if amax is 0; the largest finite
 *                fp32 if the quotient overflows)
 *   q_b[i]     = E4M3 code nearest to clamp(fp32(x_b[i] * s_b), -448, 448),
 *                ties to even (OCP E4M3FN)
 *   dequant[b] = fp32(1 / s_b), the factor pt_grouped_gemm_fwd takes
 *  q  [batch, rows, cols] bytes;  amax, dequant  [batch] fp32.
 *  Requirements: cols % 8 == 0, batch <= 65535; x and q 16-byte aligned.
 *  Deterministic: the maximum does not depend on the order of its atomics.
 */
int pt_fp8_quantize(const void *x, void *q, float *amax, float *dequant,
                    int64_t batch, int64_t rows, int64_t cols, void *stream);

/*
 * The same rule with one scale per row: for each row r of x [rows, cols]
 * (bf16), amax[r] = max |x[r, :]|, s_r = 448 / amax[r], codes as in
 * pt_fp8_quantize, dequant[r] = fp32(1 / s_r).  For B of a rowwise FP8
 * GEMM pass the weights [G, N, K] as rows = G * N, cols = K.
 *  q  [rows, cols] bytes;  amax, dequant  [rows] fp32.
 *  Requirements: cols % 8 == 0; x and q 16-byte aligned.
 */
int pt_fp8_quantize_rows(const void *x, void *q, float *amax, float *dequant,
                         int64_t rows, int64_t cols, void *stream);

/*
 * Expert weight stack in one pass (the Primus DeepSeek-V4-Flash blog,
 * "Performance optimizations", kernel-fusion table: the grouped expert weight
 * stack replaces a stack, a transpose and a contiguous copy -- two full
 * passes over the per-expert weights -- with one kernel).
 *  experts  device array of G device addresses; expert g's weight W_g is a
 *           bf16 [rows, cols] row-major matrix, 16-byte aligned.  A NULL or
 *           misaligned address reads as a zero matrix and sets error bit 3
 *           in the workspace's error word (pt_read_error_flags).
 *  out      transpose = 0: [G, rows, cols], out[g] = W_g;
 *           transpose = 1: [G, cols, rows], out[g] = W_g^T.
 *           With W_g = an expert's [out, in] linear weight, transpose = 1
 *           gives the [G, K, N] operand of pt_grouped_gemm_fwd (trans_b 0)
 *           and transpose = 0 the [G, N, K] one (trans_b 1).
 *  Requirements: rows % 8 == 0, cols % 8 == 0, G <= 65535; out 16-byte
 *  aligned, experts 8-byte aligned.  workspace optional (the error word).
 */
int pt_stack_experts(const void *const *experts, void *out, int64_t G, int64_t rows, int64_t cols, int transpose,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * The MX weight caches straight from per-expert weights, one read of each
 * (the same kernel-fusion table's single-pass weight stack, fused with the
 * quantised weight buffers that the PR page "[Megatron-LM] feat: add grouped
 * gemm fp4 support, ...", section "Changes", keeps next to the weight):
 *  q, scales      the forward cache, pt_mx_quantize of each W_g along its
 *                 columns: E4M3 [G, rows, cols] / E2M1 [G, rows, cols/2]
 *                 codes, [G, rows, cols/32] scales (cols % 32 == 0);
 *  q_t, scales_t  the data gradient's transposed cache, pt_mx_quantize_t
 *                 of each W_g: E4M3 [G, cols, rows] / E2M1 [G, cols, rows/2]
 *                 codes, [G, cols, rows/32] scales (rows % 32 == 0).
 * Either pair may be NULL (not both).  experts as for pt_stack_experts (a
 * bad address quantises a zero matrix and sets error bit 3).
 *  dtype   PT_MXFP8_E4M3 or PT_MXFP4_E2M1.  Requirements: rows % 8 == 0,
 *          cols % 8 == 0, G <= 65535; q and q_t 16-byte aligned.
 */
int pt_mx_quantize_experts(const void *const *experts, void *q, uint8_t *scales, void *q_t, uint8_t *scales_t,
                           int64_t G, int64_t rows, int64_t cols, int dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Workspace of the grouped GEMMs (optional, for every op; recommended):
 * pt_grouped_gemm_workspace_size() bytes of device memory, 256-byte aligned
 * (4-byte alignment is enough for the error word and tile queues alone).
 *  - the BF16 and MX weight gradients' full size adds the split
 *    reduction's partial slots: floor(M / L) fp32 [K, N] matrices (L as at
 *    pt_grouped_gemm_wgrad), after the MX transposed operands; the FP8
 *    weight gradient's holds its transposed codes;
 *  - word 0 receives the sticky device error bits (pt_read_error_flags);
 *    a workspace of at least 4 bytes is enough for that alone;
 *  - a workspace of the full size also holds the tile queues: every call
 *    then first zeroes them on `stream` (a one-wave kernel) and the GEMM's
 *    persistent workgroups take their tiles from them, in an order that
 *    keeps the workgroups sharing an expert's rows close together in time.
 *    Without them the tiles go in a fixed round-robin order.  Results are
 *    bit-identical either way.
 * The library keeps nothing in the workspace between calls; calls that may
 * run concurrently (on different streams) need separate workspaces.  Its
 * contents on entry do not matter.
 */
/* Bytes of workspace `op` needs for these sizes. */
size_t pt_grouped_gemm_workspace_size(int op, int64_t G, int64_t M, int64_t N,
                                      int64_t K, int dtype);

/*
 * Kernel configurations and tuning (the Primus-Turbo README, "What's New":
 * grouped GEMM autotune).  A configuration of one grouped GEMM call is a
 * number 0..3: bit 0 takes tiles in the static order even when the
 * workspace holds tile queues, bit 1 runs the 128 x 256 kernel instead of
 * the 256 x 256 one (BF16 and MX only; FP8 with tensor or row factors and the
 * SwiGLU backward have no 128 x 256 kernel, and a bit that does not apply is
 * dropped).  Every configuration computes the same sums in the same order:
 * results are bit-identical, only speed differs.
 * pt_set_gemm_config sets the process-wide mode and returns the previous one
 * (-3 for an unknown mode):
 *   PT_CONFIG_RULES  configuration 0 (the default), or configuration 1 (the
 *                    static order, one launch fewer) for a problem whose
 *                    every 256 x 256 tile can start at once: at most one
 *                    tile per compute unit, counted with M rounded up to a
 *                    power of two;
 *   PT_CONFIG_TUNE   the first call of each problem class -- (device, op,
 *                    dtype, epilogue, layout, G, N, K, and M rounded up to a
 *                    power of two) -- times every configuration that applies
 *                    on the call's own buffers (one warm-up and three timed
 *                    launches each, then a stream synchronisation) and
 *                    keeps the fastest; later calls of the class use it.
 *                    The call's outputs come from the chosen configuration.
 *                    A call that must not run twice (a weight gradient that
 *                    accumulates) or a stream under graph capture is not
 *                    timed: it uses its class's choice if there is one,
 *                    else the rules' configuration;
 *   0..3             that configuration for every call.
 * pt_gemm_config_of returns the tuned configuration of a problem class (the
 * arguments of the entry point; op PT_OP_DGRAD_SWIGLU for the SwiGLU
 * backward), or -1 if it has none.  pt_clear_gemm_tuning forgets every
 * tuned class.  The table holds 512 classes; once it is full, a class not
 * in it is not timed and takes the rules' configuration.
 */
#define PT_CONFIG_RULES (-1)
#define PT_CONFIG_TUNE (-2)
int pt_set_gemm_config(int config);
int pt_gemm_config_of(int op, int dtype, int epilogue, int trans, int64_t G, int64_t M, int64_t N, int64_t K);
void pt_clear_gemm_tuning(void);

/*
 * Sticky device error bits recorded in the first word of a workspace by the
 * grouped GEMM kernels (bit 0: a negative group length; bit 1: an expert
 * range outside [0, M] was clamped; bit 2: without group_offs, the lengths
 * do not sum to M; with group_offs, two experts' ranges overlap or come out
 * of expert order, offs[g] + lens[g] > offs[g + 1], or offs[G] lies outside
 * [0, M]) and by the expert-weight kernels (bit 3: an expert address was
 * NULL or not 16-byte aligned).  Rows between experts' ranges that no
 * expert owns (explicit offsets with gaps) are valid input and set no bit:
 * the forward and data gradient leave them unwritten, the weight gradient
 * and the token quantiser do not read them.
 * The caller zeroes the word before the calls it wants to check.  This call
 * synchronises `stream` and copies the word to *flags (host pointer).
 */
int pt_read_error_flags(const void *workspace, void *stream, uint32_t *flags);

/* Human-readable name of a pt_status. */
const char *pt_status_string(int status);

/* Library version string. */
const char *pt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PTGG_H */
