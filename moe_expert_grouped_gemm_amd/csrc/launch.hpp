// launch.hpp -- internal launcher interface between the C ABI and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptgg {

// C[m, j] = sum_q A[m, q] * Bop(j, q) per expert (forward and dgrad), or
// D[i, j] = sum over the expert's rows r of A[r, i] * B[r, j] (wgrad).
struct Bf16Params {
    const uint16_t *a;
    const uint16_t *b;
    void *out;
    uint8_t *out_scale;  // SwiGLU -> MXFP4 epilogue only
    const int64_t *lens;
    const int64_t *offs;
    uint32_t *err;
    int G;
    int64_t M;
    int Kred;          // fwd/dgrad: reduction length
    int Nout;          // output columns before the epilogue
    int Mout;          // wgrad: output rows per expert
    int lda, ldb;      // leading dimensions (elements)
    int64_t b_gstride; // fwd/dgrad: elements between experts' weight matrices
    int ldo;           // output leading dimension (elements)
    int64_t o_gstride; // wgrad: elements between experts' main_grad slices
    int tilesN;
    int tilesM;        // wgrad only
    int accumulate;    // wgrad only
    uint32_t *sched;   // tile-queue counters in the workspace, or null (static order)
    const uint16_t *aux; // SwiGLU backward: the FC1 output [gate | up] the epilogue reads
    int ldaux;           // its row stride (elements)
    int narrow;          // 1: the 128 x 256 kernel (not for kEpiDSwiglu / kEpiSwigluSave), 0: the 256 x 256 one
    float swiglu_limit;  // SwiGLU clamp (forward and backward epilogues); +inf for none
    uint16_t *save;      // kEpiSwigluSave: the GEMM output [M, Nout] bf16 (gate | up) kept for the backward
    int ldsave;          // its row stride (elements)
    int split_len;       // wgrad: token chunk length of the split reduction, or 0 (one chunk per expert)
    float *partials;     // wgrad with split_len: nslots fp32 [Mout, Nout] partial sums in the workspace
    int nslots;
};

enum Bf16Kind { kFwdKContig = 0, kFwdNContig = 1, kWgrad = 2 };
// kEpiDSwiglu: the SwiGLU backward on a data gradient dH (see store_tile_lds_w).
// kEpiSwigluSave: the SwiGLU output, and the bf16 GEMM output itself to Bf16Params::save.
// kEpiWgrad (MX kernel): the weight gradient, fp32 tiles accumulated into main_grad.
enum Epi { kEpiNone = 0, kEpiSwiglu = 1, kEpiSwigluMxfp4 = 2, kEpiDSwiglu = 3, kEpiSwigluSave = 4, kEpiWgrad = 5 };
// Does the epilogue pair gate and up columns of one tile?
constexpr bool epi_glu(int epi) { return epi == kEpiSwiglu || epi == kEpiSwigluMxfp4 || epi == kEpiSwigluSave; }

hipError_t launch_bf16(const Bf16Params &p, int kind, int epi, hipStream_t s);
// Split weight gradient, second pass: for every expert cut into more than one
// token chunk, main_grad[g] += the partial sums of chunks 1, 2, ... in order.
hipError_t launch_wgrad_split_reduce(const Bf16Params &p, hipStream_t s);
int bf16_tile_m(int narrow);
int bf16_tile_n();

struct MxParams {
    const uint8_t *a;        // [M, K] codes (E4M3) or [M, K/2] (E2M1)
    const uint8_t *as;       // [M, K/32]
    const uint8_t *b;        // [G, N, K(/2)]
    const uint8_t *bs;       // [G, N, K/32]
    void *out;
    uint8_t *out_scale;
    const int64_t *lens;
    const int64_t *offs;
    uint32_t *err;
    int G;
    int64_t M;
    int N, K;
    int ldo;                 // output row stride (elements for bf16, bytes for MXFP4)
    int tilesN;
    uint32_t *sched;         // tile-queue counters in the workspace, or null (static order)
    const uint32_t *sa;      // stage-major copies of as / bs in the workspace, or null
    const uint32_t *sb;
    const float *sfa;        // FP8 with tensor scales: A's fp32 scale (1 value), or null (MX)
    const float *sfb;        // and each expert's B scale [G]
    int sf_rows;             // sfa / sfb hold one scale per row of A [M] and per row of B [G, N]
    int narrow;              // 1: the 128 x 256 kernel on row-major scales (MX only), 0: rules
    float swiglu_limit;      // SwiGLU clamp; +inf for none
    uint16_t *save;          // kEpiSwigluSave: the GEMM output [M, N] bf16 (gate | up)
    int ldsave;              // its row stride (elements)
    const uint16_t *aux;     // kEpiDSwiglu: FC1's saved output [gate | up] [M, 2N] bf16
    int ldaux;               // its row stride (elements)
    // kEpiWgrad: a / b are the two gradients' codes transposed to channel
    // rows [wrows / wcols, pitch bytes] (launch_mx_tokens_transpose), sa / sb
    // their stage-major scale words (FP8 with tensor factors: none; sfa[0]
    // and sfb[0] are the two gradients' factors), plan the experts' block and
    // stage starts; out is main_grad, fp32 [G][wrows][ldo] at o_gstride
    // elements
    const int *plan;
    int64_t pitch;           // also the forward's: code bytes between rows of A and of B, or 0 (packed)
    int wrows, wcols;
    int64_t o_gstride;
    int tilesM;
    int accumulate;
    int split_len;           // split reduction: chunk length in padded tokens (a multiple of 256), or 0
    float *partials;         // nslots fp32 [wrows, wcols] partial sums in the workspace
    int nslots;
};

hipError_t launch_mx(const MxParams &p, int fmt, int epi, hipStream_t s);
// The MX weight gradient (p as for kEpiWgrad) on the 256 x 256 kernel: fmt
// 0 MXFP8, 1 MXFP4, 2 E4M3 codes with one factor per tensor.
hipError_t launch_mx_wgrad(const MxParams &p, int fmt, hipStream_t s);

// Stage-major copy of a row-major E8M0 scale matrix [rows, K/32] for the
// 256 x 256 MX kernel (layout at mx_scale_swizzle): mx_swizzle_bytes() bytes
// at `out`.  kMxSwzMaxK bounds K.
constexpr int64_t kMxSwzMaxK = 16384;
int64_t mx_swizzle_bytes(int64_t rows, int64_t K, int fmt);
hipError_t launch_mx_scale_swizzle(const uint8_t *scales, int64_t rows, int64_t K, int fmt, uint32_t *out,
                                   hipStream_t s);
int mx_tile_m();
int mx_wide_tile();      // rows and columns of the 256 x 256 MX kernel's tile
int mx_tile_n();

// Tile queues of the persistent kernels: kQueues counters, kQueueStride
// 32-bit words apart, starting kQueueWsOffset bytes into the caller's
// workspace (whose first word holds the error bits).
constexpr int kQueues = 8;
constexpr int kQueueStride = 32;
constexpr int kQueueWsOffset = 256;
constexpr int kQueueWsBytes = kQueueWsOffset + kQueues * kQueueStride * 4;

// Zero the tile-queue counters at `sched` on stream s (a one-wave kernel:
// a memset node would not be safe to capture in a graph).
hipError_t launch_queue_reset(uint32_t *sched, hipStream_t s);

// Blocks of 32 along the columns; code rows q_pitch bytes apart (0: packed).
hipError_t launch_quantize(const uint16_t *x, uint8_t *q, uint8_t *scales,
                           int64_t rows, int64_t cols, int fmt, hipStream_t s, int64_t q_pitch = 0);
// Blocks of 32 along the rows (axis 0): x [rows, cols] bf16 -> E4M3
// [rows, cols] / E2M1 [rows/2, cols] codes (row pairs share a byte, even row
// low) and [rows/32, cols] scales; rows % 32 == 0, cols % 4 == 0.
hipError_t launch_quantize_cols(const uint16_t *x, uint8_t *q, uint8_t *scales, int64_t rows, int64_t cols, int fmt,
                                hipStream_t s);
// batch x [rows, cols] bf16 -> the quantisation of each matrix's transpose:
// [cols, rows] codes (blocks of 32 along rows) and [cols, rows/32] scales.
hipError_t launch_quantize_t(const uint16_t *x, uint8_t *q, uint8_t *scales, int64_t batch, int64_t rows,
                             int64_t cols, int fmt, hipStream_t s);
// FP8 E4M3 with one scale per matrix (current scaling) for batch matrices of
// n bf16 values each: amax[b] = max|x_b|, q = e4m3(x * 448 / amax[b]),
// dequant[b] = amax-derived factor that multiplies the codes back.
hipError_t launch_fp8_quantize(const uint16_t *x, uint8_t *q, float *amax, float *dequant, int64_t batch,
                               int64_t n, hipStream_t s);
// The same with one scale per row of x [rows, cols].
hipError_t launch_fp8_quantize_rows(const uint16_t *x, uint8_t *q, float *amax, float *dequant, int64_t rows,
                                    int64_t cols, hipStream_t s);
// MX along tokens within each expert (blocks of 32 rows, the last
// partial), codes E4M3 [M, C] / E2M1 [M, C/2] (fmt 0 / 1) and scales
// [M / 32 + G, C].
hipError_t launch_mx_quantize_tokens(const uint16_t *x, const int64_t *lens, const int64_t *offs, int G, int64_t M,
                                     int64_t C, int fmt, uint8_t *q, uint8_t *scales, uint32_t *err, hipStream_t s);
// The MX weight gradient's operands: token-blocked codes [M, C(/2)] and
// scales [M/32 + G, C] -> channel rows qt [C, pitch] (each expert's tokens
// padded to whole blocks, expert g from byte 32 (E4M3) / 16 (E2M1) *
// bstart_g) and stage-major scale words st (global stage S_g + kt of expert
// g: word ((S_g + kt) * C + c) * WPR + w); plan[2g] = bstart_g, plan[2g+1] =
// S_g.  mx_wgrad_pitch / mx_wgrad_stages bound the row bytes and the stages
// for any lengths summing to at most M.
// scales == nullptr (codes without block scales): no scale words.
int64_t mx_wgrad_pitch(int64_t M, int G, int fmt);
int64_t mx_wgrad_stages(int64_t M, int G, int fmt);
hipError_t launch_mx_tokens_transpose(const uint8_t *q, const uint8_t *scales, const int64_t *lens,
                                      const int64_t *offs, int G, int64_t M, int64_t C, int fmt, uint8_t *qt,
                                      int64_t pitch, uint32_t *st, int *plan, hipStream_t s);
// The same operands straight from bf16 x [M, C] (quantisation along tokens
// and the transpose in one pass, bit-identical to launch_mx_quantize_tokens then
// launch_mx_tokens_transpose); err may be null.  fmt 2: E4M3 with one factor
// per tensor from amax[0] (launch_fp8_amax; bit-identical to
// launch_fp8_quantize then the transpose without scales), the dequantisation
// factor written to dequant[0]; st unused.
hipError_t launch_mx_tokens_quant_t(const uint16_t *x, const int64_t *lens, const int64_t *offs, int G, int64_t M,
                                    int64_t C, int fmt, uint8_t *qt, int64_t pitch, uint32_t *st, int *plan,
                                    uint32_t *err, const uint32_t *amax, float *dequant, hipStream_t s);
// max |x| over n bf16 values as fp32 bits into amax[0] (zeroed first).
hipError_t launch_fp8_amax(const uint16_t *x, uint32_t *amax, int64_t n, hipStream_t s);
// Expert weight stack: G separate bf16 matrices (a device array of their
// addresses) -> [G, R, C], or [G, C, R] with trans; and their MX caches
// along C ([G, R, C(/2)] + [G, R, C/32]) and/or along R of the transpose
// ([G, C, R(/2)] + [G, C, R/32]) in one read of each weight.
hipError_t launch_stack_experts(const void *const *ptrs, uint16_t *out, int G, int64_t R, int64_t C, int trans,
                                uint32_t *err, hipStream_t s);
hipError_t launch_mx_quantize_experts(const void *const *ptrs, uint8_t *q, uint8_t *scales, uint8_t *qt,
                                      uint8_t *scales_t, int G, int64_t R, int64_t C, int fmt, uint32_t *err,
                                      hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cus();

}  // namespace ptgg
