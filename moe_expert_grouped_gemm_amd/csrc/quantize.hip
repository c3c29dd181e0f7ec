// quantize.hip -- OCP-MX quantisation of a bf16 matrix along its rows:
// bf16 [rows, cols] -> E4M3 [rows, cols] or E2M1 x2 [rows, cols/2], plus one
// E8M0 scale byte per 32 consecutive values.
//
// Streaming kernel: four lanes share one 32-value block (8 values = 16 bytes
// each, so a wave reads 1 KiB of consecutive input per load), and the
// block's largest magnitude is combined across the four lanes with two DPP
// quad permutes.  The shared exponent E comes from the amax bits by integer
// arithmetic (common.hpp).  Each value is then scaled by 2^(127 - E) with
// v_ldexp_f32 (exact: a power of two, and every value that can reach a
// non-zero code stays a normal fp32 number), clamped to the element grid's
// largest magnitude, and converted by the gfx950 conversion instructions,
// which round to nearest even.  An exhaustive check on the device (every
// bf16 pattern against every scale byte the rule can produce with it: 8.9M
// E4M3 and 8.5M E2M1 pairs) found the result identical to the integer
// encoder in common.hpp, which follows the rounding rule step by step.
#include "common.hpp"
#include "launch.hpp"

namespace ptgg {

namespace {

// Largest magnitude over the 4 consecutive lanes of a quad.
__device__ __forceinline__ uint32_t quad_max(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));  // lanes ^ 1
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));  // lanes ^ 2
    return x;
}

// Quantise 8 consecutive values (one lane's share of a block).  Codes that
// consecutive lanes write to whole lines (NT) are stored with the
// non-temporal policy; the transposing kernels' codes fill half lines, which
// the default policy merges in L2 before they reach memory.
template <int FMT, bool NT = true>
__device__ __forceinline__ uint32_t encode8(const uintx4 v, uint8_t *__restrict__ q, int64_t t)
{
    constexpr int EMAX = FMT == 0 ? 8 : 2;
    constexpr float LIM = FMT == 0 ? 448.0f : 6.0f;
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = max(amax, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
    amax = quad_max(amax);
    const uint32_t E = mx_scale_byte<EMAX>(amax);
    const int e = 127 - (int)E;
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __builtin_ldexpf(bf16_to_f32(v[i] & 0xFFFFu), e);
        f[2 * i + 1] = __builtin_ldexpf(bf16_to_f32(v[i] >> 16), e);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = __builtin_fminf(__builtin_fmaxf(f[i], -LIM), LIM);
    if (FMT == 0) {
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
        if constexpr (NT)
            __builtin_nontemporal_store(uintx2{(uint32_t)w0, (uint32_t)w1}, (uintx2 *)(q + t * 8));
        else
            *(uintx2 *)(q + t * 8) = uintx2{(uint32_t)w0, (uint32_t)w1};
    } else {
        uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f[0], f[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], 1.0f, 3);
        if constexpr (NT)
            __builtin_nontemporal_store(w, (uint32_t *)(q + t * 4));
        else
            *(uint32_t *)(q + t * 4) = w;
    }
    return E;
}

// The same, and lane 0 of the quad stores the block's scale byte.
template <int FMT, bool NT = true>
__device__ __forceinline__ void quantise8(const uintx4 v, uint8_t *__restrict__ q, uint8_t *__restrict__ scales,
                                          int64_t t)
{
    const uint32_t E = encode8<FMT, NT>(v, q, t);
    if ((t & 3) == 0) scales[t >> 2] = (uint8_t)E;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(const uint16_t *__restrict__ x,
                                                               uint8_t *__restrict__ q,
                                                               uint8_t *__restrict__ scales,
                                                               int64_t nquads, int64_t gpr, int64_t extra)
{
    // t indexes 8-value groups (a block is 4 consecutive t, in 4 consecutive
    // lanes); two groups per iteration, a whole grid apart, keep two loads
    // in flight per lane.  Code rows `extra` bytes longer than the packed
    // row (gpr groups per row) move group t's codes by `extra` per row before
    // it.
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; t + stride < nquads; t += 2 * stride) {
        const uintx4 v0 = __builtin_nontemporal_load((const uintx4 *)(x + t * 8));
        const uintx4 v1 = __builtin_nontemporal_load((const uintx4 *)(x + (t + stride) * 8));
        quantise8<FMT>(v0, extra ? q + (t / gpr) * extra : q, scales, t);
        quantise8<FMT>(v1, extra ? q + ((t + stride) / gpr) * extra : q, scales, t + stride);
    }
    if (t < nquads)
        quantise8<FMT>(__builtin_nontemporal_load((const uintx4 *)(x + t * 8)), extra ? q + (t / gpr) * extra : q,
                       scales, t);
}

// Quantisation along the columns (axis 0): blocks of 32 consecutive rows of
// one column.  x [R, C] bf16 -> E4M3 [R, C] codes (x's layout) or E2M1
// [R/2, C] (rows 2i and 2i + 1 of a column share a byte, the even row in
// the low nibble), scales [R/32, C].  One thread per 4 columns of a 32-row
// block, so a wave reads 512 consecutive bytes of each of the block's rows
// and stores whole words; the four columns' values stay in registers between
// the amax and the encode, which takes the row quantiser's steps (ldexp by
// 2^(127 - E), clamp to the grid maximum, hardware nearest-even convert).
// R % 32 == 0, C % 4 == 0; grid (column groups, row blocks), the row blocks
// strided by gridDim.y.
template <int FMT>
__global__ __launch_bounds__(kThreads) void mx_quantize_cols_kernel(const uint16_t *__restrict__ x,
                                                                    uint8_t *__restrict__ q,
                                                                    uint8_t *__restrict__ scales, int64_t R,
                                                                    int64_t C)
{
    constexpr int EMAX = FMT == 0 ? 8 : 2;
    constexpr float LIM = FMT == 0 ? 448.0f : 6.0f;
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;     // group of 4 columns
    if (c >= C / 4) return;
    for (int64_t blk = blockIdx.y; blk < R / 32; blk += gridDim.y) {
        const int64_t r0 = blk * 32;
        uintx2 h[32];
        uint32_t am[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            h[i] = __builtin_nontemporal_load((const uintx2 *)(x + (r0 + i) * C + 4 * c));
#pragma unroll
            for (int k = 0; k < 4; ++k) am[k] = max(am[k], (h[i][k >> 1] >> (16 * (k & 1))) & 0x7FFFu);
        }
        int e[4];
        uint32_t Ew = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t E = mx_scale_byte<EMAX>(am[k]);
            e[k] = 127 - (int)E;
            Ew |= E << (8 * k);
        }
        auto val = [&](int i, int k) {
            const float f = __builtin_ldexpf(bf16_to_f32((h[i][k >> 1] >> (16 * (k & 1))) & 0xFFFFu), e[k]);
            return __builtin_fminf(__builtin_fmaxf(f, -LIM), LIM);
        };
        if (FMT == 0) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(val(i, 0), val(i, 1), 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(val(i, 2), val(i, 3), w, true);
                __builtin_nontemporal_store((uint32_t)w, (uint32_t *)(q + (r0 + i) * C + 4 * c));
            }
        } else {
            // byte k of a word: column 4c + k, rows 2i (low nibble) and 2i + 1
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, val(2 * i, 0), val(2 * i + 1, 0), 1.0f, 0);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(2 * i, 1), val(2 * i + 1, 1), 1.0f, 1);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(2 * i, 2), val(2 * i + 1, 2), 1.0f, 2);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(2 * i, 3), val(2 * i + 1, 3), 1.0f, 3);
                __builtin_nontemporal_store(w, (uint32_t *)(q + (r0 / 2 + i) * C + 4 * c));
            }
        }
        *(uint32_t *)(scales + blk * C + 4 * c) = Ew;
    }
}

// Transposing quantiser: x_b [R, C] bf16 (row-major) -> q_b = the MX
// quantisation of x_b^T, [C, R] codes with blocks of 32 consecutive rows of
// x_b, and scales [C, R/32].  A workgroup moves a 128 x 128 tile through LDS
// (16-byte row loads), then 16 lanes take one column's 128 rows (8 per
// lane, read down the column, four 32-row blocks of four lanes each), and
// quantise8 encodes them: the column's codes are one 128-byte run of the
// transposed output (E4M3), written by one store of those 16 lanes.  With
// 64 x 64 tiles two workgroups wrote the halves of each run.
// R % 32 == 0, C % 8 == 0.
constexpr int TB = 128;                // tile rows and columns
constexpr int TB_RS = TB * 2;          // LDS row stride (bytes): 16 chunks of 16

// LDS tiles of bf16 rows, 256 bytes each: 16-byte chunk c of row r sits at
// chunk position c ^ ((r / 8) % 16).  The readers take one column per 16
// lanes (lane l: rows 8 l .. 8 l + 7, four columns per wave), so the 16 rows
// a read instruction touches for one column fall in 16 different chunks:
// 64 distinct banks, where a padded row stride left rows 8 apart two to a
// bank (40% of the LDS cycles of the fused token quantiser in conflicts;
// the kernels' times did not move, they wait on memory).  Rows stay whole
// 16-byte chunks, so the row-wise 16-byte writes are unchanged.
__device__ __forceinline__ uint8_t *tb_chunk(uint8_t *tile, int r, int c)
{
    return tile + r * TB_RS + 16 * (c ^ ((r >> 3) & 15));
}
// bf16 element (r, col) of such a tile
__device__ __forceinline__ uint32_t tb_elem(const uint8_t *tile, int r, int col)
{
    return *(const uint16_t *)(tile + r * TB_RS + 16 * ((col >> 3) ^ ((r >> 3) & 15)) + (col & 7) * 2);
}

// This thread's eight 16-byte row chunks of a 128 x 128 tile (zeros outside
// x_b): chunk k = threadIdx.x + j * kThreads is row k / 16, columns
// 8 (k % 16) .. + 7, so a lane quad holds 32 consecutive columns of a row.
__device__ __forceinline__ void load_rows_tb(const uint16_t *xb, int64_t R, int64_t C, int64_t r0, int64_t c0,
                                             uintx4 (&v)[8])
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int k = threadIdx.x + j * kThreads;
        const int row = k >> 4, c8 = (k & 15) * 8;
        v[j] = uintx4{0u, 0u, 0u, 0u};
        if (xb && r0 + row < R && c0 + c8 < C)
            v[j] = __builtin_nontemporal_load((const uintx4 *)(xb + (r0 + row) * C + c0 + c8));
    }
}

__device__ __forceinline__ void rows_to_lds_tb(const uintx4 (&v)[8], uint8_t *tile)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int k = threadIdx.x + j * kThreads;
        uint32_t *d = (uint32_t *)tb_chunk(tile, k >> 4, k & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = v[j][e];
    }
}

// The transposed codes of a 128 x 128 LDS tile at rows r0, columns c0 of
// x_b: pass p, lane t of the workgroup takes column 16 p + t / 16 and rows
// 8 (t % 16) .. + 7.  Whole lane quads (one 32-row block) are in or out
// together (R % 32 == 0), so the DPP exchange in quantise8 only ever pairs
// active lanes.
template <int FMT>
__device__ __forceinline__ void quantise_t_tile(const uint8_t *tile, uint8_t *qb, uint8_t *sb, int64_t R, int64_t C,
                                                int64_t r0, int64_t c0)
{
    const int64_t RB = R / 8;          // 8-value groups per output row
#pragma unroll 2
    for (int p = 0; p < TB * 16 / kThreads; ++p) {
        const int t = threadIdx.x + p * kThreads;
        const int col = t >> 4, rr = (t & 15) * 8;
        uintx4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = tb_elem(tile, rr + 2 * e, col);
            const uint32_t hi = tb_elem(tile, rr + 2 * e + 1, col);
            w[e] = lo | (hi << 16);
        }
        if (c0 + col < C && r0 + (rr & ~31) < R) quantise8<FMT, false>(w, qb, sb, (c0 + col) * RB + (r0 + rr) / 8);
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void mx_quantize_t_kernel(const uint16_t *__restrict__ x,
                                                                 uint8_t *__restrict__ q,
                                                                 uint8_t *__restrict__ scales, int64_t R, int64_t C)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[TB * TB_RS];
    const int64_t b = blockIdx.z;
    const int64_t r0 = (int64_t)blockIdx.y * TB, c0 = (int64_t)blockIdx.x * TB;
    uintx4 v[8];
    load_rows_tb(x + b * R * C, R, C, r0, c0, v);
    rows_to_lds_tb(v, tile);
    __syncthreads();
    quantise_t_tile<FMT>(tile, q + b * C * (FMT == 0 ? R : R / 2), scales + b * C * (R / 32), R, C, r0, c0);
}

// ------------------------------------------------------------------ FP8, one scale per tensor
// Current scaling: each matrix b of a batch gets s_b = 448 / max|x_b| (fp32
// division; 1 for an all-zero matrix, the largest finite fp32 if the quotient
// overflows), codes e4m3(clamp(x * s_b, -448, 448)) rounded to nearest even,
// and the dequantisation factor 1 / s_b.  Pass 1 reduces max|x| into amax[b]
// with an integer atomic max on the fp32 bits (for non-negative values the
// bit order is the numeric order, so the result is exact and independent of
// the order of the atomics); pass 2 encodes.

__global__ void fp8_amax_zero_kernel(uint32_t *amax, int64_t batch)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b < batch) __hip_atomic_store(amax + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// grid (chunks, batch): each thread folds 8-value groups, each wave combines
// its lanes with xor shuffles and issues one atomic.
__global__ __launch_bounds__(kThreads) void fp8_amax_kernel(const uint16_t *__restrict__ x, uint32_t *amax,
                                                            int64_t n8)
{
    const int64_t b = blockIdx.y;
    const uint16_t *xb = x + b * n8 * 8;
    uint32_t m = 0;
    // four 16-byte loads in flight per lane, a grid apart (one took 150 us
    // for A [65536, 2880], four 115); the default cache policy, so that the
    // encode pass right after finds part of x in the last-level cache
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; t + 3 * stride < n8; t += 4 * stride) {
        uintx4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const uintx4 *)(xb + (t + u * stride) * 8);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = max(m, max(v[u][i] & 0x7FFFu, (v[u][i] >> 16) & 0x7FFFu));
    }
    for (; t < n8; t += stride) {
        const uintx4 v = *(const uintx4 *)(xb + t * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
    // one atomic per workgroup: the waves' maxima meet in LDS first (the
    // device-wide atomics on one word serialise, and most waves finish at once)
    __shared__ uint32_t wave_max[kThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) m = max(m, wave_max[w]);
        // bf16 magnitude bits -> fp32 bits of the same value
        __hip_atomic_fetch_max(amax + b, m << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ float fp8_tensor_scale(float amax)
{
    if (amax == 0.0f) return 1.0f;
    const float s = 448.0f / amax;
    return s > 3.402823466e+38f ? 3.402823466e+38f : s;
}

__global__ __launch_bounds__(kThreads) void fp8_encode_kernel(const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
                                                              const uint32_t *amax, float *dequant, int64_t n8)
{
    const int64_t b = blockIdx.y;
    const float s = fp8_tensor_scale(__uint_as_float(amax[b]));
    if (blockIdx.x == 0 && threadIdx.x == 0) dequant[b] = 1.0f / s;
    const uint16_t *xb = x + b * n8 * 8;
    uint8_t *qb = q + b * n8 * 8;
    for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < n8; t += (int64_t)gridDim.x * kThreads) {
        const uintx4 v = __builtin_nontemporal_load((const uintx4 *)(xb + t * 8));
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __builtin_fminf(__builtin_fmaxf(bf16_to_f32(v[i] & 0xFFFFu) * s, -448.0f), 448.0f);
            f[2 * i + 1] = __builtin_fminf(__builtin_fmaxf(bf16_to_f32(v[i] >> 16) * s, -448.0f), 448.0f);
        }
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
        __builtin_nontemporal_store(uintx2{(uint32_t)w0, (uint32_t)w1}, (uintx2 *)(qb + t * 8));
    }
}

// One scale per row: a wave per row, one pass for the amax (a wave
// reduction, no atomics) and one for the codes, which reads the row again
// (rows longer than 8192 values; shorter ones take the kernel below).
__global__ __launch_bounds__(kThreads) void fp8_rows_kernel(const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
                                                            float *amax, float *dequant, int64_t rows, int64_t cols)
{
    const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int lane = threadIdx.x & 63;
    const uint16_t *xr = x + r * cols;
    uint32_t m = 0;
    for (int64_t c = lane * 8; c < cols; c += 512) {
        const uintx4 v = *(const uintx4 *)(xr + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
    const float mf = __uint_as_float(m << 16);
    const float s = fp8_tensor_scale(mf);
    if (lane == 0) {
        amax[r] = mf;
        dequant[r] = 1.0f / s;
    }
    uint8_t *qr = q + r * cols;
    for (int64_t c = lane * 8; c < cols; c += 512) {
        const uintx4 v = __builtin_nontemporal_load((const uintx4 *)(xr + c));
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __builtin_fminf(__builtin_fmaxf(bf16_to_f32(v[i] & 0xFFFFu) * s, -448.0f), 448.0f);
            f[2 * i + 1] = __builtin_fminf(__builtin_fmaxf(bf16_to_f32(v[i] >> 16) * s, -448.0f), 448.0f);
        }
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
        __builtin_nontemporal_store(uintx2{(uint32_t)w0, (uint32_t)w1}, (uintx2 *)(qr + c));
    }
}

// The same with the row held in registers between the two passes, for rows
// of at most R·512 values: x is read from HBM once (rows of 5760 values re-read
// half their bytes when the second pass went back to L2, with up to 32 rows in
// flight per CU and an L2 shared by 32 CUs).
template <int R>
__global__ __launch_bounds__(kThreads) void fp8_rows_reg_kernel(const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
                                                                float *amax, float *dequant, int64_t rows, int64_t cols)
{
    const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int lane = threadIdx.x & 63;
    const uint16_t *xr = x + r * cols;
    uintx4 v[R];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t c = lane * 8 + j * 512;
        v[j] = c < cols ? __builtin_nontemporal_load((const uintx4 *)(xr + c)) : uintx4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, max(v[j][i] & 0x7FFFu, (v[j][i] >> 16) & 0x7FFFu));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
    const float mf = __uint_as_float(m << 16);
    const float s = fp8_tensor_scale(mf);
    if (lane == 0) {
        amax[r] = mf;
        dequant[r] = 1.0f / s;
    }
    uint8_t *qr = q + r * cols;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t c = lane * 8 + j * 512;
        if (c >= cols) break;
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __builtin_fminf(__builtin_fmaxf(bf16_to_f32(v[j][i] & 0xFFFFu) * s, -448.0f), 448.0f);
            f[2 * i + 1] = __builtin_fminf(__builtin_fmaxf(bf16_to_f32(v[j][i] >> 16) * s, -448.0f), 448.0f);
        }
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
        __builtin_nontemporal_store(uintx2{(uint32_t)w0, (uint32_t)w1}, (uintx2 *)(qr + c));
    }
}

// ------------------------------------------------------------------ MX along tokens
// The weight gradient reduces over tokens, so its MX operands are blocked
// along them: within each expert, blocks of 32 consecutive rows (the last one
// partial), never two experts in one block.  Block j of expert g is scale
// row tile0[g] + j of the group table built with 32-row "tiles".

__device__ __forceinline__ int tokens_table(GroupTable &tab, int *sm, const int64_t *lens, const int64_t *offs,
                                            int G, int64_t M, uint32_t *err)
{
    tab.G = G;
    tab.row0 = sm;
    tab.rows = sm + G;
    tab.tile0 = sm + 2 * G;
    return build_group_table<TilesFwd, kThreads>(tab, lens, offs, G, M, TilesFwd{32, 1}, err, tab.tile0 + G + 1);
}

// grid (scale rows, column tiles): one thread per four columns of a block
// (E4M3: 8-byte loads, 4-byte code and scale stores), or per pair of
// columns, which share a code byte (E2M1)
template <int FMT>
__global__ __launch_bounds__(kThreads) void mx_tokens_quant_kernel(const uint16_t *__restrict__ x,
                                                                   const int64_t *lens, const int64_t *offs, int G,
                                                                   int64_t M, int64_t C, uint8_t *__restrict__ q,
                                                                   uint8_t *__restrict__ scales, uint32_t *err)
{
    extern __shared__ __attribute__((aligned(16))) int sm_tok[];
    GroupTable tab;
    const int total = tokens_table(tab, sm_tok, lens, offs, G, M, err);
    const int b = blockIdx.x;
    const int64_t c = (int64_t)blockIdx.y * kThreads + threadIdx.x;
    if (b >= total || c >= (FMT == 0 ? C / 4 : C / 2)) return;
    const int g = find_group(tab, b);
    const int j = b - tab.tile0[g];
    const int64_t r0 = tab.row0[g] + 32 * j;
    const int nr = min(32, tab.rows[g] - 32 * j);
    if (FMT == 0) {
        // columns 4c .. 4c + 3: word 0 holds 4c (low half) and 4c + 1
        uintx2 h[32];
        uint32_t am[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            h[i] = i < nr ? __builtin_nontemporal_load((const uintx2 *)(x + (r0 + i) * C + 4 * c)) : uintx2{0u, 0u};
#pragma unroll
            for (int k = 0; k < 4; ++k) am[k] = max(am[k], (h[i][k >> 1] >> (16 * (k & 1))) & 0x7FFFu);
        }
        int e[4];
        uint32_t Ew = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t E = mx_scale_byte<8>(am[k]);
            e[k] = 127 - (int)E;
            Ew |= E << (8 * k);
        }
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (i < nr) {
                float f[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    f[k] = __builtin_fminf(
                        __builtin_fmaxf(__builtin_ldexpf(bf16_to_f32((h[i][k >> 1] >> (16 * (k & 1))) & 0xFFFFu), e[k]),
                                        -448.0f),
                        448.0f);
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w, true);
                __builtin_nontemporal_store((uint32_t)w, (uint32_t *)(q + (r0 + i) * C + 4 * c));
            }
        *(uint32_t *)(scales + (int64_t)b * C + 4 * c) = Ew;
    } else {
        uint32_t h[32];
        // columns 2c (low half of each word, low nibble) and 2c + 1
        uint32_t a0 = 0, a1 = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            h[i] = i < nr ? __builtin_nontemporal_load((const uint32_t *)(x + (r0 + i) * C + 2 * c)) : 0u;
            a0 = max(a0, h[i] & 0x7FFFu);
            a1 = max(a1, (h[i] >> 16) & 0x7FFFu);
        }
        const uint32_t E0 = mx_scale_byte<2>(a0), E1 = mx_scale_byte<2>(a1);
        const int e0 = 127 - (int)E0, e1 = 127 - (int)E1;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (i < nr) {
                const float f0 =
                    __builtin_fminf(__builtin_fmaxf(__builtin_ldexpf(bf16_to_f32(h[i] & 0xFFFFu), e0), -6.0f), 6.0f);
                const float f1 =
                    __builtin_fminf(__builtin_fmaxf(__builtin_ldexpf(bf16_to_f32(h[i] >> 16), e1), -6.0f), 6.0f);
                const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f0, f1, 1.0f, 0);
                q[(r0 + i) * (C / 2) + c] = (uint8_t)(w & 0xFFu);
            }
        *(uint16_t *)(scales + (int64_t)b * C + 2 * c) = (uint16_t)(E0 | (E1 << 8));
    }
}

// Exact value of an E2M1 code (OCP MX: bias 1, one mantissa bit; exponent
// field 0 holds the subnormals 0 and 0.5).
__device__ __forceinline__ float e2m1_to_f32(uint32_t n)
{
    const uint32_t mag = n & 7u;
    const float v =
        mag < 2u ? 0.5f * (float)mag : __builtin_ldexpf(1.0f + 0.5f * (float)(mag & 1u), (int)(mag >> 1) - 1);
    return (n & 8u) ? -v : v;
}

// ------------------------------------------------------------------ MX weight-gradient operands
// The MX weight gradient contracts over each expert's tokens, so the 256 x
// 256 MX kernel takes the token-blocked codes transposed: channel rows
// [C, pitch bytes] in which expert g's tokens, padded with zero codes to
// whole blocks of 32, start at byte 32 * bstart_g (E4M3) or 16 * bstart_g
// (E2M1), bstart_g being the blocks of earlier experts (the scale-row
// numbering of the token quantiser).  The scales go to the kernel's
// stage-major layout with stages numbered across experts (stage kt of expert
// g is global stage S_g + kt, S_g = stages of earlier experts, a stage being
// 128 code bytes of a row): word ((S_g + kt) * C + c) * WPR + w, E4M3 blocks
// 4kt .. 4kt + 3 in byte order (WPR 1), E2M1 word w blocks 8kt + w + 0, 2,
// 4, 6 (WPR 2); blocks past an expert's last one read zero.  plan[2g] =
// bstart_g and plan[2g + 1] = S_g (written by workgroup 0) tell the GEMM
// where each expert starts.  A work item is one stage of one expert for 128
// channels: its tokens are staged in LDS (swizzled 16-byte chunks) and read
// back as blocks of 4 tokens x 4 channels turned with byte permutes (E4M3)
// or 16 tokens x 8 channels of nibbles (E2M1), the lanes of a channel group
// writing whole 128-byte runs of its rows.
constexpr int kTrCh = 128;                              // channels per work item

template <int FMT>
__global__ __launch_bounds__(kThreads) void mx_tokens_transpose_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ scales, const int64_t *lens, const int64_t *offs,
    int G, int64_t M, int C, uint8_t *__restrict__ qt, int64_t pitch, uint32_t *__restrict__ st, int *plan)
{
    constexpr int TS = FMT == 0 ? 128 : 256;            // tokens per stage
    constexpr int RB = FMT == 0 ? kTrCh : kTrCh / 2;    // input bytes of a token's 128 channels
    constexpr int LROW = 256;                           // LDS row pitch (bytes): 16 chunks of 16
    extern __shared__ __attribute__((aligned(16))) int sm_tok[];
    GroupTable tab;
    tokens_table(tab, sm_tok, lens, offs, G, M, nullptr);      // tile0: each expert's first block
    int *sst = tab.tile0 + G + 1 + 8;                           // each expert's first stage, [G + 1]
    int *scr = sst + G + 1;
    uint8_t *tile = (uint8_t *)(scr + 8);
    {
        const int per = (G + kThreads - 1) / kThreads, g0 = threadIdx.x * per;
        int sum = 0;
        for (int i = 0; i < per; ++i)
            if (g0 + i < G) sum += (tab.rows[g0 + i] + TS - 1) / TS;
        int all;
        int pre = block_exclusive_scan<kThreads>(sum, scr, &all);
        for (int i = 0; i < per; ++i)
            if (g0 + i < G) {
                sst[g0 + i] = pre;
                pre += (tab.rows[g0 + i] + TS - 1) / TS;
            }
        if (threadIdx.x == 0) sst[G] = all;
        __syncthreads();
    }
    if (blockIdx.x == 0)
        for (int g = threadIdx.x; g < G; g += kThreads) {
            plan[2 * g] = tab.tile0[g];
            plan[2 * g + 1] = sst[g];
        }
    const int nch = (C + kTrCh - 1) / kTrCh;
    const int64_t items = (int64_t)sst[G] * nch;
    const int tid = threadIdx.x;
    for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
        const int sg = (int)(w / nch), c0 = (int)(w % nch) * kTrCh;
        int lo = 0, hi = G;                              // the last expert with sst <= sg
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sst[mid] <= sg) lo = mid; else hi = mid;
        }
        const int g = lo, kt = sg - sst[g];
        const int rows = tab.rows[g], nb = (rows + 31) / 32, tok0 = kt * TS;
        const int nvalid = min(TS, rows - tok0);        // real tokens of the stage
        const int nbytes = (FMT == 0 ? 32 : 16) * min(TS / 32, nb - kt * (TS / 32));   // output bytes per row
        const int64_t r0 = (int64_t)tab.row0[g] + tok0;
        const int64_t ob = (int64_t)(FMT == 0 ? 32 : 16) * tab.tile0[g] + (int64_t)kt * 128;
        // Stage the tokens' channel bytes: 16-byte chunk k of token row t at
        // chunk position k ^ sw(t) of a 256-byte LDS row, sw(t) = 2j ^ 8 (t & 1)
        // (E4M3) or j ^ 4 (t & 3) (E2M1) with j = t / 16, so that both the
        // row-wise writes and the column reads below hit 64 distinct banks.
        // Loads of 16 bytes where a row's bytes allow it, else 8 or 4.
        const int64_t rowb = FMT == 0 ? C : C / 2;
        const int cb0 = FMT == 0 ? c0 : c0 / 2;
        auto swz = [](int t) { return FMT == 0 ? (2 * (t >> 4)) ^ (8 * (t & 1)) : (t >> 4) ^ (4 * (t & 3)); };
        constexpr int NCH = RB / 16;                         // 16-byte chunks of a token's bytes
        const int lw = rowb % 16 == 0 ? 16 : (rowb % 8 == 0 ? 8 : 4);
        for (int e = tid; e < TS * NCH; e += kThreads) {
            const int t = e / NCH, k = e % NCH;
            uint8_t *dst = tile + t * LROW + 16 * (k ^ swz(t));
            const int64_t off = (r0 + t) * rowb + cb0 + 16 * k;
            const bool in = t < nvalid;
            const int room = (int)(rowb - (cb0 + 16 * k));      // bytes of this chunk inside the row
            if (lw == 16) {
                *(uintx4 *)dst = in && room > 0 ? *(const uintx4 *)(q + off) : uintx4{0u, 0u, 0u, 0u};
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const bool ok = in && 4 * w < room;
                    ((uint32_t *)dst)[w] = ok ? *(const uint32_t *)(q + off + 4 * w) : 0u;
                }
            }
        }
        __syncthreads();
        // 32-bit word w of token row t
        auto word = [&](int t, int w) {
            return *(const uint32_t *)(tile + t * LROW + 16 * ((w >> 2) ^ swz(t)) + 4 * (w & 3));
        };
        if constexpr (FMT == 0) {
            // thread: channels 4cq .. 4cq + 3, tokens 16j .. 16j + 15, turned
            // as 4 x 4 byte blocks with v_perm; the eight lanes of a channel
            // quad write 128 contiguous bytes of each of its four rows
            const int j = tid & 7, cq = tid >> 3;
            if (16 * j < nbytes) {
                uint32_t o[4][4];                    // [channel][token quad]
#pragma unroll
                for (int tq4 = 0; tq4 < 4; ++tq4) {
                    uint32_t w[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) w[u] = word(16 * j + 4 * tq4 + u, cq);
                    const uint32_t lo01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
                    const uint32_t lo23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
                    const uint32_t hi01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
                    const uint32_t hi23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
                    o[0][tq4] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
                    o[1][tq4] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
                    o[2][tq4] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
                    o[3][tq4] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
                }
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    if (c0 + 4 * cq + d < C)
                        *(uintx4 *)(qt + (int64_t)(c0 + 4 * cq + d) * pitch + ob + 16 * j) =
                            uintx4{o[d][0], o[d][1], o[d][2], o[d][3]};
            }
        } else {
            // thread: channels 8co .. 8co + 7 (one word per token), tokens
            // 16j .. 16j + 15 -> 8 bytes per channel; the sixteen lanes of a
            // channel octet write 128 contiguous bytes of each of its rows
            const int j = tid & 15, co = tid >> 4;
            if (8 * j < nbytes) {
                uint32_t w[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) w[u] = word(16 * j + u, co);
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    uint32_t lo = 0u, hi = 0u;
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        lo |= ((w[u] >> (4 * d)) & 0xFu) << (4 * u);
                        hi |= ((w[8 + u] >> (4 * d)) & 0xFu) << (4 * u);
                    }
                    if (c0 + 8 * co + d < C)
                        *(uintx2 *)(qt + (int64_t)(c0 + 8 * co + d) * pitch + ob + 8 * j) = uintx2{lo, hi};
                }
            }
        }
        // the stage's scale words, one channel per thread (none for codes
        // without block scales: FP8 with one factor per tensor)
        const int c = tid;
        if (scales && c < kTrCh && c0 + c < C) {
            const int64_t b0 = (int64_t)tab.tile0[g] + (int64_t)kt * (TS / 32);
            uint32_t v[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < TS / 32; ++j)
                if (kt * (TS / 32) + j < nb) v[j >> 2] |= (uint32_t)scales[(b0 + j) * C + c0 + c] << (8 * (j & 3));
            const int64_t wi = ((int64_t)(sst[g] + kt) * C + c0 + c);
            if (FMT == 0) {
                st[wi] = v[0];
            } else {
                *(uintx2 *)(st + 2 * wi) =
                    uintx2{__builtin_amdgcn_perm(v[1], v[0], 0x06040200u), __builtin_amdgcn_perm(v[1], v[0], 0x07050301u)};
            }
        }
        __syncthreads();
    }
}

// Quantisation along tokens straight into the weight gradient's operand
// layout: bf16 x [M, C] -> the channel rows and stage-major scale words that
// mx_tokens_quant_kernel followed by mx_tokens_transpose_kernel produce, bit
// for bit, without the [M, C] codes in between.  A work item is one stage of
// one expert (TS tokens) for 128 channels: its bf16 tokens go to a 128-column
// LDS tile (16-byte row loads), then 4 lanes per 32-token block of a channel
// encode it as the row quantiser does along its axis (amax over the block,
// E8M0 byte, scaled and clamped values, hardware nearest-even conversion):
// 8 codes (E4M3) or 4 bytes of token pairs (E2M1, even token in the low
// nibble) per lane, 128 contiguous bytes per channel row and stage.  Tokens
// past the expert's end read as zeros, so a partial last block is encoded
// as the token quantiser encodes it and its padding tokens get zero codes;
// blocks past the expert's last one are not written (they are the next
// expert's), and their scale bytes in the expert's stage words are zero.
template <int FMT>
__global__ __launch_bounds__(kThreads) void mx_tokens_quant_t_kernel(
    const uint16_t *__restrict__ x, const int64_t *lens, const int64_t *offs, int G, int64_t M, int C,
    uint8_t *__restrict__ qt, int64_t pitch, uint32_t *__restrict__ st, int *plan, uint32_t *err,
    const uint32_t *amax, float *dequant)
{
    // FMT 2: E4M3 with one factor per tensor (the rule of fp8_encode_kernel
    // from the tensor's amax), the E4M3 layout without scale words
    constexpr int TS = FMT == 1 ? 256 : 128;            // tokens per stage
    constexpr int NBS = TS / 32;                        // blocks per stage
    constexpr int LPC = NBS * 4;                        // lanes per channel
    extern __shared__ __attribute__((aligned(16))) int sm_tok[];
    GroupTable tab;
    tokens_table(tab, sm_tok, lens, offs, G, M, err);
    int *sst = tab.tile0 + G + 1 + 8;                   // each expert's first stage, [G + 1]
    int *scr = sst + G + 1;
    // the tile at the next 16-byte boundary, as an offset from the aligned base
    // (so that the compiler can prove the alignment of its 16-byte accesses)
    uint8_t *tile = (uint8_t *)(sm_tok + ((int)(scr + 8 - sm_tok) + 3 & ~3));
    {
        const int per = (G + kThreads - 1) / kThreads, g0 = threadIdx.x * per;
        int sum = 0;
        for (int i = 0; i < per; ++i)
            if (g0 + i < G) sum += (tab.rows[g0 + i] + TS - 1) / TS;
        int all;
        int pre = block_exclusive_scan<kThreads>(sum, scr, &all);
        for (int i = 0; i < per; ++i)
            if (g0 + i < G) {
                sst[g0 + i] = pre;
                pre += (tab.rows[g0 + i] + TS - 1) / TS;
            }
        if (threadIdx.x == 0) sst[G] = all;
        __syncthreads();
    }
    if (blockIdx.x == 0)
        for (int g = threadIdx.x; g < G; g += kThreads) {
            plan[2 * g] = tab.tile0[g];
            plan[2 * g + 1] = sst[g];
        }
    float fs = 1.0f;                                    // FMT 2: the tensor's scale
    if constexpr (FMT == 2) {
        fs = fp8_tensor_scale(__uint_as_float(amax[0]));
        if (blockIdx.x == 0 && threadIdx.x == 0) dequant[0] = 1.0f / fs;
    }
    const int nch = (C + kTrCh - 1) / kTrCh;
    const int64_t items = (int64_t)sst[G] * nch;
    const int tid = threadIdx.x;
    // An item's place: expert g, its stage kt, global stage sg, channels c0..
    struct Item {
        int g, kt, sg, c0, nvalid, nbk;
        int64_t r0, ob;
    };
    auto place = [&](int64_t w) {
        Item it;
        it.sg = (int)(w / nch);
        it.c0 = (int)(w % nch) * kTrCh;
        int lo = 0, hi = G;                              // the last expert with sst <= sg
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sst[mid] <= it.sg) lo = mid; else hi = mid;
        }
        it.g = lo;
        it.kt = it.sg - sst[lo];
        const int rows = tab.rows[lo], nb = (rows + 31) / 32, tok0 = it.kt * TS;
        it.nvalid = min(TS, rows - tok0);               // real tokens of the stage
        it.nbk = min(NBS, nb - it.kt * NBS);            // the expert's blocks in the stage
        it.r0 = (int64_t)tab.row0[lo] + tok0;
        it.ob = (int64_t)(FMT == 1 ? 16 : 32) * tab.tile0[lo] + (int64_t)it.kt * 128;
        return it;
    };
    // tokens r0 .. r0 + TS - 1, channels c0 .. c0 + 127 into registers (the
    // next item's loads fly while the current one is encoded), then to LDS
    // rows (tb_chunk)
    constexpr int NL = TS * 16 / kThreads;
    uintx4 v[NL];
    auto load = [&](const Item &it) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int k = tid + j * kThreads;
            const int t = k >> 4, c8 = (k & 15) * 8;
            v[j] = uintx4{0u, 0u, 0u, 0u};
            if (t < it.nvalid && it.c0 + c8 < C)
                v[j] = __builtin_nontemporal_load((const uintx4 *)(x + (it.r0 + t) * C + it.c0 + c8));
        }
    };
    int64_t w = blockIdx.x;
    Item cur = place(w < items ? w : 0);
    if (w < items) load(cur);
    for (; w < items; w += gridDim.x) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            // one 16-byte LDS write per chunk (the tile is 16-byte aligned; as
            // four 4-byte writes, the four rows of a wave met on 16 banks)
            const int k = tid + j * kThreads;
            *(uintx4 *)tb_chunk(tile, k >> 4, k & 15) = v[j];
        }
        __syncthreads();
        const Item it = cur;
        if (w + gridDim.x < items) {
            cur = place(w + gridDim.x);
            load(cur);
        }
        // LPC lanes per channel: lane li takes tokens 8 li .. 8 li + 7 of
        // block li / 4
#pragma unroll 2
        for (int pass = 0; pass < kTrCh * LPC / kThreads; ++pass) {
            const int u = tid + pass * kThreads;
            const int col = u / LPC, li = u % LPC, blk = li >> 2, tt = li * 8;
            if (it.c0 + col >= C) continue;              // whole channels: whole quads
            uintx4 q8;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo16 = tb_elem(tile, tt + 2 * e, col);
                const uint32_t hi16 = tb_elem(tile, tt + 2 * e + 1, col);
                q8[e] = lo16 | (hi16 << 16);
            }
            uint8_t *qrow = qt + (int64_t)(it.c0 + col) * pitch + it.ob;
            if constexpr (FMT == 2) {
                if (blk < it.nbk) {
                    float f[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[2 * e] = __builtin_fminf(__builtin_fmaxf(bf16_to_f32(q8[e] & 0xFFFFu) * fs, -448.0f), 448.0f);
                        f[2 * e + 1] = __builtin_fminf(__builtin_fmaxf(bf16_to_f32(q8[e] >> 16) * fs, -448.0f), 448.0f);
                    }
                    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
                    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
                    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
                    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
                    *(uintx2 *)(qrow + li * 8) = uintx2{(uint32_t)w0, (uint32_t)w1};
                }
                continue;
            }
            uint32_t E = 0;
            if (blk < it.nbk) E = encode8<FMT, false>(q8, qrow, li);   // whole quads: blk is uniform over one
            // the block's scale byte in the expert's stage word(s): E4M3
            // byte blk of word (sg, c); E2M1 byte blk / 2 of word 2 (sg, c) + blk % 2
            if ((li & 3) == 0) {
                const int64_t wi = (int64_t)it.sg * C + it.c0 + col;
                uint8_t *sb = (uint8_t *)st + (FMT == 0 ? wi * 4 + blk : (2 * wi + (blk & 1)) * 4 + (blk >> 1));
                *sb = (uint8_t)E;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ expert weight stack
// Per-expert weights are G separate bf16 matrices W_g [R, C] (row-major),
// given as a device array of their addresses.  One read of each builds the
// stacked operand of the grouped GEMMs -- [G, R, C], or the per-expert
// transpose [G, C, R] -- or directly its MX caches, where a stack followed
// by a transposing copy would move every byte twice.  Each workgroup owns a
// 128 x 128 tile of one expert (grid: column tiles, row tiles, experts),
// eight 16-byte loads per thread (`load_rows_tb`).  A
// NULL or misaligned address reads as a zero matrix and sets an error bit.

__device__ __forceinline__ const uint16_t *expert_ptr(const void *const *ptrs, uint32_t *err)
{
    const uint16_t *p = (const uint16_t *)ptrs[blockIdx.z];
    const bool ok = p != nullptr && ((uintptr_t)p & 15) == 0;
    if (!ok && err && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(err, kErrBadPointer);
    return ok ? p : nullptr;
}

template <int TRANS>
__global__ __launch_bounds__(kThreads) void stack_experts_kernel(const void *const *ptrs, uint16_t *__restrict__ out,
                                                                 int64_t R, int64_t C, uint32_t *err)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[TRANS ? TB * TB_RS : 16];
    const int64_t g = blockIdx.z;
    const int64_t r0 = (int64_t)blockIdx.y * TB, c0 = (int64_t)blockIdx.x * TB;
    const uint16_t *xb = expert_ptr(ptrs, err);
    if (!TRANS) {
        // a plain copy of the tile's rows: four 16-byte loads in flight per
        // thread, then their stores, twice
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uintx4 w4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = threadIdx.x + (4 * h + j) * kThreads;
                const int row = k >> 4, c8 = (k & 15) * 8;
                w4[j] = uintx4{0u, 0u, 0u, 0u};
                if (xb && r0 + row < R && c0 + c8 < C)
                    w4[j] = __builtin_nontemporal_load((const uintx4 *)(xb + (r0 + row) * C + c0 + c8));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = threadIdx.x + (4 * h + j) * kThreads;
                const int row = k >> 4, c8 = (k & 15) * 8;
                if (r0 + row < R && c0 + c8 < C)
                    __builtin_nontemporal_store(w4[j], (uintx4 *)(out + (g * R + r0 + row) * C + c0 + c8));
            }
        }
        return;
    }
    uintx4 v[8];
    load_rows_tb(xb, R, C, r0, c0, v);
    rows_to_lds_tb(v, tile);
    __syncthreads();
    // the tile's 128 columns become 128 output rows of 16 chunks of 8
    // values, each chunk read down a column of the LDS tile; the 16 lanes of
    // an output row write its 256 contiguous bytes
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int k = threadIdx.x + j * kThreads;
        const int oc = k >> 4, r8 = (k & 15) * 8;
        if (c0 + oc < C && r0 + r8 < R) {
            uintx4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = tb_elem(tile, r8 + 2 * e, oc);
                const uint32_t hi = tb_elem(tile, r8 + 2 * e + 1, oc);
                o[e] = lo | (hi << 16);
            }
            __builtin_nontemporal_store(o, (uintx4 *)(out + (g * C + c0 + oc) * R + r0 + r8));
        }
    }
}

// Both MX caches of the expert weights from one read of 128 x 128 tiles:
// q/scales quantise W_g along C (each lane quad holds 32 consecutive columns
// of one row in registers, C % 32 == 0; 16 lanes write a row's 128 code
// bytes), qt/scales_t quantise W_g^T along R through the LDS tile as
// mx_quantize_t_kernel does (R % 32 == 0).  Either pair may be absent; the
// choice is uniform over the grid.
template <int FMT>
__global__ __launch_bounds__(kThreads) void mx_quantize_experts_kernel(const void *const *ptrs,
                                                                       uint8_t *__restrict__ q,
                                                                       uint8_t *__restrict__ scales,
                                                                       uint8_t *__restrict__ qt,
                                                                       uint8_t *__restrict__ scales_t, int64_t R,
                                                                       int64_t C, uint32_t *err)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[TB * TB_RS];
    const int64_t g = blockIdx.z;
    const int64_t r0 = (int64_t)blockIdx.y * TB, c0 = (int64_t)blockIdx.x * TB;
    uintx4 v[8];
    load_rows_tb(expert_ptr(ptrs, err), R, C, r0, c0, v);
    if (qt) rows_to_lds_tb(v, tile);
    if (q) {
        uint8_t *qb = q + g * R * (FMT == 0 ? C : C / 2);
        uint8_t *sb = scales + g * R * (C / 32);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = threadIdx.x + j * kThreads;
            const int row = k >> 4, c8 = (k & 15) * 8;
            // a quad's 32 columns are in or out together (C % 32 == 0)
            if (r0 + row < R && c0 + c8 < C) quantise8<FMT>(v[j], qb, sb, ((r0 + row) * C + c0 + c8) / 8);
        }
    }
    if (!qt) return;
    __syncthreads();
    quantise_t_tile<FMT>(tile, qt + g * C * (FMT == 0 ? R : R / 2), scales_t + g * C * (R / 32), R, C, r0, c0);
}

}  // namespace

hipError_t launch_quantize(const uint16_t *x, uint8_t *q, uint8_t *scales, int64_t rows, int64_t cols,
                           int fmt, hipStream_t s, int64_t q_pitch)
{
    const int64_t nquads = rows * cols / 8;
    const int64_t extra = q_pitch ? q_pitch - (fmt == 0 ? cols : cols / 2) : 0;
    if (nquads == 0) return hipSuccess;
    // whole blocks per workgroup (256 lanes = 64 blocks), a few waves per SIMD
    int64_t grid = (nquads + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cus() * 16;
    if (grid > cap) grid = cap;
    if (fmt == 0)
        hipLaunchKernelGGL(mx_quantize_kernel<0>, dim3((unsigned)grid), dim3(kThreads), 0, s, x, q, scales, nquads,
                           cols / 8, extra);
    else
        hipLaunchKernelGGL(mx_quantize_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0, s, x, q, scales, nquads,
                           cols / 8, extra);
    return hipGetLastError();
}

hipError_t launch_quantize_cols(const uint16_t *x, uint8_t *q, uint8_t *scales, int64_t rows, int64_t cols,
                                int fmt, hipStream_t s)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t nb = rows / 32;
    const dim3 grid((unsigned)((cols / 4 + kThreads - 1) / kThreads), (unsigned)(nb < 65535 ? nb : 65535));
    if (fmt == 0)
        hipLaunchKernelGGL(mx_quantize_cols_kernel<0>, grid, dim3(kThreads), 0, s, x, q, scales, rows, cols);
    else
        hipLaunchKernelGGL(mx_quantize_cols_kernel<1>, grid, dim3(kThreads), 0, s, x, q, scales, rows, cols);
    return hipGetLastError();
}

hipError_t launch_quantize_t(const uint16_t *x, uint8_t *q, uint8_t *scales, int64_t batch, int64_t rows,
                             int64_t cols, int fmt, hipStream_t s)
{
    if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
    const dim3 grid((unsigned)((cols + TB - 1) / TB), (unsigned)((rows + TB - 1) / TB), (unsigned)batch);
    if (fmt == 0)
        hipLaunchKernelGGL(mx_quantize_t_kernel<0>, grid, dim3(kThreads), 0, s, x, q, scales, rows, cols);
    else
        hipLaunchKernelGGL(mx_quantize_t_kernel<1>, grid, dim3(kThreads), 0, s, x, q, scales, rows, cols);
    return hipGetLastError();
}

hipError_t launch_fp8_quantize(const uint16_t *x, uint8_t *q, float *amax, float *dequant, int64_t batch,
                               int64_t n, hipStream_t s)
{
    if (batch == 0) return hipSuccess;
    uint32_t *am = (uint32_t *)amax;
    hipLaunchKernelGGL(fp8_amax_zero_kernel, dim3((unsigned)((batch + 63) / 64)), dim3(64), 0, s, am, batch);
    const int64_t n8 = n / 8;
    int64_t chunks = (n8 + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cus() * 8;
    if (chunks > cap) chunks = cap;
    if (chunks < 1) chunks = 1;
    const dim3 grid((unsigned)chunks, (unsigned)batch);
    hipLaunchKernelGGL(fp8_amax_kernel, grid, dim3(kThreads), 0, s, x, am, n8);
    hipLaunchKernelGGL(fp8_encode_kernel, grid, dim3(kThreads), 0, s, x, q, am, dequant, n8);
    return hipGetLastError();
}

hipError_t launch_fp8_amax(const uint16_t *x, uint32_t *amax, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(fp8_amax_zero_kernel, dim3(1), dim3(64), 0, s, amax, (int64_t)1);
    const int64_t n8 = n / 8;
    int64_t chunks = (n8 + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cus() * 8;
    if (chunks > cap) chunks = cap;
    if (chunks < 1) chunks = 1;
    hipLaunchKernelGGL(fp8_amax_kernel, dim3((unsigned)chunks, 1u), dim3(kThreads), 0, s, x, amax, n8);
    return hipGetLastError();
}

hipError_t launch_fp8_quantize_rows(const uint16_t *x, uint8_t *q, float *amax, float *dequant, int64_t rows,
                                    int64_t cols, hipStream_t s)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t grid = (rows + kThreads / 64 - 1) / (kThreads / 64);
    const dim3 g((unsigned)grid), b(kThreads);
    if (cols <= 4 * 512)
        hipLaunchKernelGGL(fp8_rows_reg_kernel<4>, g, b, 0, s, x, q, amax, dequant, rows, cols);
    else if (cols <= 8 * 512)
        hipLaunchKernelGGL(fp8_rows_reg_kernel<8>, g, b, 0, s, x, q, amax, dequant, rows, cols);
    else if (cols <= 12 * 512)
        hipLaunchKernelGGL(fp8_rows_reg_kernel<12>, g, b, 0, s, x, q, amax, dequant, rows, cols);
    else if (cols <= 16 * 512)
        hipLaunchKernelGGL(fp8_rows_reg_kernel<16>, g, b, 0, s, x, q, amax, dequant, rows, cols);
    else
        hipLaunchKernelGGL(fp8_rows_kernel, g, b, 0, s, x, q, amax, dequant, rows, cols);
    return hipGetLastError();
}

hipError_t launch_mx_quantize_tokens(const uint16_t *x, const int64_t *lens, const int64_t *offs, int G, int64_t M,
                                     int64_t C, int fmt, uint8_t *q, uint8_t *scales, uint32_t *err, hipStream_t s)
{
    const int64_t nb = M / 32 + G;                 // scale rows an upper bound allows
    const int64_t nc = fmt == 0 ? C / 4 : C / 2;   // threads per scale row
    if (nb == 0 || nc == 0) return hipSuccess;
    const dim3 grid((unsigned)nb, (unsigned)((nc + kThreads - 1) / kThreads));
    if (fmt == 0)
        hipLaunchKernelGGL(mx_tokens_quant_kernel<0>, grid, dim3(kThreads), table_bytes(G), s, x, lens, offs, G, M, C,
                           q, scales, err);
    else
        hipLaunchKernelGGL(mx_tokens_quant_kernel<1>, grid, dim3(kThreads), table_bytes(G), s, x, lens, offs, G, M, C,
                           q, scales, err);
    return hipGetLastError();
}

int64_t mx_wgrad_pitch(int64_t M, int G, int fmt)
{
    const int64_t tokens = 32 * (M / 32 + G);             // every expert padded to whole blocks
    const int64_t bytes = fmt == 0 ? tokens : tokens / 2;
    return (bytes + 127) / 128 * 128;
}

int64_t mx_wgrad_stages(int64_t M, int G, int fmt)
{
    return mx_wgrad_pitch(M, G, fmt) / 128 + G;           // a partial last stage per expert at most
}

hipError_t launch_mx_tokens_transpose(const uint8_t *q, const uint8_t *scales, const int64_t *lens,
                                      const int64_t *offs, int G, int64_t M, int64_t C, int fmt, uint8_t *qt,
                                      int64_t pitch, uint32_t *st, int *plan, hipStream_t s)
{
    if (G == 0 || C == 0) return hipSuccess;
    const int ts = fmt == 0 ? 128 : 256;
    const size_t lds = table_bytes(G) + 4 * (G + 1) + 32 + (size_t)ts * 256;
    const int64_t items = mx_wgrad_stages(M, G, fmt) * ((C + kTrCh - 1) / kTrCh);
    int64_t grid = (int64_t)device_cus() * 4;
    if (grid > items) grid = items;
    if (grid < 1) grid = 1;
    if (fmt == 0)
        hipLaunchKernelGGL(mx_tokens_transpose_kernel<0>, dim3((unsigned)grid), dim3(kThreads), lds, s, q, scales,
                           lens, offs, G, M, (int)C, qt, pitch, st, plan);
    else
        hipLaunchKernelGGL(mx_tokens_transpose_kernel<1>, dim3((unsigned)grid), dim3(kThreads), lds, s, q, scales,
                           lens, offs, G, M, (int)C, qt, pitch, st, plan);
    return hipGetLastError();
}

hipError_t launch_mx_tokens_quant_t(const uint16_t *x, const int64_t *lens, const int64_t *offs, int G, int64_t M,
                                    int64_t C, int fmt, uint8_t *qt, int64_t pitch, uint32_t *st, int *plan,
                                    uint32_t *err, const uint32_t *amax, float *dequant, hipStream_t s)
{
    if (G == 0 || C == 0) return hipSuccess;
    const int ts = fmt == 1 ? 256 : 128;
    const size_t lds = table_bytes(G) + 4 * (G + 1) + 32 + 16 + (size_t)ts * TB_RS;
    const int64_t items = mx_wgrad_stages(M, G, fmt == 1 ? 1 : 0) * ((C + kTrCh - 1) / kTrCh);
    // as many workgroups per CU as fit beside each other in LDS (160 KiB), at
    // most four (four waves per SIMD)
    const int64_t per_cu = std::min<int64_t>(4, (int64_t)(160 * 1024) / (int64_t)lds);
    int64_t grid = (int64_t)device_cus() * std::max<int64_t>(1, per_cu);
    if (grid > items) grid = items;
    if (grid < 1) grid = 1;
    if (fmt == 0)
        hipLaunchKernelGGL(mx_tokens_quant_t_kernel<0>, dim3((unsigned)grid), dim3(kThreads), lds, s, x, lens, offs,
                           G, M, (int)C, qt, pitch, st, plan, err, amax, dequant);
    else if (fmt == 1)
        hipLaunchKernelGGL(mx_tokens_quant_t_kernel<1>, dim3((unsigned)grid), dim3(kThreads), lds, s, x, lens, offs,
                           G, M, (int)C, qt, pitch, st, plan, err, amax, dequant);
    else
        hipLaunchKernelGGL(mx_tokens_quant_t_kernel<2>, dim3((unsigned)grid), dim3(kThreads), lds, s, x, lens, offs,
                           G, M, (int)C, qt, pitch, st, plan, err, amax, dequant);
    return hipGetLastError();
}

hipError_t launch_stack_experts(const void *const *ptrs, uint16_t *out, int G, int64_t R, int64_t C, int trans,
                                uint32_t *err, hipStream_t s)
{
    if (G == 0 || R == 0 || C == 0) return hipSuccess;
    const dim3 grid((unsigned)((C + TB - 1) / TB), (unsigned)((R + TB - 1) / TB), (unsigned)G);
    if (trans)
        hipLaunchKernelGGL(stack_experts_kernel<1>, grid, dim3(kThreads), 0, s, ptrs, out, R, C, err);
    else
        hipLaunchKernelGGL(stack_experts_kernel<0>, grid, dim3(kThreads), 0, s, ptrs, out, R, C, err);
    return hipGetLastError();
}

hipError_t launch_mx_quantize_experts(const void *const *ptrs, uint8_t *q, uint8_t *scales, uint8_t *qt,
                                      uint8_t *scales_t, int G, int64_t R, int64_t C, int fmt, uint32_t *err,
                                      hipStream_t s)
{
    if (G == 0 || R == 0 || C == 0) return hipSuccess;
    const dim3 grid((unsigned)((C + TB - 1) / TB), (unsigned)((R + TB - 1) / TB), (unsigned)G);
    if (fmt == 0)
        hipLaunchKernelGGL(mx_quantize_experts_kernel<0>, grid, dim3(kThreads), 0, s, ptrs, q, scales, qt, scales_t,
                           R, C, err);
    else
        hipLaunchKernelGGL(mx_quantize_experts_kernel<1>, grid, dim3(kThreads), 0, s, ptrs, q, scales, qt, scales_t,
                           R, C, err);
    return hipGetLastError();
}


}  // namespace ptgg
