// epilogue.hpp -- stores of a 128 x 128 accumulator tile held as 2 x 2 blocks
// of 32 x 32 per wave (v_mfma_f32_32x32x* result layout: lane l, register r
// holds row (r/4)*8 + (l/32)*4 + r%4 and column l%32 of its block).
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace ptgg {

constexpr int kTileM = 128, kTileN = 128;

__device__ __forceinline__ int acc_row(int wm, int bi, int reg)
{
    const int lane = threadIdx.x & 63;
    return wm * 64 + bi * 32 + (reg >> 2) * 8 + (lane >> 5) * 4 + (reg & 3);
}
__device__ __forceinline__ int acc_col(int wn, int bj)
{
    return wn * 64 + bj * 32 + (threadIdx.x & 31);
}

// Tile column c -> logical output column.  With SwiGLU a tile covers 64
// consecutive outputs j: within each wave's 64 columns the first 32 are the
// gate columns j and the next 32 the matching up columns I + j, so one lane
// holds both factors of its output.
template <int EPI>
__device__ __forceinline__ int map_col(int nt, int c, int Nout)
{
    if (EPI == kEpiNone) return nt * kTileN + c;
    const int I = Nout >> 1;
    const int j = nt * (kTileN / 2) + (c >> 6) * 32 + (c & 31);
    return ((c >> 5) & 1) ? I + j : j;
}

// Clamp a column (or the start of a `width`-column chunk) into its half.
template <int EPI>
__device__ __forceinline__ int clamp_col(int n, int Nout, int width)
{
    if (EPI == kEpiNone) return min(n, Nout - width);
    const int I = Nout >> 1;
    return n < I ? min(n, I - width) : min(n, Nout - width);
}

// Stores rows [m0, m0+128) of one expert (global row row0 + m), masked to
// m < rows.  Output layouts:
//   kEpiNone:        bf16 out[M, ldo], columns nt*128 + c < Nout
//   kEpiSwiglu:      bf16 out[M, ldo], j < Nout/2
//   kEpiSwigluMxfp4: codes out[M, ldo bytes] (two per byte), scales
//                    out_scale[M, Nout/64]; requires (Nout/2) % 32 == 0
template <int EPI>
__device__ __forceinline__ void store_tile(const floatx16 (&acc)[2][2], void *out, uint8_t *out_scale,
                                           int64_t row0, int m0, int rows, int nt, int Nout, int ldo)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    if (EPI == kEpiNone) {
        uint16_t *o = (uint16_t *)out + row0 * ldo;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const int n = nt * kTileN + acc_col(wn, bj);
                if (n >= Nout) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + acc_row(wm, bi, r);
                    if (m < rows) o[(int64_t)m * ldo + n] = (uint16_t)bf16_rne(acc[bi][bj][r]);
                }
            }
    } else if (EPI == kEpiSwiglu) {
        uint16_t *o = (uint16_t *)out + row0 * ldo;
        const int I = Nout >> 1;
        const int j = nt * (kTileN / 2) + wn * 32 + (lane & 31);
        if (j < I) {
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + acc_row(wm, bi, r);
                    if (m < rows)
                        o[(int64_t)m * ldo + j] = (uint16_t)bf16_rne(silu_mul(acc[bi][0][r], acc[bi][1][r]));
                }
        }
    } else {
        // SwiGLU value rounded to bf16, then one MXFP4 block per 32 columns:
        // the 32 lanes of a half-wave hold the 32 consecutive j of one row.
        uint8_t *o = (uint8_t *)out + row0 * ldo;
        uint8_t *os = out_scale + row0 * (Nout / 64);
        const int I = Nout >> 1;
        const int j = nt * (kTileN / 2) + wn * 32 + (lane & 31);
        const bool jvalid = j < I;                 // uniform over the half-wave
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + acc_row(wm, bi, r);
                const uint32_t hb = bf16_rne(silu_mul(acc[bi][0][r], acc[bi][1][r]));
                uint32_t amax = hb & 0x7FFFu;
#pragma unroll
                for (int d = 1; d < 32; d <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, d, 64));
                const uint32_t E = mx_scale_byte<2>(amax);
                const uint32_t code = mx_encode<1>(hb, E);
                const uint32_t nb = (uint32_t)__shfl_xor((int)code, 1, 64);
                if (jvalid && m < rows) {
                    if ((lane & 1) == 0) o[(int64_t)m * ldo + (j >> 1)] = (uint8_t)(code | (nb << 4));
                    if ((lane & 31) == 0) os[(int64_t)m * (Nout / 64) + (j >> 5)] = (uint8_t)E;
                }
            }
    }
}

}  // namespace ptgg
