// pipeline.hpp -- pieces shared by the gfx950 grouped-GEMM mainloops (BF16
// and OCP-MX): the LDS ring filled by direct buffer->LDS loads, its waits and
// barrier, the swizzled geometry of a reduction-contiguous operand in LDS,
// the SwiGLU column map of a tile and the output epilogues.
//
// Tiles are 128 x 256 outputs computed by four waves in a 2 x 2 layout, each
// wave owning 64 x 128 outputs as 2 x 4 blocks of 32 x 32 (the result layout
// of the 32x32 MFMAs: lane l, register r holds row (r/4)*8 + (l/32)*4 + r%4
// and column l%32 of its block).  Every stage of the ring carries 64 bytes of
// each operand row along the reduction (32 BF16, 64 E4M3 or 128 E2M1 values).
#pragma once
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace ptgg {
namespace {

constexpr int BM = 128, BN = 256;
constexpr int ROW_BYTES = 64;                      // per operand row per stage
constexpr int A_BYTES = BM * ROW_BYTES;            // 8 KiB per stage
constexpr int B_BYTES = BN * ROW_BYTES;            // 16 KiB per stage
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int A_LOADS = A_BYTES / 16 / kThreads;   // 16-byte loads per thread per stage
constexpr int B_LOADS = B_BYTES / 16 / kThreads;
constexpr int LOADS = A_LOADS + B_LOADS;
constexpr uint32_t kRsrcWord3 = 0x00020000u;       // raw buffer, 32-bit data format
constexpr uint32_t kOOB = 0x80000000u;             // offset past every record bound

typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without the memory fence of __syncthreads() (which would
// wait for every outstanding load, draining the ring); the empty asm keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// 16-byte LDS read at addr + OFF, issued as inline asm: the compiler cannot
// tell it apart from reads of LDS still being filled by the in-flight direct
// loads and would otherwise wait for every outstanding load before it.
template <int OFF>
__device__ __forceinline__ uintx4 ldsr_u128(uint32_t addr)
{
    uintx4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, (int)kRsrcWord3);
}

// One 16-byte direct load per lane into LDS (lane i lands at lds + 16 i) from
// byte voff + soff of a buffer of `bytes` bytes at `base`; offsets at or past
// the bound read zeros.  Kept a plain function: the buffer-resource type is
// device-only, and inside templates clang's host pass would silently discard
// every kernel that reaches it.
__device__ __forceinline__ void dma16(const void *base, uint32_t bytes, uint8_t *lds, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base, bytes), (lds_void *)lds, 16, voff, soff, 0, 0);
}

// The same with the non-temporal cache policy (NT, bit 1 of the cache-policy
// field): for data no other workgroup reads, whose lines should be the first
// to leave L2 so that data shared between workgroups stays.
__device__ __forceinline__ void dma16_nt(const void *base, uint32_t bytes, uint8_t *lds, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base, bytes), (lds_void *)lds, 16, voff, soff, 0, 2);
}

// One operand's direct-load state for a tile: NL 16-byte loads per thread
// per stage at voff[i] + kt * kstep (bytes) inside the buffer at `base`.
template <int NL>
struct Dma {
    const void *base;
    uint32_t bytes;
    uint32_t voff[NL];
    uint32_t kstep;
};

// Issue one stage of an operand: slot i of this thread lands at LDS byte
// lds_off + (i * 256 + thread) * 16.
template <int NL>
__device__ __forceinline__ void issue(uint8_t *smem, const Dma<NL> &d, uint32_t lds_off, uint32_t soff,
                                      const uint32_t (&voff)[NL], int wave)
{
#pragma unroll
    for (int i = 0; i < NL; ++i)
        dma16(d.base, d.bytes, smem + lds_off + (i * kThreads + wave * kWave) * 16, voff[i], soff);
}

// Reduction-contiguous operand with R rows in one stage: LDS [R][64 bytes],
// chunk c (16 bytes) of row r at position c ^ ((r >> 2) & 3), so the 16-byte
// fragment reads of 32 consecutive rows spread over all banks.
__device__ __forceinline__ int kpos(int r, int c) { return c ^ ((r >> 2) & 3); }
// slot s of such a stage: tile row and source chunk
__device__ __forceinline__ void kslot(int s, int &r, int &c) { r = s >> 2; c = kpos(r, s & 3); }

// Tile column c (0..255) -> logical output column.  With SwiGLU a tile covers
// 128 consecutive outputs j: within each wave's 128 columns, blocks 0-1 are
// gate columns j and blocks 2-3 the matching up columns I + j, so one lane
// holds both factors of its outputs.
template <int EPI>
__device__ __forceinline__ int col_of(int nt, int c, int Nout)
{
    if (!epi_glu(EPI)) return nt * BN + c;
    const int I = Nout >> 1;
    const int w = c >> 7, cc = c & 127;
    const int j = nt * (BN / 2) + w * 64 + (cc & 63);
    return cc >= 64 ? I + j : j;
}

// Clamp an 8-column chunk start into the valid range of its half.
template <int EPI>
__device__ __forceinline__ int clamp8(int n, int Nout)
{
    if (!epi_glu(EPI)) return min(n, Nout - 8);
    const int I = Nout >> 1;
    return n < I ? min(n, I - 8) : min(n, Nout - 8);
}

// Clamp a single column into the valid range of its half.
template <int EPI>
__device__ __forceinline__ int clamp1(int n, int Nout)
{
    if (!epi_glu(EPI)) return min(n, Nout - 1);
    const int I = Nout >> 1;
    return n < I ? min(n, I - 1) : min(n, Nout - 1);
}

// Wave (wm, wn) holds rows wm*64 + bi*32 + .., columns wn*128 + bj*32 + lane%32.
__device__ __forceinline__ int e_row(int wm, int bi, int reg)
{
    return wm * 64 + bi * 32 + (reg >> 2) * 8 + ((threadIdx.x & 63) >> 5) * 4 + (reg & 3);
}

// Stores rows [m0, m0 + 128) of one expert (global row row0 + m), masked to
// m < rows.  Output layouts:
//   kEpiNone:        bf16 out[M, ldo], columns nt*256 + c < Nout
//   kEpiSwiglu:      bf16 out[M, ldo], outputs j < Nout/2
//   kEpiSwigluMxfp4: codes out[M, ldo bytes] (two per byte, low nibble the
//                    even output), scales out_scale[M, Nout/64]; requires
//                    (Nout/2) % 32 == 0
// lim: the SwiGLU clamp (+inf for none).
template <int EPI>
__device__ __forceinline__ void store_out(const floatx16 (&acc)[2][4], void *out, uint8_t *out_scale, int ldo,
                                          int Nout, int64_t row0, int m0, int rows, int nt, int wm, int wn, float lim)
{
    const int lane = threadIdx.x & 63;
    if (EPI == kEpiNone) {
        uint16_t *o = (uint16_t *)out + row0 * ldo;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int n = nt * BN + wn * 128 + bj * 32 + (lane & 31);
                if (n >= Nout) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + e_row(wm, bi, r);
                    if (m < rows) o[(int64_t)m * ldo + n] = (uint16_t)bf16_rne(acc[bi][bj][r]);
                }
            }
    } else if (EPI == kEpiSwiglu) {
        uint16_t *o = (uint16_t *)out + row0 * ldo;
        const int I = Nout >> 1;
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const int j = nt * (BN / 2) + wn * 64 + bj * 32 + (lane & 31);
            if (j >= I) continue;
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + e_row(wm, bi, r);
                    if (m < rows)
                        o[(int64_t)m * ldo + j] =
                            (uint16_t)bf16_rne(silu_mul(acc[bi][bj][r], acc[bi][bj + 2][r], lim));
                }
        }
    } else {
        // SwiGLU value rounded to bf16, then one MXFP4 block per 32 outputs:
        // the 32 lanes of a half-wave hold 32 consecutive j of one row.
        uint8_t *o = (uint8_t *)out + row0 * ldo;
        uint8_t *os = out_scale + row0 * (Nout / 64);
        const int I = Nout >> 1;
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const int j = nt * (BN / 2) + wn * 64 + bj * 32 + (lane & 31);
            const bool jvalid = j < I;          // uniform over a half-wave (I % 32 == 0)
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + e_row(wm, bi, r);
                    const uint32_t hb = bf16_rne(silu_mul(acc[bi][bj][r], acc[bi][bj + 2][r], lim));
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
}

// Epilogue through LDS, for a tile of TROWS (at most 64 * NWM) rows computed by NWM x 2
// waves (the ring is idle by then).  Phase 1: every wave writes its results
// as bf16 (after SwiGLU when asked) into a row-major LDS tile whose rows are
// padded by 16 bytes, so the two lane halves (rows 4 apart) of a 2-byte
// write land on different banks.  Phase 2: whole rows leave as 16-byte
// stores, or, for MXFP4, each thread encodes one 32-value block held in its
// own registers (amax, shared E8M0 byte, codes) and stores its 16 code bytes
// and its scale byte.  A wave holds MI x NJ blocks of 32 x 32 starting at
// tile row wrow0: tile columns kEpiNone 256 (nt * 256 + c, c = wn * NJ * 32 +
// bj * 32 + lane % 32), SwiGLU 128 outputs (nt * 128 + c, c = wn * NJ * 16 +
// q * 32 + lane % 32 from gate block q and up block q + NJ / 2).
template <int EPI>
__host__ __device__ constexpr int epi_row_bytes() { return (epi_glu(EPI) ? BN / 2 : BN) * 2 + 16; }
template <int EPI, int NWM>
__host__ __device__ constexpr int epi_lds_bytes() { return 64 * NWM * epi_row_bytes<EPI>(); }

template <int EPI, int NWM, int MI, int NJ, int TROWS = 64 * NWM>
__device__ __forceinline__ void store_tile_lds_w(const floatx16 (&acc)[MI][NJ], uint8_t *smem, void *out,
                                                 uint8_t *out_scale, int ldo, int Nout, int64_t row0, int m0,
                                                 int rows, int nt, int wrow0, int wn, float lim,
                                                 const uint16_t *aux = nullptr, int ldaux = 0,
                                                 uint16_t *save = nullptr, int ldsave = 0)
{
    constexpr int TR = TROWS;                              // tile rows (at most 64 * NWM)
    static_assert(TROWS <= 64 * NWM, "tile rows");
    constexpr int OC = epi_glu(EPI) ? BN / 2 : BN;         // output columns of the tile
    constexpr int RS = epi_row_bytes<EPI>();
    constexpr int NT = NWM * 2 * kWave;
    const int lane = threadIdx.x & 63;
    auto row_of = [&](int bi, int r) { return wrow0 + bi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); };
    if (!epi_glu(EPI)) {
#pragma unroll
        for (int bi = 0; bi < MI; ++bi)
#pragma unroll
            for (int bj = 0; bj < NJ; ++bj) {
                const int c = wn * NJ * 32 + bj * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    *(uint16_t *)(smem + row_of(bi, r) * RS + c * 2) = (uint16_t)bf16_rne(acc[bi][bj][r]);
            }
    } else {
        // blocks q < NJ / 2 hold gate columns, block q + NJ / 2 the matching up columns
#pragma unroll
        for (int bi = 0; bi < MI; ++bi)
#pragma unroll
            for (int q = 0; q < NJ / 2; ++q) {
                const int c = wn * NJ * 16 + q * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    *(uint16_t *)(smem + row_of(bi, r) * RS + c * 2) =
                        (uint16_t)bf16_rne(silu_mul(acc[bi][q][r], acc[bi][q + NJ / 2][r], lim));
            }
    }
    __syncthreads();
    const int ncols = epi_glu(EPI) ? Nout / 2 : Nout;      // valid output columns (multiple of 8)
    if (EPI == kEpiDSwiglu) {
        // SwiGLU backward: this tile holds bf16 dH for columns k of an
        // expert's rows; with g = aux[r, k] and u = aux[r, Nout + k] (the
        // forward's [gate | up] output), write
        //   out[r, k] = dH * u * s * (1 + g * (1 - s)),  out[r, Nout + k] = dH * g * s,
        // s = sigmoid(g), in fp32, each rounded once to bf16.  Clamped
        // (finite lim): g and u clamped as in the forward, and no gradient
        // into a clamped input (g > lim, |u| > lim).
        constexpr int CPR = OC / 8;
        uint16_t *o = (uint16_t *)out + row0 * ldo;
        const uint16_t *x = aux + row0 * ldaux;
        for (int i = threadIdx.x; i < TR * CPR; i += NT) {
            const int r = i / CPR, c = i % CPR;
            const int col = nt * OC + c * 8;
            if (m0 + r < rows && col < ncols) {
                const int64_t row = m0 + r;
                const uintx4 dh = *(const uintx4 *)(smem + r * RS + c * 16);
                const uintx4 gv = __builtin_nontemporal_load((const uintx4 *)(x + row * ldaux + col));
                const uintx4 uv = __builtin_nontemporal_load((const uintx4 *)(x + row * ldaux + Nout + col));
                uintx4 dg, du;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t pg = 0, pu = 0;
#pragma unroll
                    for (int hlf = 0; hlf < 2; ++hlf) {
                        const float d = __uint_as_float((dh[e] >> (16 * hlf)) << 16);
                        const float g0 = __uint_as_float((gv[e] >> (16 * hlf)) << 16);
                        const float u0 = __uint_as_float((uv[e] >> (16 * hlf)) << 16);
                        const float g = __builtin_fminf(g0, lim);
                        const float u = __builtin_fminf(__builtin_fmaxf(u0, -lim), lim);
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                        const float vg = g0 <= lim ? d * u * (sg * (1.0f + g * (1.0f - sg))) : 0.0f;
                        const float vu = __builtin_fabsf(u0) <= lim ? d * (g * sg) : 0.0f;
                        pg |= bf16_rne(vg) << (16 * hlf);
                        pu |= bf16_rne(vu) << (16 * hlf);
                    }
                    dg[e] = pg;
                    du[e] = pu;
                }
                __builtin_nontemporal_store(dg, (uintx4 *)(o + row * ldo + col));
                __builtin_nontemporal_store(du, (uintx4 *)(o + row * ldo + Nout + col));
            }
        }
    } else if (EPI != kEpiSwigluMxfp4) {
        constexpr int CPR = OC / 8;                        // 16-byte chunks per row
        uint16_t *o = (uint16_t *)out + row0 * ldo;
        for (int i = threadIdx.x; i < TR * CPR; i += NT) {
            const int r = i / CPR, c = i % CPR;
            const int col = nt * OC + c * 8;
            if (m0 + r < rows && col < ncols)
                __builtin_nontemporal_store(*(const uintx4 *)(smem + r * RS + c * 16), (uintx4 *)(o + (int64_t)(m0 + r) * ldo + col));
        }
    } else {
        constexpr int BPR = OC / 32;                       // MXFP4 blocks per row
        uint8_t *o = (uint8_t *)out + row0 * ldo;
        uint8_t *os = out_scale + row0 * (Nout / 64);
        for (int i = threadIdx.x; i < TR * BPR; i += NT) {
            const int r = i / BPR, b = i % BPR;
            const int j0 = nt * OC + b * 32;
            if (m0 + r >= rows || j0 >= ncols) continue;
            uintx4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = *(const uintx4 *)(smem + r * RS + b * 64 + q * 16);
            uint32_t amax = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) amax = max(amax, max(v[q][e] & 0x7FFFu, (v[q][e] >> 16) & 0x7FFFu));
            const uint32_t E = mx_scale_byte<2>(amax);
            // each value times 2^(127 - E) (exact: a power of two), clamped to
            // the grid maximum 6, then the hardware's nearest-even E2M1
            // conversion, as the row quantiser encodes (the 128 x 256 kernels'
            // integer encoder gives the same codes; the tests compare both)
            const int sc = 127 - (int)E;
            uint32_t packed[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float f[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[2 * e] = __builtin_ldexpf(bf16_to_f32(v[q][e] & 0xFFFFu), sc);
                    f[2 * e + 1] = __builtin_ldexpf(bf16_to_f32(v[q][e] >> 16), sc);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = __builtin_fminf(__builtin_fmaxf(f[e], -6.0f), 6.0f);
                uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f[0], f[1], 1.0f, 0);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], 1.0f, 1);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], 1.0f, 2);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], 1.0f, 3);
                packed[q] = w;
            }
            __builtin_nontemporal_store(uintx4{packed[0], packed[1], packed[2], packed[3]}, (uintx4 *)(o + (int64_t)(m0 + r) * ldo + (j0 >> 1)));
            os[(int64_t)(m0 + r) * (Nout / 64) + (j0 >> 5)] = (uint8_t)E;
        }
    }
    if (EPI == kEpiSwigluSave) {
        // the GEMM output itself, for the backward: the gate half, then the
        // up half, each through the same LDS tile as bf16 (column j of the
        // tile is gate column nt * OC + j, up column Nout / 2 + nt * OC + j)
        constexpr int CPR = OC / 8;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            wait_lgkm0();
            barrier();
#pragma unroll
            for (int bi = 0; bi < MI; ++bi)
#pragma unroll
                for (int q = 0; q < NJ / 2; ++q) {
                    const int c = wn * NJ * 16 + q * 32 + (lane & 31);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        *(uint16_t *)(smem + row_of(bi, r) * RS + c * 2) =
                            (uint16_t)bf16_rne(acc[bi][q + half * (NJ / 2)][r]);
                }
            __syncthreads();
            uint16_t *o = save + row0 * ldsave + half * (Nout / 2);
            for (int i = threadIdx.x; i < TR * CPR; i += NT) {
                const int r = i / CPR, c = i % CPR;
                const int col = nt * OC + c * 8;
                if (m0 + r < rows && col < ncols)
                    __builtin_nontemporal_store(*(const uintx4 *)(smem + r * RS + c * 16), (uintx4 *)(o + (int64_t)(m0 + r) * ldsave + col));
            }
        }
    }
    // The next tile's loads may overwrite the LDS tile once every wave has
    // read it; the stores stay in flight (__syncthreads() would wait for
    // their acknowledgement, since vmcnt counts stores too).
    wait_lgkm0();
    barrier();
}

// The same for a wave grid of NWM x 2 waves, wave (wm, wn) holding rows
// wm * 64 + bi * 32 + .. and columns wn * 128 + bj * 32 + lane % 32.
template <int EPI, int NWM>
__device__ __forceinline__ void store_tile_lds(const floatx16 (&acc)[2][4], uint8_t *smem, void *out,
                                               uint8_t *out_scale, int ldo, int Nout, int64_t row0, int m0, int rows,
                                               int nt, int wm, int wn, float lim, uint16_t *save = nullptr,
                                               int ldsave = 0, const uint16_t *aux = nullptr, int ldaux = 0)
{
    store_tile_lds_w<EPI, NWM, 2, 4>(acc, smem, out, out_scale, ldo, Nout, row0, m0, rows, nt, wm * 64, wn, lim,
                                     aux, ldaux, save, ldsave);
}

// ------------------------------------------------------------------ tile queues
// Dynamic tile order for the persistent 256 x 256 kernels.  The linear tile
// ids are cut into chunks of kQueueChunk consecutive ids (or more, as the
// kernel asks), and chunk c belongs to queue c % Q (Q = 8 when the grid is a
// multiple of 8, else 1).
// Workgroup b takes ids from queue b % Q first: workgroups are dispatched
// round-robin over the 8 XCDs, so that is its own XCD's queue, and the tiles
// in flight on an XCD form a sliding window of consecutive ids.  The column
// tiles of one expert then start a few stages apart and find its activation
// rows (and the m-tiles of a large expert its weight panel) still in the
// XCD's L2.  A static round-robin order lets each workgroup's start times
// drift by whole tiles, which spreads an expert's column tiles too far apart
// for that.
// Once its queue is empty a workgroup drains the others, so all workgroups
// finish within about one tile of each other.  Every id is handed out exactly
// once, whichever workgroup takes it, so results do not depend on the order.
// The counters (one 128-byte line each) live in the caller's workspace and
// are zeroed on the stream before every launch.  Takes are system-scope
// atomics: they are performed past the per-XCD L2s, so increments from every
// XCD meet in one place.
constexpr int kQueueChunk = 32;

__device__ __forceinline__ uint32_t queue_take(uint32_t *c)
{
    return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

struct TileQueue {
    uint32_t *ctr;   // kQueues counters, or null: static order (ids b, b + grid, ...)
    int total;
    int Q;
    int home;
    int tried;       // thread 0: queues found empty so far
    uint32_t got;    // thread 0: counter value of the last take
    int chunk;       // consecutive ids per queue chunk

    __device__ void init(uint32_t *c, int tot, int ch = kQueueChunk)
    {
        ctr = c;
        total = tot;
        chunk = ch;
        Q = (gridDim.x % kQueues) == 0 ? kQueues : 1;
        home = (int)blockIdx.x % Q;
        tried = 0;
        got = 0;
    }
    __device__ uint32_t *counter() const { return ctr + ((home + tried) % Q) * kQueueStride; }
    __device__ int id_of(uint32_t i) const
    {
        const int qi = (home + tried) % Q;
        const int64_t t = ((int64_t)(i / (uint32_t)chunk) * Q + qi) * chunk + i % (uint32_t)chunk;
        return t < total ? (int)t : total;
    }
    // Thread 0: ids from the current queue onwards until one is in range;
    // returns `total` once every queue is empty (at most Q failed takes).
    __device__ int take_from(uint32_t i)
    {
        int t = id_of(i);
        while (t >= total && ++tried < Q) t = id_of(queue_take(counter()));
        return t;
    }
    // Thread 0: start taking an id (the atomic's latency then overlaps
    // whatever the workgroup issues next) ...
    __device__ void issue()
    {
        if (ctr && tried < Q) got = queue_take(counter());
    }
    // ... and finish: the id the workgroup runs after `tile`.
    __device__ int resolve(int tile)
    {
        if (!ctr) return tile + (int)gridDim.x;
        return tried < Q ? take_from(got) : total;
    }
    // All threads: the first tile id (from thread 0 through s_id).
    __device__ int first(int *s_id)
    {
        if (!ctr) return xcd_logical_id();
        if (threadIdx.x == 0) {
            issue();
            *s_id = resolve(0);
        }
        __syncthreads();
        return __builtin_amdgcn_readfirstlane(*s_id);
    }
};

// The dynamic-LDS limit granted to one kernel (hipFuncSetAttribute), kept
// per device and raised only under a lock, so concurrent callers never
// lower a limit another thread's launch relies on; the fast path is one
// atomic load.
constexpr int kMaxDevices = 64;
struct LdsLimit {
    std::atomic<int> granted[kMaxDevices] = {};
    std::mutex mu;
    hipError_t ensure(const void *kern, int lds)
    {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices)
            return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (granted[dev].load(std::memory_order_acquire) >= lds) return hipSuccess;
        std::lock_guard<std::mutex> lock(mu);
        if (granted[dev].load(std::memory_order_relaxed) >= lds) return hipSuccess;
        e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e == hipSuccess) granted[dev].store(lds, std::memory_order_release);
        return e;
    }
};

// Grid of a persistent launch: enough workgroups to fill every CU at the
// kernel's occupancy, never more than there are tiles, a multiple of the 8
// XCDs when possible.
inline int64_t persistent_grid(int occ, int64_t tiles_max)
{
    int64_t grid = (int64_t)device_cus() * (occ < 1 ? 1 : occ);
    if (tiles_max < grid) grid = tiles_max;
    if (grid >= 8) grid = grid / 8 * 8;
    return grid < 1 ? 1 : grid;
}

}  // namespace
}  // namespace ptgg
