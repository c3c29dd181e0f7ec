// gemm_bf16.hip -- BF16 grouped GEMM for gfx950: forward (with optional fused
// SwiGLU epilogue), data gradient and variable-length weight gradient.
//
// One persistent kernel walks the ragged batch: every workgroup builds the
// expert/tile table in LDS from the device-resident group lengths, then takes
// linear tile ids in an XCD-aware order.  Tiles are BM x BN outputs; the
// reduction runs in BK-deep steps staged through double-buffered LDS and fed
// to v_mfma_f32_32x32x16_bf16 (fp32 accumulate).
//
//  forward / dgrad:  C[m, j] = sum_q A[m, q] * Bop(j, q), m in one expert's
//                    rows.  Bop is read either reduction-contiguous ([j][q])
//                    or column-contiguous ([q][j], transposed on the way into
//                    LDS).
//  wgrad:            D[i, j] = sum over the expert's rows r of A[r, i] * B[r, j];
//                    both operands are read row-by-row (transposed into LDS)
//                    and the result is added into the fp32 main_grad once.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace ptgg {

namespace {

constexpr int BM = kTileM, BN = kTileN, BK = 64;
constexpr int LDS_STRIDE = BK + 8;                  // bf16 per LDS row: 144 B
constexpr int TILE_A = BM * LDS_STRIDE;             // elements
constexpr int TILE_B = BN * LDS_STRIDE;
constexpr int STAGE = TILE_A + TILE_B;
constexpr int GEMM_LDS_BYTES = 2 * STAGE * 2;       // two stages of bf16

struct Frag {
    uintx4 v[4];
};

// -------------------------------------------------------------- loaders
// Reduction-contiguous operand: 128 tile rows x 64 reduction values, four
// 16-byte chunks per thread.  Row index r maps to a source row via `rowptr`.
template <class RowPtr>
__device__ __forceinline__ void load_kcontig(Frag &f, RowPtr rowptr, int k0, int Kred)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kThreads;
        int r = c >> 3, kc = c & 7;
        int k = k0 + kc * 8;
        if (k < Kred)
            f.v[i] = *(const uintx4 *)(rowptr(r) + k);
        else
            f.v[i] = uintx4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void store_kcontig(const Frag &f, uint16_t *s)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kThreads;
        int r = c >> 3, kc = c & 7;
        *(uintx4 *)(s + r * LDS_STRIDE + kc * 8) = f.v[i];
    }
}

// Column-contiguous operand: the source is [reduction][columns]; each thread
// reads 4 reduction rows x 8 columns (four 16-byte loads) and writes the
// transposed 8 x 4 block, so LDS holds [column][reduction] like the other
// operand.  colptr(q, c8) returns the source address of reduction index q,
// tile columns c8..c8+7, or nullptr when the row is outside the reduction.
template <class ColPtr>
__device__ __forceinline__ void load_ncontig(Frag &f, ColPtr colptr, int q0)
{
    const int kb = threadIdx.x & 15, nb = threadIdx.x >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t *src = colptr(q0 + kb * 4 + i, nb * 8);
        f.v[i] = src ? *(const uintx4 *)src : uintx4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void store_ncontig(const Frag &f, uint16_t *s)
{
    const int kb = threadIdx.x & 15, nb = threadIdx.x >> 4;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t r0 = f.v[0][d], r1 = f.v[1][d], r2 = f.v[2][d], r3 = f.v[3][d];
        uintx2 lo, hi;
        lo[0] = (r0 & 0xFFFFu) | (r1 << 16);
        lo[1] = (r2 & 0xFFFFu) | (r3 << 16);
        hi[0] = (r0 >> 16) | (r1 & 0xFFFF0000u);
        hi[1] = (r2 >> 16) | (r3 & 0xFFFF0000u);
        *(uintx2 *)(s + (nb * 8 + 2 * d) * LDS_STRIDE + kb * 4) = lo;
        *(uintx2 *)(s + (nb * 8 + 2 * d + 1) * LDS_STRIDE + kb * 4) = hi;
    }
}

// -------------------------------------------------------------- MFMA step
// Wave (wm, wn) owns the 64 x 64 sub-tile at (wm*64, wn*64): 2 x 2 blocks of
// 32 x 32.  Lane l supplies row (l & 31) of A and column (l & 31) of B with 8
// reduction values at offset (l >> 5) * 8 of each 16-deep step.
__device__ __forceinline__ void mma_stage(floatx16 (&acc)[2][2], const uint16_t *sA,
                                          const uint16_t *sB, int wm, int wn, int nvalid_bi)
{
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
            af[bi] = *(const bf16x8 *)(sA + (wm * 64 + bi * 32 + r) * LDS_STRIDE + ks * 16 + kh);
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
            bf[bj] = *(const bf16x8 *)(sB + (wn * 64 + bj * 32 + r) * LDS_STRIDE + ks * 16 + kh);
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
            if (bi < nvalid_bi) {
#pragma unroll
                for (int bj = 0; bj < 2; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bi], bf[bj], acc[bi][bj], 0, 0, 0);
            }
        }
    }
}

template <int KIND, int EPI>
__global__ __launch_bounds__(kThreads) void gg_bf16_kernel(Bf16Params p)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint16_t *stage0 = (uint16_t *)smem;
    GroupTable tab;
    tab.G = p.G;
    int *tb = (int *)(smem + GEMM_LDS_BYTES);
    tab.row0 = tb;
    tab.rows = tb + p.G;
    tab.tile0 = tb + 2 * p.G;
    int *s_scan = tab.tile0 + p.G + 1;

    int total;
    if (KIND == kWgrad)
        total = build_group_table(tab, p.lens, p.offs, p.G, p.M,
                                  TilesWgrad{p.tilesM * p.tilesN, p.accumulate}, p.err, s_scan);
    else
        total = build_group_table(tab, p.lens, p.offs, p.G, p.M, TilesFwd{BM, p.tilesN}, p.err, s_scan);

    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    for (int tile = xcd_logical_id(); tile < total; tile += gridDim.x) {
        const int g = find_group(tab, tile);
        const int local = tile - tab.tile0[g];
        const int row0 = tab.row0[g], rows = tab.rows[g];
        int mt, nt;
        if (KIND == kWgrad) {
            mt = local / p.tilesN;
            nt = local % p.tilesN;
        } else {
            const int tm = (rows + BM - 1) / BM;
            nt = local / tm;
            mt = local % tm;
        }
        const int m0 = mt * BM;

        floatx16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        // operand address functors
        const uint16_t *Arow = p.a + (int64_t)row0 * p.lda;
        const uint16_t *Bg = (KIND == kWgrad) ? p.b + (int64_t)row0 * p.ldb : p.b + (int64_t)g * p.b_gstride;
        const int Kred = (KIND == kWgrad) ? rows : p.Kred;
        const int nk = (Kred + BK - 1) / BK;
        int nvalid_bi = 2;
        if (KIND != kWgrad) {
            const int vr = min(BM, rows - m0) - wm * 64;   // valid rows in this wave
            nvalid_bi = vr <= 0 ? 0 : (vr > 32 ? 2 : 1);
        }

        auto a_rowptr = [&](int r) { return Arow + (int64_t)min(m0 + r, rows - 1) * p.lda; };
        auto b_rowptr = [&](int c) {
            int n = clamp_col<EPI>(map_col<EPI>(nt, c, p.Nout), p.Nout, 1);
            return Bg + (int64_t)n * p.ldb;
        };
        auto b_colptr = [&](int q, int c8) -> const uint16_t * {
            if (q >= Kred) return nullptr;
            int n = clamp_col<EPI>(map_col<EPI>(nt, c8, p.Nout), p.Nout, 8);
            return Bg + (int64_t)q * p.ldb + n;
        };
        // wgrad: A operand columns are the output rows i
        auto wa_colptr = [&](int q, int c8) -> const uint16_t * {
            if (q >= rows) return nullptr;
            int i = min(m0 + c8, p.Mout - 8);
            return Arow + (int64_t)q * p.lda + i;
        };
        auto wb_colptr = [&](int q, int c8) -> const uint16_t * {
            if (q >= rows) return nullptr;
            int n = min(nt * BN + c8, p.Nout - 8);
            return Bg + (int64_t)q * p.ldb + n;
        };

        Frag fa, fb;
        auto load = [&](int kt) {
            const int k0 = kt * BK;
            if (KIND == kWgrad) {
                load_ncontig(fa, wa_colptr, k0);
                load_ncontig(fb, wb_colptr, k0);
            } else {
                load_kcontig(fa, a_rowptr, k0, Kred);
                if (KIND == kFwdKContig)
                    load_kcontig(fb, b_rowptr, k0, Kred);
                else
                    load_ncontig(fb, b_colptr, k0);
            }
        };
        auto store = [&](uint16_t *st) {
            if (KIND == kWgrad) {
                store_ncontig(fa, st);
                store_ncontig(fb, st + TILE_A);
            } else {
                store_kcontig(fa, st);
                if (KIND == kFwdKContig)
                    store_kcontig(fb, st + TILE_A);
                else
                    store_ncontig(fb, st + TILE_A);
            }
        };

        if (nk > 0) {
            load(0);
            store(stage0);
        }
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            uint16_t *cur = stage0 + (kt & 1) * STAGE;
            uint16_t *nxt = stage0 + ((kt + 1) & 1) * STAGE;
            if (kt + 1 < nk) load(kt + 1);
            mma_stage(acc, cur, cur + TILE_A, wm, wn, nvalid_bi);
            if (kt + 1 < nk) store(nxt);
            __syncthreads();
        }

        // ------------------------------------------------------ epilogue
        if (KIND == kWgrad) {
            float *og = (float *)p.out + (int64_t)g * p.o_gstride;
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 2; ++bj) {
                    const int n = nt * BN + acc_col(wn, bj);
                    if (n >= p.Nout) continue;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = m0 + acc_row(wm, bi, r);
                        if (i < p.Mout) {
                            float *dst = og + (int64_t)i * p.ldo + n;
                            float v = acc[bi][bj][r];
                            if (p.accumulate) v = *dst + v;
                            *dst = v;
                        }
                    }
                }
        } else {
            store_tile<EPI>(acc, p.out, p.out_scale, row0, m0, rows, nt, p.Nout, p.ldo);
        }
    }
}

template <int KIND, int EPI>
hipError_t launch_one(const Bf16Params &p, hipStream_t s)
{
    const int lds = GEMM_LDS_BYTES + table_bytes(p.G);
    auto kern = gg_bf16_kernel<KIND, EPI>;
    static int configured_lds = 0;
    static int occupancy = 0;
    if (configured_lds < lds) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        configured_lds = lds;
        occupancy = 0;
    }
    int occ = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kThreads, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    (void)occupancy;
    int64_t tiles_max;
    if (KIND == kWgrad)
        tiles_max = (int64_t)p.G * p.tilesM * p.tilesN;
    else
        tiles_max = (p.M / BM + p.G) * (int64_t)p.tilesN;
    int64_t grid = (int64_t)device_cus() * occ;
    if (tiles_max < grid) grid = tiles_max;
    if (grid >= 8) grid = grid / 8 * 8;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

}  // namespace

int bf16_tile_m() { return BM; }
int bf16_tile_n() { return BN; }

hipError_t launch_bf16(const Bf16Params &p, int kind, int epi, hipStream_t s)
{
    if (kind == kWgrad) return launch_one<kWgrad, kEpiNone>(p, s);
    if (kind == kFwdKContig) {
        if (epi == kEpiSwiglu) return launch_one<kFwdKContig, kEpiSwiglu>(p, s);
        if (epi == kEpiSwigluMxfp4) return launch_one<kFwdKContig, kEpiSwigluMxfp4>(p, s);
        return launch_one<kFwdKContig, kEpiNone>(p, s);
    }
    if (epi == kEpiSwiglu) return launch_one<kFwdNContig, kEpiSwiglu>(p, s);
    if (epi == kEpiSwigluMxfp4) return launch_one<kFwdNContig, kEpiSwigluMxfp4>(p, s);
    return launch_one<kFwdNContig, kEpiNone>(p, s);
}

}  // namespace ptgg
