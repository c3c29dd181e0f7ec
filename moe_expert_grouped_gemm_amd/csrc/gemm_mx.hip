// gemm_mx.hip -- OCP-MX grouped GEMM forward for gfx950 (MXFP8 E4M3 and
// MXFP4 E2M1 operands, one E8M0 scale per 32 values along K).
//
// Same persistent ragged-batch schedule as the BF16 kernel.  Both operands are
// K-contiguous (activations [M, K], weights [G, N, K], the [experts, out, in]
// layout).  Each 128-byte slice of a row per k-step (128 E4M3 or 256 E2M1
// values) is staged through double-buffered LDS together with its 4 or 8
// scale bytes, and fed to v_mfma_scale_f32_32x32x64_f8f6f4: lane l supplies
// row (l & 31) with the 32 values of one scale block and that block's E8M0
// byte, so the block scales are applied inside the matrix core and the fp32
// accumulator receives exactly-scaled products.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace ptgg {

namespace {

constexpr int BM = kTileM, BN = kTileN;
constexpr int BKB = 128;                       // code bytes per row per k-step
constexpr int LDS_STRIDE = BKB + 16;           // 144 B rows (conflict-free 16-B reads)
constexpr int SC_STRIDE = 8;                   // scale bytes per row per k-step (<= 8 blocks)
constexpr int TILE_A = BM * LDS_STRIDE;
constexpr int TILE_B = BN * LDS_STRIDE;
constexpr int TILE_AS = BM * SC_STRIDE;
constexpr int TILE_BS = BN * SC_STRIDE;
constexpr int STAGE = TILE_A + TILE_B + TILE_AS + TILE_BS;
constexpr int GEMM_LDS_BYTES = 2 * STAGE;

// FMT 0: E4M3 (one byte per value, 128 values per k-step, 4 scale blocks)
// FMT 1: E2M1 (two values per byte, 256 values per k-step, 8 scale blocks)
template <int FMT>
struct Fmt {
    static constexpr int vals_per_byte = FMT == 0 ? 1 : 2;
    static constexpr int blocks = BKB * vals_per_byte / 32;   // scale blocks per k-step
    static constexpr int mfma_fmt = FMT == 0 ? 0 : 4;         // cbsz/blgp operand format
    static constexpr int bytes_per_lane = 32 / vals_per_byte; // one scale block
};

struct Stage {
    uintx4 a[4], b[4];
    uintx2 sc;          // this thread's row of scale bytes (A rows, then B rows)
};

template <int FMT>
__device__ __forceinline__ void load_stage(Stage &st, const uint8_t *Ab, const uint8_t *Asb,
                                           const uint8_t *Bb, const uint8_t *Bsb, int m0, int rows,
                                           int n0, int N, int Kb, int KS, int kt)
{
    using F = Fmt<FMT>;
    const int kb0 = kt * BKB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = threadIdx.x + i * kThreads;
        const int r = c >> 3, kc = c & 7;
        const int k = kb0 + kc * 16;
        const bool kv = k < Kb;
        const int ar = min(m0 + r, rows - 1);
        const int br = min(n0 + r, N - 1);
        st.a[i] = kv ? *(const uintx4 *)(Ab + (int64_t)ar * Kb + k) : uintx4{0u, 0u, 0u, 0u};
        st.b[i] = kv ? *(const uintx4 *)(Bb + (int64_t)br * Kb + k) : uintx4{0u, 0u, 0u, 0u};
    }
    // scales: thread t < 128 loads A row t, t >= 128 loads B row t - 128
    const int t = threadIdx.x;
    const uint8_t *srow = t < BM ? Asb + (int64_t)min(m0 + t, rows - 1) * KS
                                 : Bsb + (int64_t)min(n0 + t - BM, N - 1) * KS;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < F::blocks; ++j) {
        const int blk = kt * F::blocks + j;
        const uint32_t v = blk < KS ? (uint32_t)srow[blk] : 0u;
        w[j >> 2] |= v << (8 * (j & 3));
    }
    st.sc = uintx2{w[0], w[1]};
}

__device__ __forceinline__ void store_stage(const Stage &st, uint8_t *s)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = threadIdx.x + i * kThreads;
        const int r = c >> 3, kc = c & 7;
        *(uintx4 *)(s + r * LDS_STRIDE + kc * 16) = st.a[i];
        *(uintx4 *)(s + TILE_A + r * LDS_STRIDE + kc * 16) = st.b[i];
    }
    *(uintx2 *)(s + TILE_A + TILE_B + threadIdx.x * SC_STRIDE) = st.sc;
}

// One k-step of 2 x 2 blocks of 32 x 32 per wave.  MFMA step s covers the 64
// values of scale blocks 2s and 2s+1 of the k-step; lane half h = l >> 5
// supplies the E8M0 byte of block 2s + h.  Which operand bytes that scale
// multiplies depends on the element width (measured on gfx950):
//  - E2M1: the lane's 16 bytes (32 values) all belong to the lane's own
//    scale, so lane half h holds block 2s + h whole;
//  - E4M3: bytes 0-15 of BOTH lane halves take half 0's scale and bytes
//    16-31 take half 1's, so lane half h holds values 16h..16h+15 of block
//    2s in bytes 0-15 and values 16h..16h+15 of block 2s+1 in bytes 16-31.
template <int FMT>
__device__ __forceinline__ void mma_stage(floatx16 (&acc)[2][2], const uint8_t *s, int wm, int wn,
                                          int nvalid_bi)
{
    using F = Fmt<FMT>;
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, h = lane >> 5;
    const uint8_t *sA = s, *sB = s + TILE_A;
    const uint8_t *sAs = s + TILE_A + TILE_B, *sBs = sAs + TILE_AS;
    uintx2 ascale[2], bscale[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) ascale[bi] = *(const uintx2 *)(sAs + (wm * 64 + bi * 32 + r) * SC_STRIDE);
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) bscale[bj] = *(const uintx2 *)(sBs + (wn * 64 + bj * 32 + r) * SC_STRIDE);
#pragma unroll
    for (int st = 0; st < F::blocks / 2; ++st) {
        const int blk = 2 * st + h;                 // scale block of this lane
        // byte offsets (in the row's k-step slice) of the lane's two 16-byte halves
        const int off_lo = FMT == 0 ? 64 * st + 16 * h : 16 * blk;
        const int off_hi = 64 * st + 32 + 16 * h;  // E4M3 only
        intx8 af[2], bf[2];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
            const uint8_t *p = sA + (wm * 64 + bi * 32 + r) * LDS_STRIDE;
            intx4 lo = *(const intx4 *)(p + off_lo);
            intx4 hi = FMT == 0 ? *(const intx4 *)(p + off_hi) : intx4{0, 0, 0, 0};
            af[bi] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const uint8_t *p = sB + (wn * 64 + bj * 32 + r) * LDS_STRIDE;
            intx4 lo = *(const intx4 *)(p + off_lo);
            intx4 hi = FMT == 0 ? *(const intx4 *)(p + off_hi) : intx4{0, 0, 0, 0};
            bf[bj] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        int as[2], bs[2];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) as[bi] = (int)((ascale[bi][blk >> 2] >> (8 * (blk & 3))) & 0xFFu);
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) bs[bj] = (int)((bscale[bj][blk >> 2] >> (8 * (blk & 3))) & 0xFFu);
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
            if (bi < nvalid_bi) {
#pragma unroll
                for (int bj = 0; bj < 2; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[bi], bf[bj], acc[bi][bj], F::mfma_fmt, F::mfma_fmt, 0, as[bi], 0, bs[bj]);
            }
        }
    }
}

template <int FMT, int EPI>
__global__ __launch_bounds__(kThreads) void gg_mx_kernel(MxParams p)
{
    using F = Fmt<FMT>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint8_t *stage0 = (uint8_t *)smem;
    GroupTable tab;
    tab.G = p.G;
    int *tb = (int *)(smem + GEMM_LDS_BYTES);
    tab.row0 = tb;
    tab.rows = tb + p.G;
    tab.tile0 = tb + 2 * p.G;
    int *s_scan = tab.tile0 + p.G + 1;
    const int total = build_group_table(tab, p.lens, p.offs, p.G, p.M, TilesFwd{BM, p.tilesN}, p.err, s_scan);

    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int Kb = p.K / F::vals_per_byte;     // code bytes per row
    const int KS = p.K / 32;                   // scale bytes per row
    const int nk = (Kb + BKB - 1) / BKB;

    for (int tile = xcd_logical_id(); tile < total; tile += gridDim.x) {
        const int g = find_group(tab, tile);
        const int local = tile - tab.tile0[g];
        const int row0 = tab.row0[g], rows = tab.rows[g];
        const int tm = (rows + BM - 1) / BM;
        const int nt = local / tm, mt = local % tm;
        const int m0 = mt * BM;
        const int vr = min(BM, rows - m0) - wm * 64;
        const int nvalid_bi = vr <= 0 ? 0 : (vr > 32 ? 2 : 1);

        floatx16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        const uint8_t *Ab = p.a + (int64_t)row0 * Kb;
        const uint8_t *Asb = p.as + (int64_t)row0 * KS;
        const uint8_t *Bb = p.b + (int64_t)g * p.N * Kb;
        const uint8_t *Bsb = p.bs + (int64_t)g * p.N * KS;
        // B rows of this tile: for SwiGLU the tile's 128 rows are 64 gate rows
        // and the 64 matching up rows, interleaved per wave (see map_col)
        Stage st;
        auto load = [&](int kt) {
            if (EPI == kEpiNone) {
                load_stage<FMT>(st, Ab, Asb, Bb, Bsb, m0, rows, nt * BN, p.N, Kb, KS, kt);
            } else {
                // gather: B row c of the tile is weight row map_col(nt, c)
                const int kb0 = kt * BKB;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = threadIdx.x + i * kThreads;
                    const int r = c >> 3, kc = c & 7;
                    const int k = kb0 + kc * 16;
                    const bool kv = k < Kb;
                    const int ar = min(m0 + r, rows - 1);
                    const int br = clamp_col<EPI>(map_col<EPI>(nt, r, p.N), p.N, 1);
                    st.a[i] = kv ? *(const uintx4 *)(Ab + (int64_t)ar * Kb + k) : uintx4{0u, 0u, 0u, 0u};
                    st.b[i] = kv ? *(const uintx4 *)(Bb + (int64_t)br * Kb + k) : uintx4{0u, 0u, 0u, 0u};
                }
                const int t = threadIdx.x;
                const uint8_t *srow = t < BM ? Asb + (int64_t)min(m0 + t, rows - 1) * KS
                                             : Bsb + (int64_t)clamp_col<EPI>(map_col<EPI>(nt, t - BM, p.N), p.N, 1) * KS;
                uint32_t w[2] = {0u, 0u};
#pragma unroll
                for (int j = 0; j < F::blocks; ++j) {
                    const int blk = kt * F::blocks + j;
                    const uint32_t v = blk < KS ? (uint32_t)srow[blk] : 0u;
                    w[j >> 2] |= v << (8 * (j & 3));
                }
                st.sc = uintx2{w[0], w[1]};
            }
        };

        load(0);
        store_stage(st, stage0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            uint8_t *cur = stage0 + (kt & 1) * STAGE;
            uint8_t *nxt = stage0 + ((kt + 1) & 1) * STAGE;
            if (kt + 1 < nk) load(kt + 1);
            mma_stage<FMT>(acc, cur, wm, wn, nvalid_bi);
            if (kt + 1 < nk) store_stage(st, nxt);
            __syncthreads();
        }
        store_tile<EPI>(acc, p.out, p.out_scale, row0, m0, rows, nt, p.N, p.ldo);
    }
}

template <int FMT, int EPI>
hipError_t launch_one(const MxParams &p, hipStream_t s)
{
    const int lds = GEMM_LDS_BYTES + table_bytes(p.G);
    auto kern = gg_mx_kernel<FMT, EPI>;
    static int configured_lds = 0;
    if (configured_lds < lds) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        configured_lds = lds;
    }
    int occ = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kThreads, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    const int64_t tiles_max = (p.M / BM + p.G) * (int64_t)p.tilesN;
    int64_t grid = (int64_t)device_cus() * occ;
    if (tiles_max < grid) grid = tiles_max;
    if (grid >= 8) grid = grid / 8 * 8;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

}  // namespace

int mx_tile_m() { return BM; }
int mx_tile_n() { return BN; }

hipError_t launch_mx(const MxParams &p, int fmt, int epi, hipStream_t s)
{
    if (fmt == 0) {
        if (epi == kEpiSwiglu) return launch_one<0, kEpiSwiglu>(p, s);
        if (epi == kEpiSwigluMxfp4) return launch_one<0, kEpiSwigluMxfp4>(p, s);
        return launch_one<0, kEpiNone>(p, s);
    }
    if (epi == kEpiSwiglu) return launch_one<1, kEpiSwiglu>(p, s);
    if (epi == kEpiSwigluMxfp4) return launch_one<1, kEpiSwigluMxfp4>(p, s);
    return launch_one<1, kEpiNone>(p, s);
}

}  // namespace ptgg
