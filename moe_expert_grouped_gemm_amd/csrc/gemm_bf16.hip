// gemm_bf16.hip -- BF16 grouped GEMM for gfx950: forward (with optional fused
// SwiGLU / SwiGLU->MXFP4 epilogue), data gradient and variable-length weight
// gradient.
//
// One persistent kernel walks the ragged batch: every workgroup builds the
// expert/tile table in LDS from the device-resident group lengths, then takes
// linear tile ids in an XCD-aware order.  Tiles are 128 x 256 outputs; the
// reduction runs in 32-deep steps through an NSTAGE-deep ring of LDS buffers
// filled by direct buffer->LDS loads (buffer_load_dwordx4 ... lds), so several
// steps of operand traffic are in flight while the matrix cores work on the
// oldest one.  Each operand of a tile gets a buffer resource whose record
// bound is exactly the expert's slice, a fixed 32-bit offset per lane and a
// scalar offset that advances one step per k-step: issuing a stage costs no
// vector ALU work, and rows past an expert's end read as zeros.  The last,
// partial k-step (if any) gives every lane an explicit bound check instead.
//
// Operands are kept in LDS in the layout they have in memory:
//  - reduction-contiguous ([row][k]): 16-byte chunks XOR-swizzled by row,
//    read with ds_read_b128;
//  - column-contiguous ([k][col]): 16-byte chunks XOR-swizzled by k, read
//    with the gfx950 transposing ds_read_b64_tr_b16, which hands every lane
//    four consecutive k values of one column.
// Fragment reads are issued as inline asm with immediate offsets from
// per-lane bases computed once: the compiler cannot tell them apart from
// reads of the LDS still being filled by the in-flight direct loads and would
// otherwise wait for every outstanding load before each of them.
//
//  forward / dgrad:  C[m, j] = sum_q A[m, q] * Bop(j, q), m in one expert's
//                    rows; A is reduction-contiguous, Bop either layout.
//  wgrad:            D[i, j] = sum over the expert's rows r of A[r, i] * B[r, j];
//                    both operands column-contiguous; the result is added
//                    into the fp32 main_grad once per element.
#include <stdlib.h>

#include "pipeline.hpp"

namespace ptgg {

namespace {

constexpr int BK = ROW_BYTES / 2;                  // bf16 reduction depth of a stage

template <int V>
struct IC { static constexpr int value = V; };

// Wait for the oldest in-flight stage when `after` younger stages (of LOADS
// loads per thread each; at most NSTAGE - 1) may stay outstanding.
template <int NSTAGE>
__device__ __forceinline__ void wait_stage(int after)
{
    static_assert(NSTAGE >= 2 && NSTAGE <= 6, "extend wait_stage");
    switch (after) {
    case 5: wait_vmcnt<(NSTAGE > 5 ? 5 : NSTAGE - 1) * LOADS>(); break;
    case 4: wait_vmcnt<(NSTAGE > 4 ? 4 : NSTAGE - 1) * LOADS>(); break;
    case 3: wait_vmcnt<(NSTAGE > 3 ? 3 : NSTAGE - 1) * LOADS>(); break;
    case 2: wait_vmcnt<(NSTAGE > 2 ? 2 : NSTAGE - 1) * LOADS>(); break;
    case 1: wait_vmcnt<LOADS>(); break;
    default: wait_vmcnt<0>(); break;
    }
}

template <int OFF>
__device__ __forceinline__ bf16x8 ldsr_b128(uint32_t addr)
{
    return __builtin_bit_cast(bf16x8, ldsr_u128<OFF>(addr));
}
template <int OFF>
__device__ __forceinline__ uintx2 ldsr_tr(uint32_t addr)
{
    uintx2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
__device__ __forceinline__ bf16x8 join(uintx2 lo, uintx2 hi)
{
    return __builtin_bit_cast(bf16x8, uintx4{lo[0], lo[1], hi[0], hi[1]});
}

// Wait for all issued LDS reads; the fragments pass through the asm so no
// use of them can be scheduled before the wait.
__device__ __forceinline__ void frag_wait(bf16x8 (&a)[2], bf16x8 (&b)[4])
{
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}

// Column-contiguous operand with R columns in one stage: LDS [32][R] (rows of
// R*2 bytes), chunk c of k-row k at position c ^ ((k & 3) << 2), read with the
// transposing ds_read_b64_tr_b16.
__device__ __forceinline__ int npos(int k, int c) { return c ^ ((k & 3) << 2); }
// slot s of a column-contiguous stage with R columns: k row and source chunk
template <int R>
__device__ __forceinline__ void nslot(int s, int &k, int &c) { k = s / (R / 8); c = npos(k, s % (R / 8)); }

// Issue stage kt of both operands into ring slot kt % NSTAGE.  Full k-steps
// advance the scalar offset; the partial last step bounds every lane.
template <int KIND, int NSTAGE>
__device__ __forceinline__ void issue_stage(uint8_t *smem, const Dma<A_LOADS> &da, const Dma<B_LOADS> &db, int kt,
                                            int nfull, int Kred, int wave)
{
    const int tid = threadIdx.x;
    const uint32_t st = (uint32_t)(kt % NSTAGE) * STAGE_BYTES;
    if (kt < nfull) {
        issue(smem, da, st, kt * da.kstep, da.voff, wave);
        issue(smem, db, st + A_BYTES, kt * db.kstep, db.voff, wave);
        return;
    }
    uint32_t va[A_LOADS], vb[B_LOADS];
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
        int x, c;
        bool ok;
        if (KIND == kWgrad) { nslot<BM>(i * kThreads + tid, x, c); ok = k0 + x < Kred; }
        else { kslot(i * kThreads + tid, x, c); ok = k0 + c * 8 < Kred; }
        va[i] = ok ? da.voff[i] + kt * da.kstep : kOOB;
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
        int x, c;
        bool ok;
        if (KIND == kFwdKContig) { kslot(i * kThreads + tid, x, c); ok = k0 + c * 8 < Kred; }
        else { nslot<BN>(i * kThreads + tid, x, c); ok = k0 + x < Kred; }
        vb[i] = ok ? db.voff[i] + kt * db.kstep : kOOB;
    }
    issue(smem, da, st, 0u, va, wave);
    issue(smem, db, st + A_BYTES, 0u, vb, wave);
}

// Fragments of k-step KS of one stage at LDS byte address `so`: A rows
// (wm*64 + bi*32 ..) and B columns (wn*128 + bj*32 ..) of this wave, from the
// per-lane bases computed once per kernel.
template <int KIND, int KS>
__device__ __forceinline__ void load_frags(uint32_t so, const uint32_t (&aK)[2], const uint32_t (&aN)[2],
                                           const uint32_t (&bK)[2], const uint32_t (&bN)[4],
                                           bf16x8 (&af)[2], bf16x8 (&bfr)[4])
{
    constexpr int AO = KS * 16 * BM * 2, AJ = 4 * BM * 2;           // column-contiguous A
    constexpr int BO = A_BYTES + KS * 16 * BN * 2, BJ = 4 * BN * 2;  // column-contiguous B
    if constexpr (KIND == kWgrad) {
        af[0] = join(ldsr_tr<AO>(so + aN[0]), ldsr_tr<AO + AJ>(so + aN[0]));
        af[1] = join(ldsr_tr<AO>(so + aN[1]), ldsr_tr<AO + AJ>(so + aN[1]));
    } else {
        af[0] = ldsr_b128<0>(so + aK[KS]);
        af[1] = ldsr_b128<32 * 64>(so + aK[KS]);
    }
    if constexpr (KIND == kFwdKContig) {
        bfr[0] = ldsr_b128<A_BYTES + 0 * 32 * 64>(so + bK[KS]);
        bfr[1] = ldsr_b128<A_BYTES + 1 * 32 * 64>(so + bK[KS]);
        bfr[2] = ldsr_b128<A_BYTES + 2 * 32 * 64>(so + bK[KS]);
        bfr[3] = ldsr_b128<A_BYTES + 3 * 32 * 64>(so + bK[KS]);
    } else {
        bfr[0] = join(ldsr_tr<BO>(so + bN[0]), ldsr_tr<BO + BJ>(so + bN[0]));
        bfr[1] = join(ldsr_tr<BO>(so + bN[1]), ldsr_tr<BO + BJ>(so + bN[1]));
        bfr[2] = join(ldsr_tr<BO>(so + bN[2]), ldsr_tr<BO + BJ>(so + bN[2]));
        bfr[3] = join(ldsr_tr<BO>(so + bN[3]), ldsr_tr<BO + BJ>(so + bN[3]));
    }
}

// ------------------------------------------------------------------ kernel
template <int KIND, int EPI, int NSTAGE>
__global__ __launch_bounds__(kThreads, 2) void gg_bf16_kernel(Bf16Params p)
{
    constexpr int GEMM_LDS_BYTES = NSTAGE * STAGE_BYTES;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
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
    total = __builtin_amdgcn_readfirstlane(total);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t lds0 = lds_addr(smem);

    // ---- per-lane LDS read bases (fixed for the kernel)
    const int r32 = lane & 31, h = lane >> 5, g16 = (lane >> 4) & 1, s16 = lane & 15;
    uint32_t aK[2], bK[2], aN[2], bN[4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int ra = wm * 64 + r32, rb = wn * 128 + r32;
        aK[ks] = ra * 64 + kpos(ra, 2 * ks + h) * 16;
        bK[ks] = rb * 64 + kpos(rb, 2 * ks + h) * 16;
    }
    {
        const int krow = h * 8 + (s16 >> 2);                 // k & 3 == (s16 >> 2) & 3
        const int lo = 8 * (s16 & 1);                        // byte offset inside the chunk
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
            const int col = wm * 64 + bi * 32 + 16 * g16 + 4 * (s16 & 3);
            aN[bi] = krow * (BM * 2) + npos(krow, col >> 3) * 16 + lo;
        }
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int col = wn * 128 + bj * 32 + 16 * g16 + 4 * (s16 & 3);
            bN[bj] = krow * (BN * 2) + npos(krow, col >> 3) * 16 + lo;
        }
    }

    for (int tile = xcd_logical_id(); tile < total; tile += gridDim.x) {
        const int g = __builtin_amdgcn_readfirstlane(find_group(tab, tile));
        const int local = tile - __builtin_amdgcn_readfirstlane(tab.tile0[g]);
        const int row0 = __builtin_amdgcn_readfirstlane(tab.row0[g]);
        const int rows = __builtin_amdgcn_readfirstlane(tab.rows[g]);
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
        const int Kred = (KIND == kWgrad) ? rows : p.Kred;
        const int nk = (Kred + BK - 1) / BK, nfull = Kred / BK;
        int nvalid_bi = 2;
        if (KIND != kWgrad) {
            const int vr = min(BM, rows - m0) - wm * 64;
            nvalid_bi = vr <= 0 ? 0 : (vr > 32 ? 2 : 1);
        }

        // ---- operand buffers and per-lane offsets for this tile
        Dma<A_LOADS> da;
        Dma<B_LOADS> db;
        const uint16_t *Arow = p.a + (int64_t)row0 * p.lda;
        if (KIND == kWgrad) {
            // A operand: [token][i] slice of the expert, columns m0.. of A
            da.base = Arow;
            da.bytes = (uint32_t)rows * p.lda * 2;
            da.kstep = BK * p.lda * 2;
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i) {
                int k, c;
                nslot<BM>(i * kThreads + tid, k, c);
                da.voff[i] = (uint32_t)(k * p.lda + min(m0 + c * 8, p.Mout - 8)) * 2;
            }
            const uint16_t *Brow = p.b + (int64_t)row0 * p.ldb;
            db.base = Brow;
            db.bytes = (uint32_t)rows * p.ldb * 2;
            db.kstep = BK * p.ldb * 2;
#pragma unroll
            for (int i = 0; i < B_LOADS; ++i) {
                int k, c;
                nslot<BN>(i * kThreads + tid, k, c);
                db.voff[i] = (uint32_t)(k * p.ldb + min(nt * BN + c * 8, p.Nout - 8)) * 2;
            }
        } else {
            // A operand: the expert's rows; rows past its end fall outside the bound
            da.base = Arow;
            da.bytes = (uint32_t)rows * p.lda * 2;
            da.kstep = BK * 2;
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i) {
                int r, c;
                kslot(i * kThreads + tid, r, c);
                da.voff[i] = (uint32_t)((m0 + r) * p.lda + c * 8) * 2;
            }
            const uint16_t *Bg = p.b + (int64_t)g * p.b_gstride;
            if (KIND == kFwdKContig) {
                db.base = Bg;
            db.bytes = (uint32_t)p.Nout * p.ldb * 2;
                db.kstep = BK * 2;
#pragma unroll
                for (int i = 0; i < B_LOADS; ++i) {
                    int r, c;
                    kslot(i * kThreads + tid, r, c);
                    int n = col_of<EPI>(nt, r, p.Nout);
                    n = !epi_glu(EPI) ? min(n, p.Nout - 1) : clamp8<EPI>(n & ~7, p.Nout) + (n & 7);
                    db.voff[i] = (uint32_t)(n * p.ldb + c * 8) * 2;
                }
            } else {
                db.base = Bg;
            db.bytes = (uint32_t)Kred * p.ldb * 2;
                db.kstep = BK * p.ldb * 2;
#pragma unroll
                for (int i = 0; i < B_LOADS; ++i) {
                    int k, c;
                    nslot<BN>(i * kThreads + tid, k, c);
                    const int n = clamp8<EPI>(col_of<EPI>(nt, c * 8, p.Nout), p.Nout);
                    db.voff[i] = (uint32_t)(k * p.ldb + n) * 2;
                }
            }
        }

        // Accumulators start at zero, or for an accumulating wgrad at the
        // main_grad tile itself: its loads go out before the operand
        // prologue and overlap it, and the tile ends with plain stores (both
        // non-temporal: main_grad is touched once).
        floatx16 acc[2][4];
        if (KIND == kWgrad && p.accumulate) {
            const float *og = (const float *)p.out + (int64_t)g * p.o_gstride;
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) {
                    const int n = nt * BN + wn * 128 + bj * 32 + (lane & 31);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = m0 + e_row(wm, bi, r);
                        acc[bi][bj][r] = (n < p.Nout && i < p.Mout) ? __builtin_nontemporal_load(og + (int64_t)i * p.ldo + n) : 0.0f;
                    }
                }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        }

        auto mma = [&](const bf16x8 (&af)[2], const bf16x8 (&bfr)[4]) {
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
                if (bi < nvalid_bi) {
#pragma unroll
                    for (int bj = 0; bj < 4; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bi], bfr[bj], acc[bi][bj], 0, 0, 0);
                }
        };

        // Schedule per k-step kt (two 16-deep MFMA steps per stage):
        //   read step-1 fragments of kt | MFMA step 0 of kt
        //   wait for stage kt+1, barrier (kt fully read by every wave)
        //   load stage kt+NSTAGE into kt's slot
        //   read step-0 fragments of kt+1 | MFMA step 1 of kt
        // so LDS reads overlap MFMAs and NSTAGE-1 stages stay in flight.
        static_assert(BK == 32, "two k-steps per stage");
#pragma unroll
        for (int s = 0; s < NSTAGE; ++s)
            if (s < nk) issue_stage<KIND, NSTAGE>(smem, da, db, s, nfull, Kred, wave);
        bf16x8 a0[2], b0[4], a1[2], b1[4];
        if (nk > 0) {
            wait_stage<NSTAGE>(min(NSTAGE - 1, nk - 1));
            barrier();
            load_frags<KIND, 0>(lds0, aK, aN, bK, bN, a0, b0);
            frag_wait(a0, b0);
        }
        int slot = 0;
        for (int kt = 0; kt < nk; ++kt) {
            const uint32_t so = lds0 + (uint32_t)slot * STAGE_BYTES;
            load_frags<KIND, 1>(so, aK, aN, bK, bN, a1, b1);
            mma(a0, b0);
            const int nslot_ = slot + 1 == NSTAGE ? 0 : slot + 1;
            if (kt + 1 < nk) wait_stage<NSTAGE>(min(NSTAGE - 2, nk - 2 - kt));
            frag_wait(a1, b1);
            barrier();
            if (kt + NSTAGE < nk) issue_stage<KIND, NSTAGE>(smem, da, db, kt + NSTAGE, nfull, Kred, wave);
            if (kt + 1 < nk) load_frags<KIND, 0>(lds0 + (uint32_t)nslot_ * STAGE_BYTES, aK, aN, bK, bN, a0, b0);
            mma(a1, b1);
            if (kt + 1 < nk) frag_wait(a0, b0);
            slot = nslot_;
        }
        wait_lgkm0();
        barrier();                                       // LDS free for the next tile

        if (KIND == kWgrad) {
            // Nothing is outstanding here; saying so explicitly keeps the
            // compiler from waiting for every earlier store before each one
            // (vmcnt counts stores too) when it cannot prove the seeded
            // accumulators have arrived.
            wait_vmcnt<0>();
            float *og = (float *)p.out + (int64_t)g * p.o_gstride;
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) {
                    const int n = nt * BN + wn * 128 + bj * 32 + (lane & 31);
                    if (n >= p.Nout) continue;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = m0 + e_row(wm, bi, r);
                        if (i < p.Mout) __builtin_nontemporal_store(acc[bi][bj][r], og + (int64_t)i * p.ldo + n);
                    }
                }
        } else {
            store_out<EPI>(acc, p.out, p.out_scale, p.ldo, p.Nout, row0, m0, rows, nt, wm, wn, p.swiglu_limit);
        }
    }
}

// Ring depth: a tuning knob (3..5 stages of 24 KiB); PTGG_NSTAGE overrides
// the default for experiments.  Results do not depend on it.
int ring_depth()
{
    static int depth = [] {
        const char *e = getenv("PTGG_NSTAGE");
        int d = e ? atoi(e) : 3;
        return (d >= 3 && d <= 5) ? d : 3;
    }();
    return depth;
}

template <int KIND, int EPI, int NSTAGE>
hipError_t launch_one(const Bf16Params &p, hipStream_t s)
{
    const int lds = NSTAGE * STAGE_BYTES + table_bytes(p.G);
    auto kern = gg_bf16_kernel<KIND, EPI, NSTAGE>;
    static LdsLimit lds_limit;
    hipError_t e = lds_limit.ensure((const void *)kern, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kThreads, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    int64_t tiles_max;
    if (KIND == kWgrad)
        tiles_max = (int64_t)p.G * p.tilesM * p.tilesN;
    else
        tiles_max = (p.M / BM + p.G) * (int64_t)p.tilesN;
    const int64_t grid = persistent_grid(occ, tiles_max);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

template <int KIND, int EPI>
hipError_t launch_depth(const Bf16Params &p, hipStream_t s)
{
    switch (ring_depth()) {
    case 4: return launch_one<KIND, EPI, 4>(p, s);
    case 5: return launch_one<KIND, EPI, 5>(p, s);
    default: return launch_one<KIND, EPI, 3>(p, s);
    }
}

// ====================================================================== wide
// The main BF16 kernel: one workgroup of 8 waves per CU (two waves per SIMD)
// computes 256 x 256 tiles; wave (wm, wn), wm = 0..3, owns 64 x 128 outputs
// as 2 x 4 blocks of 32 x 32, and a tile moves a third fewer operand bytes
// per product than 128 x 256.  The ring holds NSLOT stages of WK reduction
// values (WRing); the loads of stage kt + NSLOT - 1 go out at the start of
// stage kt into the slot stage kt - 1 freed, so NSLOT - 1 stages are in
// flight while one computes.  LDS: [A slots | B slots], 128 KiB in all, so
// slot and k-step offsets fit the 16-bit immediates of the fragment reads.
//  - reduction-contiguous operand: [256 rows][2 WK bytes] per slot, chunk c
//    of row r at position kswz(r, c), so that the 16 lanes of a
//    ds_read_b128 pass, reading one chunk of 16 consecutive rows, cover all
//    64 banks; the chunk 2j + h a lane reads is at base ^ (j << 5);
//  - column-contiguous operand: [WK k][512 B], chunk c of k-row k at
//    c ^ ((k & 3) << 2), read with ds_read_b64_tr_b16 (four k values of one
//    column per lane).
constexpr int WBM = 256, WBN = 256, WTHREADS = 512;

// Ring shapes: reduction values per stage and slots, for A and for B.
//   0: both 64-deep in 2 slots (128-byte rows: whole lines per load);
//   1: both 32-deep in 4 slots (three stages in flight);
//   2: A 64-deep in 2 slots, B 32-deep in 4 slots: a column-contiguous B
//      three stages ahead while A keeps whole-line rows.  The k-loop steps
//      through B's 32-deep stages; A's stage a serves steps 2a and 2a + 1.
template <int RING>
struct WRing {
    static constexpr int WKA = RING == 1 ? 32 : 64, NSA = RING == 1 ? 4 : 2;
    static constexpr int WKB = RING == 0 ? 64 : 32, NSB = RING == 0 ? 2 : 4;
    static constexpr int ROWBA = WKA * 2, KCPRA = ROWBA / 16, SLOTA = 256 * ROWBA;
    static constexpr int ROWBB = WKB * 2, KCPRB = ROWBB / 16, SLOTB = 256 * ROWBB;
    static constexpr int B_REGION = NSA * SLOTA;          // B slots start here
    static constexpr int BYTES = B_REGION + NSB * SLOTB;  // 128 KiB
    static constexpr int NLA = SLOTA / 16 / WTHREADS, NLB = SLOTB / 16 / WTHREADS;
    static constexpr int RPLA = WTHREADS / KCPRA, RPLB = WTHREADS / KCPRB;
};
constexpr int WRING = WRing<0>::BYTES;
static_assert(WRing<1>::BYTES == WRING && WRing<2>::BYTES == WRING, "every ring shape uses the same LDS");

// Position of chunk c of row r in a reduction-contiguous stage: the rows of
// a 16-row group fall on distinct 16-byte bank groups for any one chunk.
template <int KCPR>
__device__ __forceinline__ int kswz(int r, int c)
{
    return KCPR == 8 ? c ^ ((r >> 1) & 7) : c ^ ((r >> 2) & 3);
}
// Per-lane part of the fragment address of chunk 2j + h of tile row r (the
// row base is a multiple of the row length, so chunk 2j + h is at
// (row base + kswz_base) ^ (j << 5)).
template <int KCPR>
__device__ __forceinline__ uint32_t kswz_base(int r32, int h)
{
    const int sw = KCPR == 8 ? (r32 >> 1) & 7 : (r32 >> 2) & 3;
    return (uint32_t)((h ^ sw) & 1) * 16u | (uint32_t)((sw & (KCPR - 2)) << 4);
}

// Both operands reduction-contiguous (4 x 2 wave grid, 64-deep stages): a
// 256-row tile keeps two 64 KiB slots, one stage in flight while one
// computes; a tile of at most 128 rows has 16 KiB A slots, so three 48 KiB
// slots fit and two stages are in flight (such a tile has half the MFMAs per
// stage, and its loads would otherwise wait).
template <int KIND, int RING, int WL>
constexpr bool kc_three_slots() { return KIND == kFwdKContig && RING == 0 && WL == 0; }
constexpr int KC3_SLOTA = 128 * WRing<0>::ROWBA;              // 16 KiB
constexpr int KC3_RING = 3 * (KC3_SLOTA + WRing<0>::SLOTB);     // 144 KiB

template <int KIND, int EPI, int RING, int WL>
constexpr int wide_lds_bytes()
{
    constexpr int ring = kc_three_slots<KIND, RING, WL>() ? KC3_RING : WRING;
    return ring > epi_lds_bytes<EPI, 4>() ? ring : epi_lds_bytes<EPI, 4>();
}

// One operand's loads of a tile: NL per thread per stage, all at one
// per-thread offset plus wave-uniform distances; stage kt starts kt * kstep
// bytes further on.  `chunk` (reduction-contiguous only) is the byte offset
// of the thread's chunk inside a stage row, for the partial last stage.
template <int NL>
struct WOp {
    const void *base;
    uint32_t bytes;
    uint32_t voff;
    uint32_t delta[NL];
    uint32_t kstep;
    int chunk;
};

// Issue one operand's loads of stage kt into LDS at `lds` (slot base).
// Branch-free: a stage past the end, and in a partial last stage a chunk of
// a reduction-contiguous row at or past the reduction length, get an offset
// past the bound; rows of a column-contiguous stage past the reduction
// length lie past the operand's bound already.
template <bool KCONTIG, int WK, int NL>
__device__ __forceinline__ void wissue(uint8_t *lds, const WOp<NL> &o, int kt, int nk, int Kred, int wave,
                                       bool once = false)
{
    bool ok = kt < nk;
    if (KCONTIG) ok = ok && kt * WK + o.chunk / 2 < Kred;
    const uint32_t v = ok ? o.voff + (uint32_t)kt * o.kstep : kOOB;
    uint8_t *d = lds + wave * kWave * 16;
    if (once) {
#pragma unroll
        for (int i = 0; i < NL; ++i) dma16_nt(o.base, o.bytes, d + i * WTHREADS * 16, v, o.delta[i]);
    } else {
#pragma unroll
        for (int i = 0; i < NL; ++i) dma16(o.base, o.bytes, d + i * WTHREADS * 16, v, o.delta[i]);
    }
}

__device__ __forceinline__ void wfrag_wait(bf16x8 (&a)[2], bf16x8 (&b)[4]) { frag_wait(a, b); }
__device__ __forceinline__ void wfrag_wait(bf16x8 (&a)[4], bf16x8 (&b)[2])
{
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]));
}
// Keep the MFMAs on these fragments after the preceding asm (the barrier and
// the reads of the next stage): an empty asm the fragments pass through.
__device__ __forceinline__ void wfrag_wait(bf16x8 (&a)[2], bf16x8 (&b)[2])
{
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]));
}
__device__ __forceinline__ void wfrag_wait(bf16x8 (&a)[1], bf16x8 (&b)[2])
{
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(b[0]), "+v"(b[1]));
}
__device__ __forceinline__ void wfrag_wait(bf16x8 (&a)[1], bf16x8 (&b)[4])
{
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}
__device__ __forceinline__ void wfrag_pin(bf16x8 (&a)[1], bf16x8 (&b)[4])
{
    asm volatile("" : "+v"(a[0]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}
__device__ __forceinline__ void wfrag_pin(bf16x8 (&a)[2], bf16x8 (&b)[2])
{
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]));
}
__device__ __forceinline__ void wfrag_pin(bf16x8 (&a)[1], bf16x8 (&b)[2])
{
    asm volatile("" : "+v"(a[0]), "+v"(b[0]), "+v"(b[1]));
}
__device__ __forceinline__ void wfrag_pin(bf16x8 (&a)[2], bf16x8 (&b)[4])
{
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}
__device__ __forceinline__ void wfrag_pin(bf16x8 (&a)[4], bf16x8 (&b)[2])
{
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]));
}

// Wave grids of the 256 x 256 tile: WL 0, 4 x 2 waves of 64 x 128 (2 x 4
// blocks of 32 x 32); WL 1, 2 x 4 waves of 128 x 64 (4 x 2 blocks).  WL 1
// reads half as many B fragments and twice as many A fragments per MFMA,
// which pays when B is the column-contiguous operand: its transposing reads
// stream from LDS at about two thirds the rate of ds_read_b128.  With
// SwiGLU, block q < NJ / 2 of a wave holds gate columns and block
// q + NJ / 2 the up columns of the same outputs.
template <int WL>
struct WGrid {
    static constexpr int MI = WL ? 4 : 2, NJ = WL ? 2 : 4;
    static constexpr int WM_SHIFT = WL ? 2 : 1;
};
// Tile column (B row of the tile) of block bj of wave wn.  The SwiGLU tile
// columns are 64-column groups gate j, up j, gate j + 64, up j + 64.
template <int WL, int EPI>
__device__ __forceinline__ int wgrid_bcol(int wn, int bj)
{
    if (WL == 0 || !epi_glu(EPI)) return wn * WGrid<WL>::NJ * 32 + bj * 32;
    return (wn >> 1) * 128 + (wn & 1) * 32 + bj * 64;
}

template <int KIND, int EPI, int RING, int WL>
__global__ __launch_bounds__(WTHREADS, 1) void gg_bf16_wide_kernel(Bf16Params p)
{
    using R = WRing<RING>;
    constexpr int MI = WGrid<WL>::MI, NJ = WGrid<WL>::NJ;
    static_assert(WL == 0 || KIND != kWgrad, "wgrad keeps the 4 x 2 wave grid");
    static_assert(RING != 2 || KIND == kFwdNContig, "the split ring is for a column-contiguous B with a reduction-contiguous A");
    constexpr int WKA = R::WKA, WKB = R::WKB, NSB = R::NSB;
    constexpr int SLOTA = R::SLOTA, SLOTB = R::SLOTB, B_REGION = R::B_REGION;
    constexpr int NLA = R::NLA, NLB = R::NLB;
    constexpr int LDS_BYTES = wide_lds_bytes<KIND, EPI, RING, WL>();
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    GroupTable tab;
    tab.G = p.G;
    int *tb = (int *)(smem + LDS_BYTES);
    tab.row0 = tb;
    tab.rows = tb + p.G;
    tab.tile0 = tb + 2 * p.G;
    int *s_scan = tab.tile0 + p.G + 1;
    int total;
    const TilesWgradSplit tw{p.tilesM * p.tilesN, p.accumulate, p.split_len};
    int *slot0 = (int *)(smem + LDS_BYTES + table_bytes(p.G));       // wgrad only
    if (KIND == kWgrad) {
        total = build_group_table<TilesWgradSplit, WTHREADS>(tab, p.lens, p.offs, p.G, p.M, tw, p.err, s_scan);
        if (p.split_len > 0) wgrad_slot_table<WTHREADS>(tab, tw, slot0, s_scan);
    } else {
        total = build_group_table<TilesFwd, WTHREADS>(tab, p.lens, p.offs, p.G, p.M, TilesFwd{WBM, p.tilesN}, p.err,
                                                      s_scan);
    }
    total = __builtin_amdgcn_readfirstlane(total);
    // the scan scratch is free once the table is built: it passes tile ids
    TileQueue tq;
    // the weight gradient hands out an expert's output tiles (of one token
    // chunk) as one queue chunk: they all run on one XCD, which then reads
    // that expert's activations and output gradient from HBM once, where
    // chunks of 32 tiles spread them over every XCD's L2 (measured -3 to -4%;
    // the MX weight gradient, whose experts hold thousands of tokens, lost
    // 3% that way and keeps chunks of 32)
    tq.init(p.sched, total, KIND == kWgrad ? max(kQueueChunk, p.tilesM * p.tilesN) : kQueueChunk);
    int *s_id = s_scan;
    int par = 0;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> WGrid<WL>::WM_SHIFT, wn = wave & ((1 << WGrid<WL>::WM_SHIFT) - 1);
    const uint32_t lds0 = lds_addr(smem);
    const int r32 = lane & 31, h = lane >> 5, g16 = (lane >> 4) & 1, s16 = lane & 15;

    // ---- per-lane B fragment bases (slot 0; other slots by immediate); the
    // A bases depend on the tile's height and are set per tile below.
    // reduction-contiguous: chunk 2j + h of the lane's first row at base ^ (j << 5)
    const uint32_t bK = lds0 + B_REGION + (uint32_t)(wgrid_bcol<WL, EPI>(wn, 0) + r32) * R::ROWBB + kswz_base<R::KCPRB>(r32, h);
    // column-contiguous: transposing reads of k-rows h*8 + s16/4 (+4), columns
    // 16 g16 + 4 (s16 & 3) of each 32-column block
    const int krow = h * 8 + (s16 >> 2);
    const int klo = 8 * (s16 & 1);
    uint32_t bN[NJ];
#pragma unroll
    for (int bj = 0; bj < NJ; ++bj) {
        const int col = wgrid_bcol<WL, EPI>(wn, bj) + 16 * g16 + 4 * (s16 & 3);
        bN[bj] = lds0 + B_REGION + krow * 512 + npos(krow, col >> 3) * 16 + klo;
    }
    // ---- per-thread load slots: reduction-contiguous row i*RPL + t/KCPR,
    // chunk kswz(row, t % KCPR); column-contiguous k-row i*16 + t/32, chunk
    // (t & 31) ^ (((t >> 5) & 3) << 2)
    const int ka_row = tid / R::KCPRA, ka_chunk = kswz<R::KCPRA>(ka_row, tid % R::KCPRA);
    const int kb_row = tid / R::KCPRB, kb_chunk = kswz<R::KCPRB>(kb_row, tid % R::KCPRB);
    const int nc_row = tid >> 5, nc_chunk = (tid & 31) ^ (((tid >> 5) & 3) << 2);

    for (int tile = tq.first(s_id); tile < total;) {
        const int g = __builtin_amdgcn_readfirstlane(find_group(tab, tile));
        const int local = tile - __builtin_amdgcn_readfirstlane(tab.tile0[g]);
        const int row0 = __builtin_amdgcn_readfirstlane(tab.row0[g]);
        const int rows = __builtin_amdgcn_readfirstlane(tab.rows[g]);
        int mt, nt;
        // the weight panel of an expert that fits one row block is read by
        // this tile alone
        bool b_once = false;
        // wgrad: the tile's token chunk (rows crow0 .. crow0 + crows of the expert)
        int chunk = 0, crow0 = 0, crows = rows;
        if (KIND == kWgrad) {
            const int ntl = p.tilesM * p.tilesN;
            chunk = local / ntl;
            const int rest = local - chunk * ntl;
            mt = rest / p.tilesN;
            nt = rest % p.tilesN;
            if (p.split_len > 0) {
                crow0 = chunk * p.split_len;
                crows = min(rows - crow0, p.split_len);
            }
        } else {
            const int tm = (rows + WBM - 1) / WBM;
            grouped_tile_order(local, tm, p.tilesN, mt, nt);
            b_once = tm == 1;
        }
        const int m0 = mt * WBM;
        const int Kred = (KIND == kWgrad) ? crows : p.Kred;
        const int nka = (Kred + WKA - 1) / WKA;     // A stages
        const int nk = (Kred + WKB - 1) / WKB;      // B stages: the steps of the k-loop

        // One tile of TMI 32-row blocks per wave (tile height TMI * 32 per
        // row of waves).  In the forward and data gradient a row block
        // holding at most 128 (or, on the 2 x 4 grid, 64) valid rows runs as
        // a tile of that height: A loads, A fragment reads and MFMAs then
        // scale with the valid rows while every wave keeps working.  The tile
        // ids, the B panel and the order of every accumulation are the same
        // for each height, so results do not depend on it.
        auto run_tile = [&](auto MIC) {
        constexpr int TMI = decltype(MIC)::value;
        constexpr int TBM = TMI * 32 * (WL ? 2 : 4);          // rows of this tile height
        constexpr int TNLA = KIND == kWgrad ? NLA : TBM / R::RPLA;
        static_assert(TMI <= MI && TNLA >= 1 && TNLA <= NLA, "tile height");
        // the ring of this tile height: three slots for a 128-row tile of
        // the reduction-contiguous kind, else the kind's own
        constexpr bool R3 = kc_three_slots<KIND, RING, WL>() && TMI == 1;
        constexpr int NS = R3 ? 3 : NSB;
        constexpr int SA = R3 ? KC3_SLOTA : SLOTA;           // A slot bytes
        constexpr int BR = R3 ? 3 * KC3_SLOTA : B_REGION;     // B slots start here
        static_assert(!R3 || (TNLA == 2 && BR + NS * SLOTB == KC3_RING && KC3_RING <= LDS_BYTES), "three-slot ring");
        // B fragment bases of the three-slot ring: slots 0 and 1 from one
        // base, slot 2 from a second 64 KiB on (a read's offset field holds
        // 16 bits); both derived per tile through a zero the compiler cannot
        // see through, so they are not kept live through the other paths
        uint32_t z3 = 0;
        if constexpr (R3) asm volatile("" : "+v"(z3));
        const uint32_t bK3 = bK - (uint32_t)(B_REGION - BR) + z3, bK3b = bK3 + 2u * SLOTB;
        const int wrow0 = wm * TMI * 32;
        // reduction-contiguous A: chunk 2j + h of the lane's first row at base ^ (j << 5)
        const uint32_t aK = lds0 + (uint32_t)(wrow0 + r32) * R::ROWBA + kswz_base<R::KCPRA>(r32, h);
        uint32_t aN[TMI];
#pragma unroll
        for (int bi = 0; bi < TMI; ++bi) {
            const int col = wrow0 + bi * 32 + 16 * g16 + 4 * (s16 & 3);
            aN[bi] = lds0 + krow * 512 + npos(krow, col >> 3) * 16 + klo;
        }
        int nvalid_bi = TMI;
        if (KIND != kWgrad) {
            const int vr = min(TBM, rows - m0) - wrow0;
            nvalid_bi = vr <= 0 ? 0 : min(TMI, (vr + 31) >> 5);
        }

        WOp<TNLA> oa;
        WOp<NLB> ob;
        if (KIND == kWgrad) {
            // [token][i] and [token][j] slices of the tile's token chunk: column-contiguous
            oa.base = p.a + (int64_t)(row0 + crow0) * p.lda;
            oa.bytes = (uint32_t)crows * p.lda * 2;
            oa.voff = (uint32_t)(nc_row * p.lda + min(m0 + nc_chunk * 8, p.Mout - 8)) * 2;
            ob.base = p.b + (int64_t)(row0 + crow0) * p.ldb;
            ob.bytes = (uint32_t)crows * p.ldb * 2;
            ob.voff = (uint32_t)(nc_row * p.ldb + min(nt * WBN + nc_chunk * 8, p.Nout - 8)) * 2;
#pragma unroll
            for (int i = 0; i < TNLA; ++i) oa.delta[i] = (uint32_t)(i * 16 * p.lda) * 2;
#pragma unroll
            for (int i = 0; i < NLB; ++i) ob.delta[i] = (uint32_t)(i * 16 * p.ldb) * 2;
            oa.kstep = (uint32_t)WKA * p.lda * 2;
            ob.kstep = (uint32_t)WKB * p.ldb * 2;
        } else {
            // A: the expert's rows, reduction-contiguous; rows past its end read zeros
            oa.base = p.a + (int64_t)row0 * p.lda;
            oa.bytes = (uint32_t)rows * p.lda * 2;
            oa.voff = (uint32_t)(m0 + ka_row) * p.lda * 2 + ka_chunk * 16;
#pragma unroll
            for (int i = 0; i < TNLA; ++i) oa.delta[i] = (uint32_t)(i * R::RPLA * p.lda) * 2;
            oa.kstep = WKA * 2;
            oa.chunk = ka_chunk * 16;
            const uint16_t *Bg = p.b + (int64_t)g * p.b_gstride;
            ob.base = Bg;
            if (KIND == kFwdKContig) {
                // tile rows i*RPL + t/KCPR: B rows col_of(i*RPL + t/KCPR); with
                // SwiGLU the 64-row groups are gate j, up I+j, gate j+64, up I+j+64
                ob.bytes = (uint32_t)p.Nout * p.ldb * 2;
                const int n0 = col_of<EPI>(nt, kb_row, p.Nout);
                ob.voff = (uint32_t)n0 * p.ldb * 2 + kb_chunk * 16;
#pragma unroll
                for (int i = 0; i < NLB; ++i)
                    ob.delta[i] =
                        (uint32_t)(col_of<EPI>(nt, i * R::RPLB, p.Nout) - col_of<EPI>(nt, 0, p.Nout)) * p.ldb * 2;
                ob.kstep = WKB * 2;
                ob.chunk = kb_chunk * 16;
            } else {
                ob.bytes = (uint32_t)p.Kred * p.ldb * 2;
                const int n = clamp8<EPI>(col_of<EPI>(nt, nc_chunk * 8, p.Nout), p.Nout);
                ob.voff = (uint32_t)(nc_row * p.ldb + n) * 2;
#pragma unroll
                for (int i = 0; i < NLB; ++i) ob.delta[i] = (uint32_t)(i * 16 * p.ldb) * 2;
                ob.kstep = (uint32_t)WKB * p.ldb * 2;
            }
        }

        // Accumulators start at zero, or for an accumulating wgrad at the
        // main_grad tile itself (loads overlap the operand prologue).
        // main_grad is read and written once, with the non-temporal policy,
        // so its stream leaves L2 first and the operand panels stay.
        floatx16 acc[TMI][NJ];
        if (KIND == kWgrad && p.accumulate && chunk == 0) {
            const float *og = (const float *)p.out + (int64_t)g * p.o_gstride;
#pragma unroll
            for (int bi = 0; bi < TMI; ++bi)
#pragma unroll
                for (int bj = 0; bj < NJ; ++bj) {
                    const int n = nt * WBN + wgrid_bcol<WL, EPI>(wn, bj) + (lane & 31);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = m0 + wrow0 + bi * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                        acc[bi][bj][r] = (n < p.Nout && i < p.Mout) ? __builtin_nontemporal_load(og + (int64_t)i * p.ldo + n) : 0.0f;
                    }
                }
        } else {
#pragma unroll
            for (int i = 0; i < TMI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        }

        auto issue_a = [&](int ka, int slot) {
            wissue<KIND != kWgrad, WKA>(smem + slot * SA, oa, ka, nka, Kred, wave);
        };
        auto issue_b = [&](int kb, int slot) {
            wissue<KIND == kFwdKContig, WKB>(smem + BR + slot * SLOTB, ob, kb, nk, Kred, wave, b_once);
        };
        // A fragments of k-step KS of A slot S; B fragments of k-step KS of B slot S
        auto rd_a = [&](auto KSC, auto SC, bf16x8 (&af)[TMI]) {
            constexpr int KS = decltype(KSC)::value, SO = decltype(SC)::value * SA;
            if constexpr (KIND == kWgrad) {
                constexpr int NO = SO + KS * 16 * 512, NJ = 4 * 512;  // k-step, +4 k-rows
                af[0] = join(ldsr_tr<NO>(aN[0]), ldsr_tr<NO + NJ>(aN[0]));
                af[1] = join(ldsr_tr<NO>(aN[1]), ldsr_tr<NO + NJ>(aN[1]));
            } else {
                const uint32_t x = aK ^ (uint32_t)(KS << 5);
                af[0] = ldsr_b128<SO>(x);
                if constexpr (TMI >= 2) af[1] = ldsr_b128<SO + 32 * R::ROWBA>(x);
                if constexpr (TMI == 4) {
                    af[2] = ldsr_b128<SO + 64 * R::ROWBA>(x);
                    af[3] = ldsr_b128<SO + 96 * R::ROWBA>(x);
                }
            }
        };
        auto rd_b = [&](auto KSC, auto SC, bf16x8 (&bf)[NJ]) {
            constexpr int KS = decltype(KSC)::value, SO = decltype(SC)::value * SLOTB;
            if constexpr (KIND == kFwdKContig) {
                constexpr int SL = decltype(SC)::value;
                constexpr int SOB = R3 ? (SL == 2 ? 0 : SL * SLOTB) : SO;
                const uint32_t x = (R3 ? (SL == 2 ? bK3b : bK3) : bK) ^ (uint32_t)(KS << 5);
                bf[0] = ldsr_b128<SOB + 0 * 32 * R::ROWBB>(x);
                bf[1] = ldsr_b128<SOB + 1 * 32 * R::ROWBB>(x);
                bf[2] = ldsr_b128<SOB + 2 * 32 * R::ROWBB>(x);
                bf[3] = ldsr_b128<SOB + 3 * 32 * R::ROWBB>(x);
            } else {
                constexpr int NO = SO + KS * 16 * 512, K4 = 4 * 512;
#pragma unroll
                for (int bj = 0; bj < NJ; ++bj) bf[bj] = join(ldsr_tr<NO>(bN[bj]), ldsr_tr<NO + K4>(bN[bj]));
            }
        };
        auto mma = [&](const bf16x8 (&af)[TMI], const bf16x8 (&bf)[NJ]) {
#pragma unroll
            for (int bi = 0; bi < TMI; ++bi)
                if (bi < nvalid_bi) {
#pragma unroll
                    for (int bj = 0; bj < NJ; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bi], bf[bj], acc[bi][bj], 0, 0, 0);
                }
        };
        bf16x8 fa[2][TMI], fb[2][NJ];
        int kt0 = 0;

        // prologue, and the id of the next tile (its atomic goes out first and
        // lands under the stages' loads)
        if (tid == 0) tq.issue();
        if constexpr (RING == 2) {
            issue_a(0, 0);
            issue_b(0, 0);
            issue_b(1, 1);
            issue_b(2, 2);
            wait_vmcnt<2 * NLB>();           // A stage 0 and B stage 0
        } else {
#pragma unroll
            for (int st = 0; st < NS - 1; ++st) {
                issue_a(st, st);
                issue_b(st, st);
            }
            wait_vmcnt<(NS - 2) * (TNLA + NLB)>();
        }
        if (tid == 0) s_id[par ^ 1] = tq.resolve(tile);
        wait_lgkm0();
        barrier();
        rd_a(IC<0>{}, IC<0>{}, fa[0]);
        rd_b(IC<0>{}, IC<0>{}, fb[0]);
        wfrag_wait(fa[0], fb[0]);

        // One step of the k-loop over B's stage kt = kt0 + P in B slot P.  The
        // MFMAs of the step's last k-step run after the closing barrier, on
        // fragments already in registers, while the first fragments of the
        // next stage are read: the barrier lines up all waves of a SIMD, and
        // an MFMA-free wait for those reads would idle the SIMD.  Past the
        // last stage the reads fetch unused bytes of the ring (no branch).
        auto stage = [&](auto PC) {
            constexpr int P = decltype(PC)::value;
            constexpr int Q = (P + 1) % NS;
            const int kt = kt0 + P;
            if constexpr (RING == 2) {
                // A stage kt/2 sits in A slot P/2, k-steps 2(P & 1) + 0, 1; on
                // even steps A's next stage goes out first, into the other slot
                constexpr int SA = P >> 1, JA = 2 * (P & 1);
                if constexpr ((P & 1) == 0) issue_a(kt / 2 + 1, SA ^ 1);
                issue_b(kt + 3, (P + 3) & 3);
                rd_a(IC<JA + 1>{}, IC<SA>{}, fa[1]);
                rd_b(IC<1>{}, PC, fb[1]);
                mma(fa[0], fb[0]);
                wfrag_wait(fa[1], fb[1]);
                // even: B's next stage landed; odd: A's next stage too
                if constexpr ((P & 1) == 0)
                    wait_vmcnt<2 * NLB + TNLA>();
                else
                    wait_vmcnt<2 * NLB>();
                barrier();
                constexpr int SA1 = Q >> 1, JA1 = 2 * (Q & 1);
                rd_a(IC<JA1>{}, IC<SA1>{}, fa[0]);
                rd_b(IC<0>{}, IC<Q>{}, fb[0]);
                wfrag_pin(fa[1], fb[1]);
                mma(fa[1], fb[1]);
                wfrag_wait(fa[0], fb[0]);
            } else {
                constexpr int PN = (P + NS - 1) % NS;
                issue_a(kt + NS - 1, PN);        // the slot stage kt-1 freed at its barrier
                issue_b(kt + NS - 1, PN);
                auto rd = [&](auto KSC, bf16x8 (&af)[TMI], bf16x8 (&bf)[NJ]) {
                    rd_a(KSC, PC, af);
                    rd_b(KSC, PC, bf);
                };
                if constexpr (WKB == 64) {
                    rd(IC<1>{}, fa[1], fb[1]);
                    mma(fa[0], fb[0]);
                    wfrag_wait(fa[1], fb[1]);
                    rd(IC<2>{}, fa[0], fb[0]);
                    mma(fa[1], fb[1]);
                    wfrag_wait(fa[0], fb[0]);
                    rd(IC<3>{}, fa[1], fb[1]);
                    mma(fa[0], fb[0]);
                    wfrag_wait(fa[1], fb[1]);
                } else {
                    rd(IC<1>{}, fa[1], fb[1]);
                    mma(fa[0], fb[0]);
                    wfrag_wait(fa[1], fb[1]);
                }
                // stage kt+1 landed for this wave (later stages may still be
                // in flight), after the barrier for all waves, and every wave
                // is done reading slot P
                wait_vmcnt<(NS - 2) * (TNLA + NLB)>();
                barrier();
                rd_a(IC<0>{}, IC<Q>{}, fa[0]);
                rd_b(IC<0>{}, IC<Q>{}, fb[0]);
                wfrag_pin(fa[1], fb[1]);
                mma(fa[1], fb[1]);
                wfrag_wait(fa[0], fb[0]);
            }
        };
        // whole rounds of slots, then the last steps: no early exit, so the
        // compiler sees no path between slots that skips a stage's loads
        if constexpr (NS == 2) {
            for (; kt0 + 2 <= nk; kt0 += 2) {
                stage(IC<0>{});
                stage(IC<1>{});
            }
            if (kt0 < nk) stage(IC<0>{});
        } else if constexpr (NS == 3) {
            for (; kt0 + 3 <= nk; kt0 += 3) {
                stage(IC<0>{});
                stage(IC<1>{});
                stage(IC<2>{});
            }
            if (kt0 < nk) stage(IC<0>{});
            if (kt0 + 1 < nk) stage(IC<1>{});
            // the loads of the stage past the end (zeros) may still be
            // landing in the ring, which the epilogue and the next tile reuse
            wait_vmcnt<0>();
            barrier();
        } else {
            for (; kt0 + 4 <= nk; kt0 += 4) {
                stage(IC<0>{});
                stage(IC<1>{});
                stage(IC<2>{});
                stage(IC<3>{});
            }
            if (kt0 < nk) stage(IC<0>{});
            if (kt0 + 1 < nk) stage(IC<1>{});
            if (kt0 + 2 < nk) stage(IC<2>{});
            // the loads of stages past the end (zeros) may still be landing in
            // the ring, which the epilogue and the next tile reuse
            wait_vmcnt<0>();
            barrier();
        }

        if constexpr (KIND == kWgrad) {
            // nothing outstanding here; saying so keeps the compiler from
            // waiting for every earlier store before each one
            wait_vmcnt<0>();
            // chunk 0: main_grad; chunk c >= 1: its partial slot (none past
            // the workspace's slots, which only malformed lengths reach)
            float *og = (float *)p.out + (int64_t)g * p.o_gstride;
            bool keep = true;
            if (chunk > 0) {
                const int slot = slot0[g] + chunk - 1;
                keep = slot < p.nslots;
                og = p.partials + (int64_t)slot * p.o_gstride;
            }
#pragma unroll
            for (int bi = 0; bi < TMI; ++bi)
#pragma unroll
                for (int bj = 0; bj < NJ; ++bj) {
                    const int n = nt * WBN + wgrid_bcol<WL, EPI>(wn, bj) + (lane & 31);
                    if (n >= p.Nout || !keep) continue;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = m0 + wrow0 + bi * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                        if (i < p.Mout) __builtin_nontemporal_store(acc[bi][bj][r], og + (int64_t)i * p.ldo + n);
                    }
                }
        } else {
            store_tile_lds_w<EPI, 4, TMI, NJ, TBM>(acc, smem, p.out, p.out_scale, p.ldo, p.Nout, row0, m0, rows, nt,
                                                  wrow0, wn, p.swiglu_limit, p.aux, p.ldaux, p.save, p.ldsave);
        }
        };  // run_tile
        if constexpr (KIND == kFwdNContig && WL == 1) {
            const int hb = rows - m0;        // valid rows of the row block
            if (hb <= 64) run_tile(IC<1>{});
            else if (hb <= 128) run_tile(IC<2>{});
            else run_tile(IC<MI>{});
        } else if constexpr (KIND == kFwdKContig && WL == 0) {
            if (rows - m0 <= 128) run_tile(IC<1>{});
            else run_tile(IC<MI>{});
        } else {
            run_tile(IC<MI>{});
        }
        barrier();
        tile = __builtin_amdgcn_readfirstlane(s_id[par ^ 1]);
        par ^= 1;
    }
}

template <int KIND, int EPI, int RING, int WL>
hipError_t launch_wide(const Bf16Params &p, hipStream_t s)
{
    const int lds = wide_lds_bytes<KIND, EPI, RING, WL>() + table_bytes(p.G) + (KIND == kWgrad ? 4 * p.G : 0);
    auto kern = gg_bf16_wide_kernel<KIND, EPI, RING, WL>;
    static LdsLimit lds_limit;
    hipError_t e = lds_limit.ensure((const void *)kern, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, WTHREADS, lds);
    if (e != hipSuccess) return e;
    int64_t tiles_max;
    if (KIND == kWgrad)
        tiles_max = ((int64_t)p.G + (p.split_len > 0 ? p.M / p.split_len : 0)) * p.tilesM * p.tilesN;
    else
        tiles_max = (p.M / WBM + p.G) * (int64_t)p.tilesN;
    const int64_t grid = persistent_grid(occ, tiles_max);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WTHREADS), lds, s, p);
    return hipGetLastError();
}

// Ring shape per kind: B's stages three ahead where B is column-contiguous
// (forward with [G,K,N] weights: the split ring, A keeping 64-deep stages of
// whole-line rows; wgrad, both operands column-contiguous: 32-deep stages in
// 4 slots).  With both operands reduction-contiguous, 32-deep stages would
// give them 64-byte rows (half lines; dgrad measured +18%), so those kinds
// keep 64-deep stages in 2 slots.
template <int KIND, int EPI>
hipError_t launch_wide_ring(const Bf16Params &p, hipStream_t s)
{
    return launch_wide<KIND, EPI, KIND == kFwdKContig ? 0 : KIND == kFwdNContig ? 2 : 1, KIND == kFwdNContig ? 1 : 0>(p, s);
}

// Second pass of the split weight gradient.  Every workgroup rebuilds the
// chunk table from the lengths, lists the experts cut into more than one
// chunk, then walks (expert, 1024-float block) pairs: main_grad += partial of
// chunk 1, then chunk 2, ..., each add one fp32 rounding, in chunk order.
__global__ __launch_bounds__(256) void wgrad_split_reduce_kernel(Bf16Params p)
{
    extern __shared__ __attribute__((aligned(16))) int sm_red[];
    GroupTable tab;
    tab.G = p.G;
    tab.row0 = sm_red;
    tab.rows = sm_red + p.G;
    tab.tile0 = sm_red + 2 * p.G;
    int *s_scan = tab.tile0 + p.G + 1;
    int *slot0 = sm_red + 3 * p.G + 1 + 8;
    int *list = slot0 + p.G;                // split experts, in order
    const TilesWgradSplit tw{1, p.accumulate, p.split_len};
    build_group_table<TilesWgradSplit, 256>(tab, p.lens, p.offs, p.G, p.M, tw, nullptr, s_scan);
    wgrad_slot_table<256>(tab, tw, slot0, s_scan);
    // compact list of the experts with more than one chunk
    const int per = (p.G + 255) / 256, g0 = (int)threadIdx.x * per;
    int v = 0;
    for (int i = 0; i < per; ++i)
        if (g0 + i < p.G && tw.chunks(tab.rows[g0 + i]) > 1) ++v;
    int nsplit;
    int pos = block_exclusive_scan<256>(v, s_scan, &nsplit);
    for (int i = 0; i < per; ++i)
        if (g0 + i < p.G && tw.chunks(tab.rows[g0 + i]) > 1) list[pos++] = g0 + i;
    __syncthreads();
    const int64_t P = (int64_t)p.Mout * p.Nout;        // floats per expert (a multiple of 4)
    const int64_t nblk = (P / 4 + 255) / 256;
    for (int64_t w = blockIdx.x; w < (int64_t)nsplit * nblk; w += gridDim.x) {
        const int g = list[w / nblk];
        const int64_t q = (w % nblk) * 256 + threadIdx.x;   // float4 index inside the expert
        if (q >= P / 4) continue;
        const int nch = tw.chunks(tab.rows[g]);
        floatx4 *mg = (floatx4 *)((float *)p.out + (int64_t)g * p.o_gstride) + q;
        floatx4 acc = __builtin_nontemporal_load(mg);
        for (int c = 1; c < nch; ++c) {
            const int slot = slot0[g] + c - 1;
            if (slot >= p.nslots) break;
            const floatx4 v4 = __builtin_nontemporal_load((const floatx4 *)(p.partials + (int64_t)slot * p.o_gstride) + q);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += v4[e];
        }
        __builtin_nontemporal_store(acc, mg);
    }
}

__global__ void queue_reset_kernel(uint32_t *sched)
{
    const int i = threadIdx.x;
    if (i < kQueues) __hip_atomic_store(sched + i * kQueueStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

int bf16_tile_m(int narrow) { return narrow ? BM : WBM; }
int bf16_tile_n() { return BN; }

hipError_t launch_wgrad_split_reduce(const Bf16Params &p, hipStream_t s)
{
    const int lds = 4 * (5 * p.G + 1 + 8);
    const int64_t P4 = (int64_t)p.Mout * p.Nout / 4;
    int64_t grid = (int64_t)device_cus() * 4;
    const int64_t most = ((P4 + 255) / 256) * (p.M / p.split_len);   // split experts <= M / split_len
    if (grid > most) grid = most;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(wgrad_split_reduce_kernel, dim3((unsigned)grid), dim3(256), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_queue_reset(uint32_t *sched, hipStream_t s)
{
    hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(kWave), 0, s, sched);
    return hipGetLastError();
}

hipError_t launch_bf16(const Bf16Params &p, int kind, int epi, hipStream_t s)
{
    // the SwiGLU backward epilogue and the SwiGLU that keeps its input exist
    // for the 256 x 256 kernel only
    if (epi == kEpiDSwiglu) {
        if (kind == kFwdKContig) return launch_wide_ring<kFwdKContig, kEpiDSwiglu>(p, s);
        if (kind == kFwdNContig) return launch_wide_ring<kFwdNContig, kEpiDSwiglu>(p, s);
        return hipErrorInvalidValue;
    }
    if (epi == kEpiSwigluSave) {
        if (kind == kFwdKContig) return launch_wide_ring<kFwdKContig, kEpiSwigluSave>(p, s);
        if (kind == kFwdNContig) return launch_wide_ring<kFwdNContig, kEpiSwigluSave>(p, s);
        return hipErrorInvalidValue;
    }
    // the 256 x 256 kernel, or the 128 x 256 one (bit-identical results)
    if (!p.narrow) {
        if (kind == kWgrad) return launch_wide_ring<kWgrad, kEpiNone>(p, s);
        if (kind == kFwdKContig) {
            if (epi == kEpiSwiglu) return launch_wide_ring<kFwdKContig, kEpiSwiglu>(p, s);
            if (epi == kEpiSwigluMxfp4) return launch_wide_ring<kFwdKContig, kEpiSwigluMxfp4>(p, s);
            return launch_wide_ring<kFwdKContig, kEpiNone>(p, s);
        }
        if (epi == kEpiSwiglu) return launch_wide_ring<kFwdNContig, kEpiSwiglu>(p, s);
        if (epi == kEpiSwigluMxfp4) return launch_wide_ring<kFwdNContig, kEpiSwigluMxfp4>(p, s);
        return launch_wide_ring<kFwdNContig, kEpiNone>(p, s);
    }
    if (kind == kWgrad) return launch_depth<kWgrad, kEpiNone>(p, s);
    if (kind == kFwdKContig) {
        if (epi == kEpiSwiglu) return launch_depth<kFwdKContig, kEpiSwiglu>(p, s);
        if (epi == kEpiSwigluMxfp4) return launch_depth<kFwdKContig, kEpiSwigluMxfp4>(p, s);
        return launch_depth<kFwdKContig, kEpiNone>(p, s);
    }
    if (epi == kEpiSwiglu) return launch_depth<kFwdNContig, kEpiSwiglu>(p, s);
    if (epi == kEpiSwigluMxfp4) return launch_depth<kFwdNContig, kEpiSwigluMxfp4>(p, s);
    return launch_depth<kFwdNContig, kEpiNone>(p, s);
}

}  // namespace ptgg
