// gemm_mx.hip -- OCP-MX grouped GEMM forward for gfx950 (MXFP8 E4M3 and
// MXFP4 E2M1 operands, one E8M0 scale per 32 values along K).
//
// Same persistent ragged-batch schedule, tile shape and LDS ring as the BF16
// kernel: both operands are K-contiguous (activations [M, K], weights
// [G, N, K], the [experts, out, in] layout), and every stage of the ring holds
// 64 code bytes of each of the tile's 128 A rows and 256 B rows (64 E4M3 or
// 128 E2M1 values), filled by direct buffer->LDS loads.  The products run on
// v_mfma_scale_f32_32x32x64_f8f6f4, which applies one E8M0 byte per lane to
// the 32 values of a block inside the matrix core, so the fp32 accumulator
// receives exactly scaled products.
//
// A stage's fragments are the same LDS bytes for both element widths: lane l
// of a wave reads the 16-byte chunks h and 2 + h (h = l >> 5) of its row.
//  - E2M1: each chunk is one 32-value block, and one MFMA per chunk consumes
//    it (two MFMA steps of 64 values per stage); lane half h supplies the
//    scale of block 2s + h of step s.
//  - E4M3: one MFMA consumes the whole stage.  Bytes 0-15 of every lane take
//    the scale supplied by lane half 0 and bytes 16-31 the one supplied by
//    lane half 1 (measured on gfx950), so lane half h holds values
//    16h..16h+15 of block 0 (chunk h) in bytes 0-15 and the same values of
//    block 1 (chunk 2 + h) in bytes 16-31, and supplies block h's scale.
//
// Scale bytes bypass LDS: every lane loads the bytes of its own rows for a
// stage into registers when the stage's operand loads are issued, three
// stages ahead, so the k-loop is unrolled by the ring depth to keep each
// slot's registers and LDS offsets static.  Stages past the end are still
// issued, with offsets past every bound (zeros, no memory traffic), so that
// every wait in the loop has the same count.
#include <stdlib.h>

#include "pipeline.hpp"

namespace ptgg {

namespace {

constexpr int NSTAGE = 3;
typedef unsigned int uintx8 __attribute__((ext_vector_type(8)));

// How a lane fetches its scale bytes for one stage.  Every load is one
// aligned 32-bit word; the bytes are extracted where they are used.  (Byte or
// 16-bit loads would leave narrow values in the loop-carried registers, and
// the masking copies the compiler then adds at the loop back-edge each wait
// for their load.)
enum ScaleMode {
    kScE4M3 = 0,      // the word holding byte 2*kt + h of the row
    kScE2M1Word = 1,  // K % 128 == 0: the word of bytes 4*kt .. 4*kt + 3
    kScE2M1Span = 2,  // any K: lane half h loads aligned word h of the two
                      // that cover bytes 4*kt .. 4*kt + 3; the halves swap
                      // words and realign them
};
template <int SCM>
struct Sc {
    static constexpr int regs = 6;                    // 2 A rows + 4 B rows per lane
    static constexpr int per_stage = LOADS + regs;    // vector-memory ops per stage
};

template <int V>
struct IC { static constexpr int value = V; };

__device__ __forceinline__ uint32_t ld_u32(const void *base, uint32_t bytes, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(base, bytes), voff, soff, 0);
}

// Scale rows of this lane for a tile: A rows bi = 0, 1 and B rows bj = 0..3,
// as byte offsets from the start of the scale tensors (both 4-byte aligned);
// the record bounds are the tensors' sizes rounded up to whole words, so an
// aligned word never reaches past the page of the tensor's last byte.
struct ScRows {
    const uint8_t *a;
    const uint8_t *b;
    uint32_t abytes, bbytes;
    uint32_t row[6];
    uint32_t astride, bstride;      // stage-major copies: bytes from one stage to the next
};

// E4M3: byte of the row that lane half h needs for stage kt.  The partial
// last stage (kt == nfull) holds block 0 only, and block 1's lanes take its
// byte: a finite scale for codes that are all zero.
__device__ __forceinline__ uint32_t e4m3_byte(int kt, int nfull, int h)
{
    return 2u * kt + ((kt == nfull) ? 0u : (uint32_t)h);
}

// Load this lane's scale words of stage kt (a dummy stage past the end reads
// zeros without touching memory).
template <int SCM>
__device__ __forceinline__ void load_scales(uint32_t (&sc)[6], const ScRows &sr, int kt, int nk, int nfull, int h)
{
    const uint32_t soff = kt >= nk ? kOOB : 0u;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const uint8_t *base = i < 2 ? sr.a : sr.b;
        const uint32_t bytes = i < 2 ? sr.abytes : sr.bbytes;
        uint32_t a;
        if constexpr (SCM == kScE4M3) a = (sr.row[i] + e4m3_byte(kt, nfull, h)) & ~3u;
        else if constexpr (SCM == kScE2M1Word) a = sr.row[i] + 4u * kt;
        else a = ((sr.row[i] + 4u * kt) & ~3u) + 4u * h;
        sc[i] = ld_u32(base, bytes, a, soff);
    }
}

// Per-stage scale words: E4M3 the lane's byte at bits 0-7; E2M1 the row's
// four bytes of the stage in order, those of missing blocks in a partial
// last stage cleared (a finite scale for codes that are all zero).
template <int SCM>
__device__ __forceinline__ void scale_words(const uint32_t (&sc)[6], uint32_t (&w)[6], const ScRows &sr, int kt,
                                            int nfull, int nb_last, int h)
{
    const uint32_t keep = (kt == nfull) ? (1u << (8 * nb_last)) - 1u : 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        if constexpr (SCM == kScE4M3) {
            w[i] = __builtin_amdgcn_ubfe(sc[i], ((sr.row[i] + e4m3_byte(kt, nfull, h)) & 3u) * 8u, 8u);
        } else if constexpr (SCM == kScE2M1Word) {
            w[i] = sc[i];
        } else {
            const auto r = __builtin_amdgcn_permlane32_swap(sc[i], sc[i], false, false);
            w[i] = __builtin_amdgcn_alignbyte(r[1], r[0], (sr.row[i] + 4u * kt) & 3u) & keep;
        }
    }
}

// Scale operand of row slot i (A rows 0-1, B rows 2-5) for MFMA step s.
template <int SCM>
__device__ __forceinline__ int scale_of(const uint32_t (&w)[6], int i, int s, uint32_t sh)
{
    if constexpr (SCM == kScE4M3) return (int)w[i];
    else return (int)__builtin_amdgcn_ubfe(w[i], sh + 16u * s, 8u);
}

// Direct-load state of one tile.  Slot i * 256 + t of a stage (thread t,
// load i) holds chunk c = (t & 3) ^ ((t >> 4) & 3) of tile row i * 64 + t / 4,
// so a thread's loads share one chunk and one 32-bit offset per operand; the
// rows of loads 1.. sit at wave-uniform distances from load 0's, passed as
// scalar offsets.
struct Ops {
    const uint8_t *a;
    const uint8_t *b;
    uint32_t abytes, bbytes;
    uint32_t avoff, bvoff;          // load 0 of this thread, chunk included
    uint32_t adelta;                // A rows of load 1: + 64 rows
    uint32_t bdelta[B_LOADS];       // B rows of loads 0..3
    uint32_t chunk;                 // byte offset of the chunk inside a stage row
};

// Issue the operand loads of stage kt into LDS byte offset st.  Branch-free,
// so that every path issues the same loads and the compiler's own waits for
// the scale registers see the true number of loads in flight: in a partial
// last stage a thread whose chunk lies at or past the row length, and every
// thread of a stage past the end, gets an offset past the bound.
__device__ __forceinline__ void issue_stage(uint8_t *smem, const Ops &o, uint32_t st, int kt, int nk, int Kb,
                                            int wave)
{
    const int k0 = kt * ROW_BYTES;
    const int room = kt < nk ? Kb - k0 : 0;              // bytes left in each row from k0
    const bool ok = (int)o.chunk < room;
    const uint32_t va = ok ? o.avoff + k0 : kOOB, vb = ok ? o.bvoff + k0 : kOOB;
    uint8_t *lds = smem + st + wave * kWave * 16;
    dma16(o.a, o.abytes, lds, va, 0u);
    dma16(o.a, o.abytes, lds + kThreads * 16, va, o.adelta);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) dma16(o.b, o.bbytes, lds + A_BYTES + i * kThreads * 16, vb, o.bdelta[i]);
}

__device__ __forceinline__ intx8 cat8(uintx4 lo, uintx4 hi)
{
    return __builtin_bit_cast(intx8, uintx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}
__device__ __forceinline__ intx8 pad8(uintx4 lo) { return cat8(lo, uintx4{0u, 0u, 0u, 0u}); }

// Wait for all issued LDS reads; the fragments pass through the asm so no
// use of them can be scheduled before the wait.
__device__ __forceinline__ void frag_wait(uintx4 (&a)[2], uintx4 (&b)[4])
{
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}
__device__ __forceinline__ void frag_wait(uintx4 (&a)[2][2], uintx4 (&b)[2][4], int j0)
{
    if (j0 == 0)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[1][0]), "+v"(a[1][1]), "+v"(b[0][0]), "+v"(b[0][1]),
                       "+v"(b[1][0]), "+v"(b[1][1]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(b[0][2]), "+v"(b[0][3]), "+v"(b[1][2]), "+v"(b[1][3]));
}

// ------------------------------------------------------------------ kernel
// FMT 0: E4M3 (64 values per row per stage); FMT 1: E2M1 (128 values).
template <int FMT, int EPI, int SCM>
__global__ __launch_bounds__(kThreads, 2) void gg_mx_kernel(MxParams p)
{
    static_assert(NSTAGE == 3, "the k-loop below is unrolled for three slots");
    constexpr int GEMM_LDS_BYTES = NSTAGE * STAGE_BYTES;
    constexpr int MF = FMT == 0 ? 0 : 4;                  // operand format code of the scaled MFMA
    constexpr int RB = 32 * ROW_BYTES;                    // LDS bytes of 32 rows
    using S = Sc<SCM>;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    GroupTable tab;
    tab.G = p.G;
    int *tb = (int *)(smem + GEMM_LDS_BYTES);
    tab.row0 = tb;
    tab.rows = tb + p.G;
    tab.tile0 = tb + 2 * p.G;
    int *s_scan = tab.tile0 + p.G + 1;
    int total = build_group_table(tab, p.lens, p.offs, p.G, p.M, TilesFwd{BM, p.tilesN}, p.err, s_scan);
    total = __builtin_amdgcn_readfirstlane(total);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t lds0 = lds_addr(smem);
    const int r32 = lane & 31, h = lane >> 5;
    const uint32_t sh = 8u * h;

    const int Kb = FMT == 0 ? p.K : p.K / 2;              // code bytes per row
    const int KS = p.K / 32;                               // scale bytes per row
    const int nk = (Kb + ROW_BYTES - 1) / ROW_BYTES, nfull = Kb / ROW_BYTES;
    const int nb_last = (Kb - nfull * ROW_BYTES) / 16;     // blocks of the partial stage (E2M1)

    // per-lane LDS read bases: chunks h and 2 + h of the lane's first A / B row
    uint32_t aK[2], bK[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ra = wm * 64 + r32, rb = wn * 128 + r32;
        aK[c] = lds0 + ra * ROW_BYTES + kpos(ra, 2 * c + h) * 16;
        bK[c] = lds0 + A_BYTES + rb * ROW_BYTES + kpos(rb, 2 * c + h) * 16;
    }

    for (int tile = xcd_logical_id(); tile < total; tile += gridDim.x) {
        const int g = __builtin_amdgcn_readfirstlane(find_group(tab, tile));
        const int local = tile - __builtin_amdgcn_readfirstlane(tab.tile0[g]);
        const int row0 = __builtin_amdgcn_readfirstlane(tab.row0[g]);
        const int rows = __builtin_amdgcn_readfirstlane(tab.rows[g]);
        const int tm = (rows + BM - 1) / BM;
        const int nt = local / tm, mt = local % tm;
        const int m0 = mt * BM;
        const int vr = min(BM, rows - m0) - wm * 64;
        const int nvalid_bi = vr <= 0 ? 0 : (vr > 32 ? 2 : 1);

        // ---- operand buffers and per-thread offsets for this tile.  A rows
        // past the expert's end and B rows past N fall outside the record
        // bounds and read zeros; with SwiGLU, gate rows past N/2 read up rows
        // whose outputs are never stored.
        Ops o;
        o.a = p.a + (int64_t)row0 * Kb;
        o.abytes = (uint32_t)rows * Kb;
        o.b = p.b + (int64_t)g * p.N * Kb;
        o.bbytes = (uint32_t)p.N * Kb;
        o.chunk = (uint32_t)(((tid & 3) ^ ((tid >> 4) & 3)) * 16);
        o.avoff = (uint32_t)(m0 + (tid >> 2)) * Kb + o.chunk;
        o.adelta = 64u * Kb;
        if (EPI == kEpiNone) {
            o.bvoff = (uint32_t)(nt * BN + (tid >> 2)) * Kb + o.chunk;
#pragma unroll
            for (int i = 0; i < B_LOADS; ++i) o.bdelta[i] = (uint32_t)(i * 64) * Kb;
        } else {
            // tile rows 0-63 / 64-127 / 128-191 / 192-255: gate j, up I + j,
            // gate j + 64, up I + j + 64, with j = nt * 128 + row % 64
            const int I = p.N >> 1;
            o.bvoff = (uint32_t)(nt * (BN / 2) + (tid >> 2)) * Kb + o.chunk;
            o.bdelta[0] = 0u;
            o.bdelta[1] = (uint32_t)I * Kb;
            o.bdelta[2] = 64u * Kb;
            o.bdelta[3] = (uint32_t)(I + 64) * Kb;
        }
        ScRows sr;
        sr.a = p.as;
        sr.abytes = (uint32_t)((p.M * KS + 3) & ~3ll);
        sr.b = p.bs;
        sr.bbytes = (uint32_t)(((int64_t)p.G * p.N * KS + 3) & ~3ll);
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
            sr.row[bi] = (uint32_t)((row0 + min(m0 + wm * 64 + bi * 32 + r32, rows - 1)) * KS);
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
            sr.row[2 + bj] =
                (uint32_t)((g * p.N + clamp1<EPI>(col_of<EPI>(nt, wn * 128 + bj * 32 + r32, p.N), p.N)) * KS);

        floatx16 acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        // The explicit waits below count a stage's loads (operands, then
        // scales) as one group in program order; a compiler fence after each
        // group keeps the scheduler from moving loads of different stages
        // past one another.
        uint32_t sc[NSTAGE][S::regs];
        // prologue: stages 0 .. NSTAGE-1 (dummies past the end)
        issue_stage(smem, o, 0 * STAGE_BYTES, 0, nk, Kb, wave);
        load_scales<SCM>(sc[0], sr, 0, nk, nfull, h);
        asm volatile("" ::: "memory");
        issue_stage(smem, o, 1 * STAGE_BYTES, 1, nk, Kb, wave);
        load_scales<SCM>(sc[1], sr, 1, nk, nfull, h);
        asm volatile("" ::: "memory");
        issue_stage(smem, o, 2 * STAGE_BYTES, 2, nk, Kb, wave);
        load_scales<SCM>(sc[2], sr, 2, nk, nfull, h);
        asm volatile("" ::: "memory");
        wait_vmcnt<(NSTAGE - 1) * S::per_stage>();
        barrier();

        // Fragments: fa[c][bi] / fb[c][bj] hold chunk (c == 0 ? h : 2 + h) of
        // the lane's rows.  E2M1 runs one MFMA step per chunk; E4M3 one MFMA
        // over both chunks, split by B blocks (0-1, then 2-3).  Registers are
        // refilled as soon as the last MFMA reading them has been issued.
        uintx4 fa[2][2], fb[2][4];
        if constexpr (FMT == 1) {
            fa[0][0] = ldsr_u128<0>(aK[0]);
            fa[0][1] = ldsr_u128<RB>(aK[0]);
            fb[0][0] = ldsr_u128<0 * RB>(bK[0]);
            fb[0][1] = ldsr_u128<1 * RB>(bK[0]);
            fb[0][2] = ldsr_u128<2 * RB>(bK[0]);
            fb[0][3] = ldsr_u128<3 * RB>(bK[0]);
            frag_wait(fa[0], fb[0]);
        } else {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                fa[c][0] = ldsr_u128<0>(aK[c]);
                fa[c][1] = ldsr_u128<RB>(aK[c]);
                fb[c][0] = ldsr_u128<0>(bK[c]);
                fb[c][1] = ldsr_u128<RB>(bK[c]);
            }
            frag_wait(fa, fb, 0);
        }

        auto mfma = [&](int bi, int bj, intx8 a, intx8 b, const uint32_t (&w)[S::regs], int s) {
            acc[bi][bj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                a, b, acc[bi][bj], MF, MF, 0, scale_of<SCM>(w, bi, s, sh), 0, scale_of<SCM>(w, 2 + bj, s, sh));
        };

        int kt0 = 0;
        auto step = [&](auto PC) {
            constexpr int P = decltype(PC)::value;          // ring slot of stage kt
            constexpr int SO = P * STAGE_BYTES, SN = ((P + 1) % NSTAGE) * STAGE_BYTES;
            const int kt = kt0 + P;
            uint32_t w[S::regs];
            scale_words<SCM>(sc[P], w, sr, kt, nfull, nb_last, h);
            if constexpr (FMT == 1) {
                // read chunk 2 + h of stage kt | MFMA step 0
                uintx4 ga[2], gb[4];
                ga[0] = ldsr_u128<SO>(aK[1]);
                ga[1] = ldsr_u128<SO + RB>(aK[1]);
                gb[0] = ldsr_u128<SO + 0 * RB>(bK[1]);
                gb[1] = ldsr_u128<SO + 1 * RB>(bK[1]);
                gb[2] = ldsr_u128<SO + 2 * RB>(bK[1]);
                gb[3] = ldsr_u128<SO + 3 * RB>(bK[1]);
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
                    if (bi < nvalid_bi) {
#pragma unroll
                        for (int bj = 0; bj < 4; ++bj) mfma(bi, bj, pad8(fa[0][bi]), pad8(fb[0][bj]), w, 0);
                    }
                // stage kt+1 landed and every wave is done with slot P
                wait_vmcnt<(NSTAGE - 2) * S::per_stage>();
                frag_wait(ga, gb);
                barrier();
                issue_stage(smem, o, SO, kt + NSTAGE, nk, Kb, wave);
                // read chunk h of stage kt+1 | MFMA step 1
                fa[0][0] = ldsr_u128<SN>(aK[0]);
                fa[0][1] = ldsr_u128<SN + RB>(aK[0]);
                fb[0][0] = ldsr_u128<SN + 0 * RB>(bK[0]);
                fb[0][1] = ldsr_u128<SN + 1 * RB>(bK[0]);
                fb[0][2] = ldsr_u128<SN + 2 * RB>(bK[0]);
                fb[0][3] = ldsr_u128<SN + 3 * RB>(bK[0]);
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
                    if (bi < nvalid_bi) {
#pragma unroll
                        for (int bj = 0; bj < 4; ++bj) mfma(bi, bj, pad8(ga[bi]), pad8(gb[bj]), w, 1);
                    }
                load_scales<SCM>(sc[P], sr, kt + NSTAGE, nk, nfull, h);
                asm volatile("" ::: "memory");
                frag_wait(fa[0], fb[0]);
            } else {
                // read B blocks 2-3 of stage kt | MFMA on B blocks 0-1
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    fb[c][2] = ldsr_u128<SO + 2 * RB>(bK[c]);
                    fb[c][3] = ldsr_u128<SO + 3 * RB>(bK[c]);
                }
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
                    if (bi < nvalid_bi) {
#pragma unroll
                        for (int bj = 0; bj < 2; ++bj)
                            mfma(bi, bj, cat8(fa[0][bi], fa[1][bi]), cat8(fb[0][bj], fb[1][bj]), w, 0);
                    }
                wait_vmcnt<(NSTAGE - 2) * S::per_stage>();
                frag_wait(fa, fb, 2);
                barrier();
                issue_stage(smem, o, SO, kt + NSTAGE, nk, Kb, wave);
                // read B blocks 0-1 of stage kt+1 | MFMA on B blocks 2-3 | read A of stage kt+1
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    fb[c][0] = ldsr_u128<SN>(bK[c]);
                    fb[c][1] = ldsr_u128<SN + RB>(bK[c]);
                }
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
                    if (bi < nvalid_bi) {
#pragma unroll
                        for (int bj = 2; bj < 4; ++bj)
                            mfma(bi, bj, cat8(fa[0][bi], fa[1][bi]), cat8(fb[0][bj], fb[1][bj]), w, 0);
                    }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    fa[c][0] = ldsr_u128<SN>(aK[c]);
                    fa[c][1] = ldsr_u128<SN + RB>(aK[c]);
                }
                load_scales<SCM>(sc[P], sr, kt + NSTAGE, nk, nfull, h);
                asm volatile("" ::: "memory");
                frag_wait(fa, fb, 0);
            }
        };
        // Whole rounds of the three slots, then the last one or two stages.
        // The loop has no early exit: the compiler's own waits for the scale
        // registers assume every path it can see, and an exit taken between
        // slots would show it a way back to the loop head past the other
        // slots' loads.
        for (; kt0 + NSTAGE <= nk; kt0 += NSTAGE) {
            step(IC<0>{});
            step(IC<1>{});
            step(IC<2>{});
        }
        if (kt0 < nk) {
            step(IC<0>{});
            if (kt0 + 1 < nk) step(IC<1>{});
        }
        // drain the dummy stages still in flight before the slots are reused
        wait_vmcnt<0>();
        barrier();
        store_out<EPI>(acc, p.out, p.out_scale, p.ldo, p.N, row0, m0, rows, nt, wm, wn, p.swiglu_limit);
    }
}

// ====================================================================== wide
// The main MX kernel: one workgroup of 8 waves per CU (still two waves per
// SIMD), 256 x 256 tiles (wave (wm, wn), wm = 0..3, owns 64 x 128 outputs as
// before) and 128 code bytes of every operand row per stage, so that each
// direct load fetches whole 128-byte lines (64-byte half lines stream from
// L2 at roughly half the rate) and a tile moves a third fewer operand bytes
// per product than 128 x 256.  Two 64 KiB ring slots: the loads of stage
// kt+1 go out at the start of stage kt and land while it computes.
//
// LDS rows are 128 bytes, chunk c (16 bytes) of row r at position
// c ^ ((r >> 1) & 7).  ds_read_b128 serves 16 lanes per pass, and the same
// chunk of 16 consecutive rows then covers all 64 banks (with c ^ (r & 7),
// rows r and r + 8 collided: a 2-way conflict on every read, measured as
// 46% of the LDS's busy cycles).  A lane reads chunks 2j + h of its rows;
// with the row's base 128-byte aligned, the address of chunk 2j + h is
// base ^ (j << 5) for a per-lane base that folds in h and (r >> 1) & 7.
//
// Per stage a row holds 4 scale blocks (E4M3) or 8 (E2M1, K % 256 == 0).
constexpr int WBM = 256, WBN = 256, WROW = 128, WTHREADS = 512;
constexpr int WA_BYTES = WBM * WROW;                   // 32 KiB
constexpr int WSTAGE = WA_BYTES + WBN * WROW;          // 64 KiB
constexpr int W_LOADS = WA_BYTES / 16 / WTHREADS;      // per operand per thread per stage (4)

enum WideScale {
    kWE4M3Word = 0,   // E4M3, K % 128 == 0: the word of bytes 4kt .. 4kt+3
    kWE4M3Span = 1,   // E4M3, other K: two words exchanged between lane halves
    kWE2M1Pair = 2,   // E2M1, K % 256 == 0: words 8kt and 8kt+4, one per lane half, exchanged
    kWE4M3Swz = 3,    // E4M3, stage-major copy: the stage's word of the row (any K)
    kWE2M1Swz = 4,    // E2M1, stage-major copy: the lane half's word of the row (any K)
    kWConst = 5,      // E4M3 with one fp32 scale per operand tensor: block scales all 1 (byte 127)
    kWConstRow = 6,   // the same with one fp32 scale per row of A and per row of B (output column)
};

// Load this lane's scale word of each of its rows for stage kt: NA A rows
// (a 128-row tile uses one) and the 4 B rows.  Only rows the MFMAs read are
// loaded: the k-loop waits on exact counts of its vector-memory operations,
// and a load whose result is never used would be dropped by the compiler,
// leaving one operation fewer in flight than counted (the wait for a stage
// would then let that stage's last direct load still be landing).
template <int WSC, int NA = 2>
__device__ __forceinline__ void wload_scales(uint32_t (&sc)[6], const ScRows &sr, int kt, int nk, int h)
{
    if constexpr (WSC == kWConst || WSC == kWConstRow) {
#pragma unroll
        for (int i = 0; i < 6; ++i) sc[i] = 0x7F7F7F7Fu;
        return;
    }
    const uint32_t soff = kt >= nk ? kOOB : 0u;
    if constexpr (NA < 2) sc[1] = 0u;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        if (i == 1 && NA < 2) continue;
        const uint8_t *base = i < 2 ? sr.a : sr.b;
        const uint32_t bytes = i < 2 ? sr.abytes : sr.bbytes;
        uint32_t a;
        if constexpr (WSC == kWE4M3Word) a = sr.row[i] + 4u * kt;
        else if constexpr (WSC == kWE4M3Span) a = ((sr.row[i] + 4u * kt) & ~3u) + 4u * h;
        else if constexpr (WSC == kWE2M1Pair) a = sr.row[i] + 8u * kt + 4u * h;
        else a = sr.row[i] + (uint32_t)kt * (i < 2 ? sr.astride : sr.bstride);
        sc[i] = ld_u32(base, bytes, a, soff);
    }
}

// Stage scale words, one per row: E4M3 the row's 4 bytes of the stage in
// order (missing blocks of a partial last stage cleared), so step s of lane
// half h takes byte 2s + h; E2M1 the 4 bytes this lane half uses, in step
// order (bytes h, 2 + h, 4 + h, 6 + h of the row's 8, picked by v_perm_b32).
template <int WSC>
__device__ __forceinline__ void wscale_words(const uint32_t (&sc)[6], uint32_t (&w)[6], const ScRows &sr, int kt,
                                             int nfull, int nb_last, int h)
{
    const uint32_t keep = (kt == nfull) ? (1u << (8 * nb_last)) - 1u : 0xFFFFFFFFu;
    const uint32_t sel = h ? 0x07050301u : 0x06040200u;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        if constexpr (WSC == kWE4M3Word || WSC == kWE4M3Swz || WSC == kWE2M1Swz || WSC == kWConst ||
                      WSC == kWConstRow) {
            w[i] = sc[i];
        } else if constexpr (WSC == kWE4M3Span) {
            const auto r = __builtin_amdgcn_permlane32_swap(sc[i], sc[i], false, false);
            w[i] = __builtin_amdgcn_alignbyte(r[1], r[0], (sr.row[i] + 4u * kt) & 3u) & keep;
        } else {
            const auto r = __builtin_amdgcn_permlane32_swap(sc[i], sc[i], false, false);
            w[i] = __builtin_amdgcn_perm(r[1], r[0], sel);
        }
    }
}

// Scale operand of row slot i for MFMA step s of a stage.
template <int WSC>
__device__ __forceinline__ int wscale_of(const uint32_t (&w)[6], int i, int s, uint32_t sh)
{
    if constexpr (WSC == kWConst || WSC == kWConstRow) return 127;
    if constexpr (WSC == kWE2M1Pair || WSC == kWE2M1Swz) return (int)__builtin_amdgcn_ubfe(w[i], 8u * s, 8u);
    else return (int)__builtin_amdgcn_ubfe(w[i], sh + 16u * s, 8u);
}

struct WOps {
    const uint8_t *a;
    const uint8_t *b;
    uint32_t abytes, bbytes;
    uint32_t avoff, bvoff;          // load 0 of this thread, chunk included
    uint32_t adelta[W_LOADS];       // row distances of loads 0..3 (bytes)
    uint32_t bdelta[W_LOADS];
    uint32_t chunk;
    bool b_once;                    // weights read by this tile alone: non-temporal
};

// Issue the operand loads of stage kt into the ring slot at LDS byte st: NA
// A loads per thread (the tile's rows), then the B loads at st + boff
// (branch-free: a thread whose chunk lies past the row length in a partial
// last stage, and every thread of a stage past the end, gets an offset past
// the bound).
template <int NA>
__device__ __forceinline__ void wissue_stage(uint8_t *smem, const WOps &o, uint32_t st, int kt, int nk, int Kb,
                                             int wave, uint32_t boff)
{
    const int k0 = kt * WROW;
    const int room = kt < nk ? Kb - k0 : 0;
    const bool ok = (int)o.chunk < room;
    const uint32_t va = ok ? o.avoff + k0 : kOOB, vb = ok ? o.bvoff + k0 : kOOB;
    uint8_t *lds = smem + st + wave * kWave * 16;
#pragma unroll
    for (int i = 0; i < NA; ++i) dma16(o.a, o.abytes, lds + i * WTHREADS * 16, va, o.adelta[i]);
    if (o.b_once) {
#pragma unroll
        for (int i = 0; i < W_LOADS; ++i) dma16_nt(o.b, o.bbytes, lds + boff + i * WTHREADS * 16, vb, o.bdelta[i]);
    } else {
#pragma unroll
        for (int i = 0; i < W_LOADS; ++i) dma16(o.b, o.bbytes, lds + boff + i * WTHREADS * 16, vb, o.bdelta[i]);
    }
}

// 16-byte LDS read at a run-time address plus immediate OFF (bi / bj rows).
template <int OFF>
__device__ __forceinline__ uintx4 wld(uint32_t addr)
{
    return ldsr_u128<OFF>(addr);
}

// 4-byte LDS read (inline asm, for the same reason as the fragment reads)
__device__ __forceinline__ uint32_t wld32(uint32_t addr)
{
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

// The ring per tile height: a 256-row tile keeps two 64 KiB slots (one
// stage in flight while one computes); a tile of at most 128 rows has 16 KiB
// A slots, so three 48 KiB slots fit and two stages are in flight -- such a
// tile has half the MFMAs per stage, and its loads would otherwise wait.
constexpr int MX_RING = 3 * (128 * WROW + WBN * WROW);
// LDS row pitch of the weight gradient's fp32 epilogue rows: 256 values and
// 32 bytes, so rows 4 apart (the two lane halves of a store) are 32 banks apart
constexpr int WG_RP = WBN * 4 + 32;
// 256-row tiles with stage-major scale copies: each ring slot's scale words
// (A's 256 rows, then B's, 4 bytes per row for E4M3 and 8 for E2M1) come in
// by direct loads with the stage, into this area after the two slots
constexpr int WSC_LDS = 2 * WSTAGE;
constexpr int WSC_SLOT = 2 * 256 * 8;                   // 4 KiB
static_assert(WSC_LDS + 2 * WSC_SLOT <= MX_RING, "scale slots fit beside the ring");
static_assert(MX_RING >= 2 * WSTAGE, "ring sizes");

// LDS of the ring or of the epilogue tile, whichever is larger; the group
// table follows it.
template <int EPI>
constexpr int wide_lds_bytes()
{
    // the weight gradient: 256-row tiles only; its epilogue stages half a
    // tile of fp32 rows (WG_RP bytes apart)
    if constexpr (EPI == kEpiWgrad) return WSC_LDS + 2 * WSC_SLOT > 128 * WG_RP ? WSC_LDS + 2 * WSC_SLOT : 128 * WG_RP;
    return MX_RING > epi_lds_bytes<EPI, 4>() ? MX_RING : epi_lds_bytes<EPI, 4>();
}

template <int FMT, int EPI, int WSC>
__global__ __launch_bounds__(WTHREADS, 1) void gg_mx_wide_kernel(MxParams p)
{
    constexpr int GEMM_LDS_BYTES = wide_lds_bytes<EPI>();
    constexpr int MF = FMT == 0 ? 0 : 4;
    constexpr int RB = 32 * WROW;                           // LDS bytes of 32 rows (bi / bj step)
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    GroupTable tab;
    tab.G = p.G;
    int *tb = (int *)(smem + GEMM_LDS_BYTES);
    tab.row0 = tb;
    tab.rows = tb + p.G;
    tab.tile0 = tb + 2 * p.G;
    int *s_scan = tab.tile0 + p.G + 1;
    // kEpiWgrad: the weight gradient, whose rows are the first gradient's
    // channels and whose reduction runs over each expert's (padded) tokens
    constexpr bool WG = EPI == kEpiWgrad;
    int total;
    const TilesWgradSplit tw{p.tilesM * p.tilesN, p.accumulate, p.split_len};
    int *slot0 = (int *)(smem + GEMM_LDS_BYTES + table_bytes(p.G));   // weight gradient, split
    if constexpr (WG) {
        total = build_group_table<TilesWgradSplit, WTHREADS>(tab, p.lens, p.offs, p.G, p.M, tw, p.err, s_scan);
        if (p.split_len > 0) wgrad_slot_table<WTHREADS>(tab, tw, slot0, s_scan);
    } else
        total = build_group_table<TilesFwd, WTHREADS>(tab, p.lens, p.offs, p.G, p.M, TilesFwd{WBM, p.tilesN}, p.err,
                                                      s_scan);
    total = __builtin_amdgcn_readfirstlane(total);
    // the scan scratch is free once the table is built: it passes tile ids
    TileQueue tq;
    tq.init(p.sched, total);
    int *s_id = s_scan;
    int par = 0;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t lds0 = lds_addr(smem);
    const int r32 = lane & 31, h = lane >> 5;
    const uint32_t sh = 8u * h;

    // reduction bytes per row and their stages (the weight gradient sets
    // them per expert)
    int Kb = FMT == 0 ? p.K : p.K / 2;
    const int KS = p.K / 32;
    int nk = (Kb + WROW - 1) / WROW, nfull = Kb / WROW;
    int nb_last = (Kb - nfull * WROW) / 32;                 // E4M3 blocks of the partial stage

    // per-lane fragment bases of a 256-row tile in slot 0 / 1: chunk 2j + h
    // of the lane's first A row / B row is at base ^ (j << 5)
    uint32_t aT[2], bT[2];
    {
        const uint32_t y = (uint32_t)((h ^ (r32 >> 1)) & 1) * 16u | (uint32_t)(((r32 >> 1) & 6) << 4);
        const uint32_t ra = (uint32_t)(wm * 64 + r32), rb = (uint32_t)(wn * 128 + r32);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            aT[s] = lds0 + s * WSTAGE + ra * WROW + y;
            bT[s] = lds0 + s * WSTAGE + WA_BYTES + rb * WROW + y;
        }
    }

    for (int tile = tq.first(s_id); tile < total;) {
        const int g = __builtin_amdgcn_readfirstlane(find_group(tab, tile));
        const int local = tile - __builtin_amdgcn_readfirstlane(tab.tile0[g]);
        int row0 = __builtin_amdgcn_readfirstlane(tab.row0[g]);
        int rows = __builtin_amdgcn_readfirstlane(tab.rows[g]);
        int tm = (rows + WBM - 1) / WBM;
        int nt, mt;
        grouped_tile_order(local, tm, p.tilesN, mt, nt);
        // weight gradient: the tile's token chunk of the expert (all of its
        // tokens, padded to whole blocks, without a split) starts at byte pb
        // of every channel row, its scale words at global stage s0
        uint32_t pb = 0;
        int s0 = 0, chunk = 0;
        if constexpr (WG) {
            constexpr int TPB = FMT == 0 ? 1 : 2;       // tokens per code byte
            const int ntl = p.tilesM * p.tilesN;
            chunk = local / ntl;
            const int rest = local - chunk * ntl;
            // channel tiles in bands as in the forward: a window of tiles
            // shares a few A and dY channel panels (measured on the MXFP8
            // shape: -2.3%; the BF16 weight gradient, whose experts are a few
            // hundred tokens, keeps its column-first order: +1.7% in bands)
            grouped_tile_order(rest, p.tilesM, p.tilesN, mt, nt);
            const int padded = 32 * ((rows + 31) / 32);
            const int c0 = chunk * p.split_len;
            const int clen = p.split_len > 0 ? min(p.split_len, padded - c0) : padded;
            pb = (uint32_t)(32 * __builtin_amdgcn_readfirstlane(p.plan[2 * g]) + c0) / TPB;
            s0 = __builtin_amdgcn_readfirstlane(p.plan[2 * g + 1]) + c0 / (WROW * TPB);
            Kb = clen / TPB;
            nk = (Kb + WROW - 1) / WROW;
            nfull = Kb / WROW;
            nb_last = (Kb - nfull * WROW) / 32;
            row0 = 0;
            rows = p.wrows;
            tm = p.tilesM;
        }
        const int m0 = mt * WBM;

        // One tile of TMI 32-row blocks per wave: a row block holding at most
        // 128 valid rows runs as a 128-row tile (every wave 32 rows) on the
        // three-slot ring, others as a 256-row tile on two slots.  The tile
        // ids, B panel and the order of every accumulation are the same for
        // both heights, so results do not depend on it.
        auto run_tile = [&](auto MIC) {
        constexpr int TMI = decltype(MIC)::value;
        constexpr int TBM = TMI * 128;                      // tile rows
        constexpr int NS = TMI == 2 ? 2 : 3;                // ring slots
        constexpr int ASLOT = TBM * WROW, SLOT = ASLOT + WBN * WROW;
        constexpr int TNA = ASLOT / 16 / WTHREADS;          // A loads per thread per stage
        constexpr bool CONST_SC = WSC == kWConst || WSC == kWConstRow;
        constexpr int NLS = TNA + W_LOADS + (CONST_SC ? 0 : TMI + 4);   // vector-memory ops per stage
        static_assert(NS * SLOT <= MX_RING, "ring fits");
        // a 128-row tile's per-wave offsets take a zero the compiler cannot
        // see through, so they are computed per tile rather than hoisted out
        // of the tile loop and kept live through the 256-row path
        uint32_t z = 0;
        if constexpr (TMI == 1) asm volatile("" : "+s"(z));
        const int wrow0 = wm * TMI * 32 + (int)z;
        const int vr = min(TBM, rows - m0) - wrow0;
        const int nvalid_bi = vr <= 0 ? 0 : min(TMI, (vr + 31) >> 5);
        // LDS address of chunk pair c (c = j << 5) in ring slot sl.  A 128-row
        // tile derives it from the 256-row tile's slot-0 bases (slot and row
        // offsets are multiples of 256 bytes, so they add after the XOR).
        const uint32_t a1 = aT[0] + z, b1 = bT[0] + z;
        auto aX = [&](int sl, uint32_t c) {
            if constexpr (TMI == 2) return aT[sl] ^ c;
            else return (a1 ^ c) + ((uint32_t)(sl * SLOT) - (uint32_t)(wm * 32 * WROW));
        };
        auto bX = [&](int sl, uint32_t c) {
            if constexpr (TMI == 2) return bT[sl] ^ c;
            else return (b1 ^ c) + (uint32_t)(sl * SLOT - (WA_BYTES - ASLOT));
        };

        // ---- operand loads: slot i * 512 + t holds chunk c = (t & 7) ^ ((t >> 4) & 7)
        // of tile row i * 64 + t / 8
        WOps o;
        // row pitch of the operands: the reduction length, or the channel
        // rows' pitch of the weight gradient
        // (the forward's codes may also come with a longer, line-aligned pitch)
        const uint32_t ap = (WG || p.pitch) ? (uint32_t)p.pitch : (uint32_t)Kb;
        o.b_once = !WG && tm == 1;   // an expert within one row block: no other tile reads its weights
        o.a = WG ? p.a + pb : p.a + (int64_t)row0 * ap;
        o.abytes = WG ? (uint32_t)rows * ap - pb : (uint32_t)rows * ap;
        o.b = WG ? p.b + pb : p.b + (int64_t)g * p.N * ap;
        o.bbytes = WG ? (uint32_t)p.wcols * ap - pb : (uint32_t)p.N * ap;
        o.chunk = (uint32_t)(((tid & 7) ^ ((tid >> 4) & 7)) * 16);
        o.avoff = (uint32_t)(m0 + (tid >> 3)) * ap + o.chunk;
#pragma unroll
        for (int i = 0; i < TNA; ++i) o.adelta[i] = (uint32_t)(i * 64) * ap;
        if (!epi_glu(EPI)) {
            o.bvoff = (uint32_t)(nt * WBN + (tid >> 3)) * ap + o.chunk;
#pragma unroll
            for (int i = 0; i < W_LOADS; ++i) o.bdelta[i] = (uint32_t)(i * 64) * ap;
        } else {
            // tile rows 0-63 / 64-127 / 128-191 / 192-255: gate j, up I + j,
            // gate j + 64, up I + j + 64, with j = nt * 128 + row % 64
            const int I = p.N >> 1;
            o.bvoff = (uint32_t)(nt * (WBN / 2) + (tid >> 3)) * ap + o.chunk;
            o.bdelta[0] = 0u;
            o.bdelta[1] = (uint32_t)I * ap;
            o.bdelta[2] = 64u * ap;
            o.bdelta[3] = (uint32_t)(I + 64) * ap;
        }
        ScRows sr;
        if constexpr (WSC == kWE4M3Swz || WSC == kWE2M1Swz) {
            // word (kt * rows + r) * WPR + (E2M1: lane half) of the copies
            constexpr uint32_t WPR = WSC == kWE4M3Swz ? 1u : 2u;
            const uint32_t hw = WSC == kWE2M1Swz ? 4u * h : 0u;
            sr.a = (const uint8_t *)p.sa;
            sr.astride = (uint32_t)(WG ? p.wrows : p.M) * WPR * 4u;
            sr.b = (const uint8_t *)p.sb;
            sr.bstride = WG ? (uint32_t)p.wcols * WPR * 4u : (uint32_t)p.G * (uint32_t)p.N * WPR * 4u;
            if constexpr (WG) {
                // the expert's stages start at global stage s0
                sr.a += (int64_t)s0 * sr.astride;
                sr.b += (int64_t)s0 * sr.bstride;
            }
            sr.abytes = sr.astride * (uint32_t)nk;
            sr.bbytes = sr.bstride * (uint32_t)nk;
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
                sr.row[bi] = (uint32_t)(row0 + min(m0 + wrow0 + bi * 32 + r32, rows - 1)) * WPR * 4u + hw;
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                sr.row[2 + bj] =
                    WG ? (uint32_t)min(nt * WBN + wn * 128 + bj * 32 + r32, p.wcols - 1) * WPR * 4u + hw
                       : (uint32_t)(g * p.N + clamp1<EPI>(col_of<EPI>(nt, wn * 128 + bj * 32 + r32, p.N), p.N)) *
                                 WPR * 4u +
                             hw;
        } else {
            sr.a = p.as;
            sr.abytes = (uint32_t)((p.M * KS + 3) & ~3ll);
            sr.b = p.bs;
            sr.bbytes = (uint32_t)(((int64_t)p.G * p.N * KS + 3) & ~3ll);
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
                sr.row[bi] = (uint32_t)((row0 + min(m0 + wrow0 + bi * 32 + r32, rows - 1)) * KS);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                sr.row[2 + bj] =
                    (uint32_t)((g * p.N + clamp1<EPI>(col_of<EPI>(nt, wn * 128 + bj * 32 + r32, p.N), p.N)) * KS);
        }

        // accumulators start at zero (the weight gradient adds main_grad in
        // its epilogue)
        floatx16 acc[TMI][4];
        {
#pragma unroll
            for (int i = 0; i < TMI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        }

        auto mfma = [&](int bi, int bj, intx8 a, intx8 b, const uint32_t (&w)[6], int s) {
            acc[bi][bj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                a, b, acc[bi][bj], MF, MF, 0, wscale_of<WSC>(w, bi, s, sh), 0, wscale_of<WSC>(w, 2 + bj, s, sh));
        };

        // prologue: stage 0 (the loads of each stage form one group in
        // program order), and the id of the next tile (its atomic goes out
        // first and lands under the stage's loads)
        // scale words through LDS (256-row tiles, stage-major copies): waves
        // 0 .. NSW / 2 - 1 load A's 256 rows of stage kt, the next NSW / 2
        // B's, 16 bytes per lane in row order (B's SwiGLU order: runs of 64
        // rows gate j, up I + j, gate j + 64, up I + j + 64); every lane then
        // reads its 6 rows' words after the stage's barrier
        constexpr bool LSC = TMI == 2 && (WSC == kWE4M3Swz || WSC == kWE2M1Swz);
        constexpr int SWPR = WSC == kWE2M1Swz ? 2 : 1;      // words per row
        constexpr int NSW = 2 * SWPR;                        // loading waves
        uint32_t scvoff = 0, scstride = 0, scbytes = 0;
        const uint8_t *scbase = sr.a;
        uint32_t wsc[6] = {0, 0, 0, 0, 0, 0};
        if constexpr (LSC) {
            const int isb = wave >= SWPR;                      // B's scale words
            const int pc = (wave - isb * SWPR) * 64 + lane;    // 16-byte piece of the operand's 256 rows
            const int tr = pc * 4 / SWPR;                      // its first tile row
            uint32_t row;
            if (!isb) {
                row = (uint32_t)(row0 + m0 + tr);
            } else if (!epi_glu(EPI)) {
                row = (uint32_t)((WG ? 0 : g * p.N) + nt * WBN + tr);
            } else {
                const int q = tr >> 6;
                row = (uint32_t)(g * p.N + (q & 1) * (p.N >> 1) + nt * (WBN / 2) + (q >> 1) * 64 + (tr & 63));
            }
            scvoff = row * SWPR * 4u;
            scbase = isb ? sr.b : sr.a;
            scstride = isb ? sr.bstride : sr.astride;
            scbytes = isb ? sr.bbytes : sr.abytes;
        }
        // stage kt's words into scale slot sl (past the end: nothing read)
        auto issue_sc = [&](int kt, int sl) {
            if (wave < NSW)
                dma16(scbase, scbytes,
                      smem + WSC_LDS + sl * WSC_SLOT + (wave >= SWPR ? 256 * SWPR * 4 : 0) + (wave % SWPR) * 1024,
                      kt < nk ? scvoff + (uint32_t)kt * scstride : kOOB, 0u);
        };
        // this lane's 6 words of scale slot sl: A rows wrow0 + 32 bi + r32, B
        // rows wn * 128 + 32 bj + r32 (E2M1: the lane half's word)
        auto read_sc = [&](int sl) {
            const uint32_t b0 = lds0 + WSC_LDS + sl * WSC_SLOT + (WSC == kWE2M1Swz ? 4u * h : 0u);
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) wsc[bi] = wld32(b0 + (uint32_t)(wrow0 + bi * 32 + r32) * SWPR * 4);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                wsc[2 + bj] = wld32(b0 + 256 * SWPR * 4 + (uint32_t)(wn * 128 + bj * 32 + r32) * SWPR * 4);
        };
        auto wait_sc = [&]() {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(wsc[0]), "+v"(wsc[1]), "+v"(wsc[2]), "+v"(wsc[3]), "+v"(wsc[4]), "+v"(wsc[5]));
        };
        uint32_t sc[NS][6];
        if (tid == 0) tq.issue();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int st = 0; st < NS - 1; ++st) {
            wissue_stage<TNA>(smem, o, st * SLOT, st, nk, Kb, wave, ASLOT);
            // the scale words' loads (if any) last in the stage's group
            asm volatile("" ::: "memory");
            if constexpr (LSC) issue_sc(st, st);
            else wload_scales<WSC, TMI>(sc[st], sr, st, nk, h);
            asm volatile("" ::: "memory");
        }
        wait_vmcnt<(NS - 2) * NLS>();              // stage 0 landed
        if (tid == 0) s_id[par ^ 1] = tq.resolve(tile);
        wait_lgkm0();
        barrier();
        if constexpr (LSC) {
            read_sc(0);
            wait_sc();
        }

        // Fragments.  E2M1: f*[s & 1] hold chunk 2s + h for MFMA step s (A 2 x,
        // B 4 x 16 bytes).  E4M3: step s uses chunks 4s + h and 4s + 2 + h;
        // A of the current step sits in ea, B blocks 0-1 / 2-3 in eb[0] / eb[1].
        uintx4 fa[2][2], fb[2][4];          // E2M1
        uintx4 ea[2][2], eb[2][2][2];       // E4M3 A [chunk][block], B [half][chunk][block]
        auto rdA = [&](uintx4 (&x)[2], uint32_t addr) {
            x[0] = wld<0>(addr);
            if constexpr (TMI == 2) x[1] = wld<RB>(addr);
        };
        if constexpr (FMT == 1) {
            rdA(fa[0], aX(0, 0));
            fb[0][0] = wld<0 * RB>(bX(0, 0));
            fb[0][1] = wld<1 * RB>(bX(0, 0));
            fb[0][2] = wld<2 * RB>(bX(0, 0));
            fb[0][3] = wld<3 * RB>(bX(0, 0));
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fb[0][0]), "+v"(fb[0][1]),
                         "+v"(fb[0][2]), "+v"(fb[0][3]));
        } else {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                rdA(ea[c], aX(0, (uint32_t)(c << 5)));
                eb[0][c][0] = wld<0>(bX(0, (uint32_t)(c << 5)));
                eb[0][c][1] = wld<RB>(bX(0, (uint32_t)(c << 5)));
            }
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(ea[0][0]), "+v"(ea[0][1]), "+v"(ea[1][0]), "+v"(ea[1][1]),
                         "+v"(eb[0][0][0]), "+v"(eb[0][0][1]), "+v"(eb[0][1][0]), "+v"(eb[0][1][1]));
        }

        int kt0 = 0;
        auto stage = [&](auto PC) {
            constexpr int P = decltype(PC)::value;          // ring slot of stage kt
            constexpr int Q = (P + 1) % NS, PN = (P + NS - 1) % NS;
            const int kt = kt0 + P;
            uint32_t w[6];
            if constexpr (LSC) {
#pragma unroll
                for (int i = 0; i < 6; ++i) w[i] = wsc[i];
            } else {
                wscale_words<WSC>(sc[P], w, sr, kt, nfull, nb_last, h);
            }
            // stage kt + NS - 1 goes to the slot stage kt - 1 freed at its barrier
            wissue_stage<TNA>(smem, o, PN * SLOT, kt + NS - 1, nk, Kb, wave, ASLOT);
            // the scale words' loads (if any) last in the stage's group
            asm volatile("" ::: "memory");
            if constexpr (LSC) issue_sc(kt + NS - 1, PN);
            else wload_scales<WSC, TMI>(sc[PN], sr, kt + NS - 1, nk, h);
            asm volatile("" ::: "memory");
            if constexpr (FMT == 1) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int cur = s & 1, nxt = cur ^ 1;
                    if (s < 3) {
                        const uint32_t xa = aX(P, (uint32_t)((s + 1) << 5)), xb = bX(P, (uint32_t)((s + 1) << 5));
                        rdA(fa[nxt], xa);
                        fb[nxt][0] = wld<0 * RB>(xb);
                        fb[nxt][1] = wld<1 * RB>(xb);
                        fb[nxt][2] = wld<2 * RB>(xb);
                        fb[nxt][3] = wld<3 * RB>(xb);
                    }
#pragma unroll
                    for (int bi = 0; bi < TMI; ++bi)
                        if (bi < nvalid_bi) {
#pragma unroll
                            for (int bj = 0; bj < 4; ++bj) mfma(bi, bj, pad8(fa[cur][bi]), pad8(fb[cur][bj]), w, s);
                        }
                    if (s < 3)
                        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[nxt][0]), "+v"(fa[nxt][1]), "+v"(fb[nxt][0]),
                                     "+v"(fb[nxt][1]), "+v"(fb[nxt][2]), "+v"(fb[nxt][3]));
                }
            } else {
                // substeps: (step 0, B 0-1), (0, 2-3), (1, 0-1), (1, 2-3).  One A
                // buffer: step 1's A is read once the last MFMA on step 0's A
                // has been issued.
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int s = q >> 1, half = q & 1;
                    // read ahead: B half 1 of step s, or B half 0 of step 1
                    if (q == 0 || q == 2) {
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            const uint32_t xb = bX(P, (uint32_t)((2 * s + c) << 5));
                            eb[1][c][0] = wld<2 * RB>(xb);
                            eb[1][c][1] = wld<3 * RB>(xb);
                        }
                    } else if (q == 1) {
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            const uint32_t xb = bX(P, (uint32_t)((2 + c) << 5));
                            eb[0][c][0] = wld<0>(xb);
                            eb[0][c][1] = wld<RB>(xb);
                        }
                    }
#pragma unroll
                    for (int bi = 0; bi < TMI; ++bi)
                        if (bi < nvalid_bi) {
#pragma unroll
                            for (int k = 0; k < 2; ++k)
                                mfma(bi, 2 * half + k, cat8(ea[0][bi], ea[1][bi]), cat8(eb[half][0][k], eb[half][1][k]),
                                     w, s);
                        }
                    if (q == 1) {
#pragma unroll
                        for (int c = 0; c < 2; ++c) rdA(ea[c], aX(P, (uint32_t)((2 + c) << 5)));
                    }
                    if (q == 0 || q == 2)
                        asm volatile("s_waitcnt lgkmcnt(0)"
                                     : "+v"(eb[1][0][0]), "+v"(eb[1][0][1]), "+v"(eb[1][1][0]), "+v"(eb[1][1][1]));
                    else if (q == 1)
                        asm volatile("s_waitcnt lgkmcnt(0)"
                                     : "+v"(ea[0][0]), "+v"(ea[0][1]), "+v"(ea[1][0]), "+v"(ea[1][1]),
                                       "+v"(eb[0][0][0]), "+v"(eb[0][0][1]), "+v"(eb[0][1][0]), "+v"(eb[0][1][1]));
                }
            }
            // stage kt+1 landed for this wave (NS - 2 later stages may still be
            // in flight); after the barrier for all waves, and every wave is
            // done reading slot P
            wait_vmcnt<(NS - 2) * NLS>();
            barrier();
            if (kt + 1 < nk) {
                if constexpr (LSC) read_sc(Q);
                if constexpr (FMT == 1) {
                    rdA(fa[0], aX(Q, 0));
                    fb[0][0] = wld<0 * RB>(bX(Q, 0));
                    fb[0][1] = wld<1 * RB>(bX(Q, 0));
                    fb[0][2] = wld<2 * RB>(bX(Q, 0));
                    fb[0][3] = wld<3 * RB>(bX(Q, 0));
                    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fb[0][0]),
                                 "+v"(fb[0][1]), "+v"(fb[0][2]), "+v"(fb[0][3]));
                } else {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        rdA(ea[c], aX(Q, (uint32_t)(c << 5)));
                        eb[0][c][0] = wld<0>(bX(Q, (uint32_t)(c << 5)));
                        eb[0][c][1] = wld<RB>(bX(Q, (uint32_t)(c << 5)));
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)"
                                 : "+v"(ea[0][0]), "+v"(ea[0][1]), "+v"(ea[1][0]), "+v"(ea[1][1]),
                                   "+v"(eb[0][0][0]), "+v"(eb[0][0][1]), "+v"(eb[0][1][0]), "+v"(eb[0][1][1]));
                }
                if constexpr (LSC) wait_sc();
            }
        };
        // whole rounds of the slots, then the last stages; no early exit (see
        // the 128 x 256 kernel)
        if constexpr (NS == 2) {
            for (; kt0 + 2 <= nk; kt0 += 2) {
                stage(IC<0>{});
                stage(IC<1>{});
            }
            if (kt0 < nk) stage(IC<0>{});
        } else {
            for (; kt0 + 3 <= nk; kt0 += 3) {
                stage(IC<0>{});
                stage(IC<1>{});
                stage(IC<2>{});
            }
            if (kt0 < nk) {
                stage(IC<0>{});
                if (kt0 + 1 < nk) stage(IC<1>{});
            }
            // the loads of a stage past the end (zeros) may still be landing in
            // the ring, which the epilogue and the next tile reuse
            wait_vmcnt<0>();
            barrier();
        }
        if constexpr (WSC == kWConst && !WG) {
            // one fp32 factor per tile: the product of the two tensors' scales
            const float f = p.sfa[0] * p.sfb[g];
#pragma unroll
            for (int i = 0; i < TMI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] *= f;
        } else if constexpr (WSC == kWConstRow) {
            // one factor per output row (A's row scale) and per column (the
            // expert's B row scale), multiplied together in fp32 first
            float fb[4];
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                fb[bj] = p.sfb[(int64_t)g * p.N + clamp1<EPI>(col_of<EPI>(nt, wn * 128 + bj * 32 + r32, p.N), p.N)];
#pragma unroll
            for (int bi = 0; bi < TMI; ++bi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float fa = p.sfa[row0 + min(m0 + wrow0 + bi * 32 + (r >> 2) * 8 + h * 4 + (r & 3), rows - 1)];
#pragma unroll
                    for (int bj = 0; bj < 4; ++bj) acc[bi][bj][r] *= fa * fb[bj];
                }
        }
        if constexpr (WG) {
            // The fp32 tile goes through LDS half a tile (128 rows) at a time,
            // so that main_grad is read, added to and written in whole 16-byte
            // pieces (a lane's accumulators hold one column of 16 rows), with
            // the non-temporal policy: that stream then leaves L2 before the
            // operand panels that other tiles still read.  Chunk
            // 0 adds the sum into main_grad (or overwrites it when not
            // accumulating), chunk c >= 1 writes its partial slot (none past the
            // workspace's slots, which only malformed lengths reach).  The ring
            // is free: the k-loop ended with a barrier and nothing in flight.
            float *og = (float *)p.out + (int64_t)g * p.o_gstride;
            bool keep = true;
            if (chunk > 0) {
                const int slot = slot0[g] + chunk - 1;
                keep = slot < p.nslots;
                og = p.partials + (int64_t)slot * p.o_gstride;
            }
            const bool rmw = p.accumulate && chunk == 0;
            float fwg = 1.0f;
            if constexpr (WSC == kWConst) fwg = p.sfa[0] * p.sfb[0];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if ((wm >> 1) == half) {
#pragma unroll
                    for (int bi = 0; bi < TMI; ++bi)
#pragma unroll
                        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int row = wrow0 - 128 * half + bi * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
                                *(float *)(smem + row * WG_RP + (wn * 128 + bj * 32 + r32) * 4) = acc[bi][bj][r];
                            }
                }
                wait_lgkm0();
                barrier();
                // 128 rows of 64 pieces, 16 per thread, in two rounds whose
                // main_grad pieces are loaded first, all at once
                constexpr int NPC = 128 * (WBN / 4) / WTHREADS / 2;
#pragma unroll
                for (int rd = 0; rd < 2; ++rd) {
                    floatx4 mgv[NPC];
#pragma unroll
                    for (int k = 0; k < NPC; ++k) {
                        const int ci = (rd * NPC + k) * WTHREADS + tid, rr = ci >> 6, c4 = ci & 63;
                        const int i = m0 + 128 * half + rr, n = nt * WBN + 4 * c4;
                        mgv[k] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                        if (rmw && i < rows && n < p.wcols) mgv[k] = __builtin_nontemporal_load((const floatx4 *)(og + (int64_t)i * p.ldo + n));
                    }
#pragma unroll
                    for (int k = 0; k < NPC; ++k) {
                        const int ci = (rd * NPC + k) * WTHREADS + tid, rr = ci >> 6, c4 = ci & 63;
                        const int i = m0 + 128 * half + rr, n = nt * WBN + 4 * c4;
                        const floatx4 v = *(const floatx4 *)(smem + rr * WG_RP + c4 * 16);
                        floatx4 r;
                        if constexpr (WSC == kWConst) {
                            // FP8 codes with one factor per tensor: the sum times
                            // fp32(d_a * d_dy), added by one fused multiply-add
#pragma unroll
                            for (int e = 0; e < 4; ++e) r[e] = __builtin_fmaf(fwg, v[e], mgv[k][e]);
                        } else {
                            r = mgv[k] + v;
                        }
                        if (keep && i < rows && n < p.wcols) __builtin_nontemporal_store(r, (floatx4 *)(og + (int64_t)i * p.ldo + n));
                    }
                }
                wait_lgkm0();
                barrier();
            }
        } else {
            store_tile_lds_w<EPI, 4, TMI, 4, TBM>(acc, smem, p.out, p.out_scale, p.ldo, p.N, row0, m0, rows, nt, wrow0,
                                                  wn, p.swiglu_limit, p.aux, p.ldaux, p.save, p.ldsave);
        }
        };  // run_tile
        if constexpr (WG) {
            run_tile(IC<2>{});
        } else {
            if (rows - m0 <= 128) run_tile(IC<1>{});
            else run_tile(IC<2>{});
        }
        tile = __builtin_amdgcn_readfirstlane(s_id[par ^ 1]);
        par ^= 1;
    }
}

template <int FMT, int EPI, int WSC>
hipError_t launch_wide(const MxParams &p, hipStream_t s)
{
    const int lds = wide_lds_bytes<EPI>() + table_bytes(p.G);
    auto kern = gg_mx_wide_kernel<FMT, EPI, WSC>;
    static LdsLimit lds_limit;
    hipError_t e = lds_limit.ensure((const void *)kern, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, WTHREADS, lds);
    if (e != hipSuccess) return e;
    const int64_t tiles_max = (p.M / WBM + p.G) * (int64_t)p.tilesN;
    const int64_t grid = persistent_grid(occ, tiles_max);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WTHREADS), lds, s, p);
    return hipGetLastError();
}

template <int FMT, int WSC>
hipError_t launch_wide_wgrad(const MxParams &p, hipStream_t s)
{
    const int lds = wide_lds_bytes<kEpiWgrad>() + table_bytes(p.G) + 4 * p.G;
    auto kern = gg_mx_wide_kernel<FMT, kEpiWgrad, WSC>;
    static LdsLimit lds_limit;
    hipError_t e = lds_limit.ensure((const void *)kern, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, WTHREADS, lds);
    if (e != hipSuccess) return e;
    const int64_t chunks_max = p.G + (p.split_len > 0 ? p.M / p.split_len + 1 : 0);
    const int64_t tiles_max = chunks_max * p.tilesM * p.tilesN;
    const int64_t grid = persistent_grid(occ, tiles_max);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WTHREADS), lds, s, p);
    return hipGetLastError();
}

template <int FMT, int WSC>
hipError_t launch_wide_epi(const MxParams &p, int epi, hipStream_t s)
{
    if (epi == kEpiSwiglu) return launch_wide<FMT, kEpiSwiglu, WSC>(p, s);
    if (epi == kEpiSwigluMxfp4) return launch_wide<FMT, kEpiSwigluMxfp4, WSC>(p, s);
    if (epi == kEpiSwigluSave) return launch_wide<FMT, kEpiSwigluSave, WSC>(p, s);
    if (epi == kEpiDSwiglu) return launch_wide<FMT, kEpiDSwiglu, WSC>(p, s);
    return launch_wide<FMT, kEpiNone, WSC>(p, s);
}

template <int FMT, int EPI, int SCM>
hipError_t launch_one(const MxParams &p, hipStream_t s)
{
    const int lds = NSTAGE * STAGE_BYTES + table_bytes(p.G);
    auto kern = gg_mx_kernel<FMT, EPI, SCM>;
    static LdsLimit lds_limit;
    hipError_t e = lds_limit.ensure((const void *)kern, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kThreads, lds);
    if (e != hipSuccess) return e;
    const int64_t tiles_max = (p.M / BM + p.G) * (int64_t)p.tilesN;
    const int64_t grid = persistent_grid(occ, tiles_max);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

template <int FMT, int SCM>
hipError_t launch_epi(const MxParams &p, int epi, hipStream_t s)
{
    if (epi == kEpiSwigluSave || epi == kEpiDSwiglu) return hipErrorInvalidValue;   // the 256 x 256 kernel only
    if (epi == kEpiSwiglu) return launch_one<FMT, kEpiSwiglu, SCM>(p, s);
    if (epi == kEpiSwigluMxfp4) return launch_one<FMT, kEpiSwigluMxfp4, SCM>(p, s);
    return launch_one<FMT, kEpiNone, SCM>(p, s);
}

}  // namespace

int mx_tile_m() { return BM; }
int mx_wide_tile() { return WBM; }
int mx_tile_n() { return BN; }

// Stage-major copy of a row-major E8M0 scale matrix [R][KS] for the 256 x 256
// kernel: word w of stage kt of row r lands at ((kt * R + r) * WPR + w).
// E4M3 (WPR 1): blocks 4kt .. 4kt+3 in byte order; E2M1 (WPR 2): word w holds
// blocks 8kt + w + 0, 2, 4, 6, the four that lane half w of the MFMA uses.
// Blocks past the row read as zero: a finite scale for the zero codes of a
// partial last stage.  One stage's words of 32 consecutive rows are then 32
// consecutive words (64 for E2M1), one or two cache lines per wave-wide scale
// load, where the row-major layout puts every row on a line of its own.
// One thread per row, consecutive rows in consecutive lanes, so each stage's
// words leave as one contiguous run per workgroup; a thread walks its row in
// chunks of four stages, realigning the covering words with v_alignbyte.
template <int FMT>
__global__ __launch_bounds__(256) void mx_scale_swizzle_kernel(const uint8_t *sc, uint32_t sbytes, uint32_t *out,
                                                               int R, int KS, int NS)
{
    constexpr int SB = FMT == 0 ? 4 : 8;               // scale bytes per stage
    constexpr int CH = 4;                              // stages per chunk
    constexpr int NW = CH * SB / 4 + 1;                // covering words per chunk
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= R) return;
    for (int c = 0; c * CH < NS; ++c) {
        const uint32_t start = (uint32_t)r * (uint32_t)KS + (uint32_t)(c * CH * SB);
        const uint32_t w0 = start >> 2, sh = start & 3u;
        uint32_t wd[NW];
#pragma unroll
        for (int j = 0; j < NW; ++j) wd[j] = ld_u32(sc, sbytes, (w0 + j) * 4u, 0u);
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int kt = c * CH + k;
            if (kt >= NS) break;
            // bytes of the stage's words that lie inside the row
            const int n0 = KS - kt * SB;
            const uint32_t keep0 = n0 >= 4 ? 0xFFFFFFFFu : (n0 <= 0 ? 0u : (1u << (8 * n0)) - 1u);
            const uint32_t v0 = __builtin_amdgcn_alignbyte(wd[k * SB / 4 + 1], wd[k * SB / 4], sh) & keep0;
            if (FMT == 0) {
                out[(int64_t)kt * R + r] = v0;
            } else {
                const int n1 = n0 - 4;
                const uint32_t keep1 = n1 >= 4 ? 0xFFFFFFFFu : (n1 <= 0 ? 0u : (1u << (8 * n1)) - 1u);
                const uint32_t v1 = __builtin_amdgcn_alignbyte(wd[k * 2 + 2], wd[k * 2 + 1], sh) & keep1;
                *(uintx2 *)(out + ((int64_t)kt * R + r) * 2) =
                    uintx2{__builtin_amdgcn_perm(v1, v0, 0x06040200u), __builtin_amdgcn_perm(v1, v0, 0x07050301u)};
            }
        }
    }
}

int64_t mx_swizzle_bytes(int64_t rows, int64_t K, int fmt)
{
    const int64_t KS = K / 32, NS = fmt == 0 ? (KS + 3) / 4 : (KS + 7) / 8;
    return NS * rows * (fmt == 0 ? 1 : 2) * 4;
}

hipError_t launch_mx_scale_swizzle(const uint8_t *scales, int64_t rows, int64_t K, int fmt, uint32_t *out,
                                   hipStream_t s)
{
    const int KS = (int)(K / 32), NS = fmt == 0 ? (KS + 3) / 4 : (KS + 7) / 8;
    const uint32_t sbytes = (uint32_t)((rows * KS + 3) & ~3ll);
    const dim3 grid((unsigned)((rows + 255) / 256));
    if (fmt == 0)
        hipLaunchKernelGGL(mx_scale_swizzle_kernel<0>, grid, dim3(256), 0, s, scales, sbytes, out, (int)rows, KS, NS);
    else
        hipLaunchKernelGGL(mx_scale_swizzle_kernel<1>, grid, dim3(256), 0, s, scales, sbytes, out, (int)rows, KS, NS);
    return hipGetLastError();
}

hipError_t launch_mx_wgrad(const MxParams &p, int fmt, hipStream_t s)
{
    if (fmt == 2) return launch_wide_wgrad<0, kWConst>(p, s);     // E4M3 codes with one factor per tensor
    return fmt == 0 ? launch_wide_wgrad<0, kWE4M3Swz>(p, s) : launch_wide_wgrad<1, kWE2M1Swz>(p, s);
}

hipError_t launch_mx(const MxParams &p, int fmt, int epi, hipStream_t s)
{
    if (p.sfa) return p.sf_rows ? launch_wide_epi<0, kWConstRow>(p, epi, s) : launch_wide_epi<0, kWConst>(p, epi, s);
    // the 128 x 256 kernel on row-major scales when asked (bit-identical results)
    if (p.narrow) {
        if (fmt == 0) return launch_epi<0, kScE4M3>(p, epi, s);
        return p.K % 128 == 0 ? launch_epi<1, kScE2M1Word>(p, epi, s) : launch_epi<1, kScE2M1Span>(p, epi, s);
    }
    if (p.sa && p.sb)
        return fmt == 0 ? launch_wide_epi<0, kWE4M3Swz>(p, epi, s) : launch_wide_epi<1, kWE2M1Swz>(p, epi, s);
    if (fmt == 0) {
        if (p.K % 128 == 0) return launch_wide_epi<0, kWE4M3Word>(p, epi, s);
        return launch_wide_epi<0, kWE4M3Span>(p, epi, s);
    }
    if (p.K % 256 == 0) return launch_wide_epi<1, kWE2M1Pair>(p, epi, s);
    // E2M1 whose stage of 8 scale blocks would not start on a word
    if (p.K % 128 == 0) return launch_epi<1, kScE2M1Word>(p, epi, s);
    return launch_epi<1, kScE2M1Span>(p, epi, s);
}

}  // namespace ptgg
