// common.hpp -- device helpers shared by the grouped GEMM and quantise kernels
// (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptgg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uintx2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;    // 4 wave64s per workgroup
constexpr int kWave = 64;

// sticky device error bits (same meaning as documented in ptgg.h)
constexpr uint32_t kErrNegativeLen = 1u;
constexpr uint32_t kErrClamped = 2u;
constexpr uint32_t kErrSumMismatch = 4u;
constexpr uint32_t kErrBadPointer = 8u;     // an expert weight address NULL or not 16-byte aligned

// ------------------------------------------------------------------ numerics
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// fp32 -> bf16 bits, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = f32_bits(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return bits_f32(h << 16); }

// silu(gate) * up = gate / (1 + e^-gate) * up, with the hardware reciprocal
// (1 ulp) instead of an IEEE division; 1/inf = 0 gives the limit for very
// negative gates.
// With a finite lim the clamped form: gate at most lim, up within
// [-lim, lim]; lim = +inf leaves both as they are.
__device__ __forceinline__ float silu_mul(float gate, float up, float lim)
{
    gate = __builtin_fminf(gate, lim);
    up = __builtin_fminf(__builtin_fmaxf(up, -lim), lim);
    return gate * __builtin_amdgcn_rcpf(1.0f + __expf(-gate)) * up;
}

// ------------------------------------------------------------------ MX encode
// Integer-exact OCP-MX encoding from bf16 bits.  A bf16 value is
//   Mant * 2^t0  with Mant = 128 + m (normal, t0 = e - 134) or m (subnormal,
//   t0 = -133).  Scaling by 2^(127 - E) only moves t0, so every step below is
//   exact integer arithmetic with one round-to-nearest-even.

// These three are plain integer code, also compiled for the host so that the
// encoder can be checked exhaustively against the rounding rule on a CPU.

// Shared block exponent byte from the largest magnitude's bf16 bits (sign
// cleared): floor(log2 amax) - emax + 127, clamped to [0, 254]; a subnormal or
// zero amax always clamps to 0 for both element formats.
template <int EMAX>
__host__ __device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits)
{
    int ef = (int)(amax_bits >> 7) & 0xFF;
    int E = ef - EMAX;            // floor(log2) = ef - 127; + 127 - EMAX
    E = E < 0 ? 0 : E;
    return (uint32_t)(E > 254 ? 254 : E);
}

// Round Mant * 2^s to the nearest integer, ties to even (Mant < 2^8).
__host__ __device__ __forceinline__ uint32_t rne_shift(uint32_t mant, int s)
{
    if (s >= 0)
        return mant << s;
    int sh = -s;
    if (sh > 9)
        return 0;                  // < 2^8 / 2^10 < 1/2
    uint32_t q = mant >> sh;
    uint32_t rem = mant & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
    return q;
}

// Code of one element (bf16 bits h) under block exponent byte E.
// FMT 0: E4M3 (byte), FMT 1: E2M1 (nibble).
template <int FMT>
__host__ __device__ __forceinline__ uint32_t mx_encode(uint32_t h, uint32_t E)
{
    uint32_t sign = (h >> 15) & 1u;
    int ef = (int)(h >> 7) & 0xFF;
    uint32_t mant = ef ? (128u | (h & 0x7Fu)) : (h & 0x7Fu);
    int t = (ef ? ef - 134 : -133) + 127 - (int)E;
    uint32_t code;
    if (mant == 0) {
        code = 0;
    } else {
        int L = (31 - __builtin_clz(mant)) + t;           // floor(log2 |x|)
        if (FMT == 0) {
            if (L >= -6) {
                uint32_t q = rne_shift(mant, t - (L - 3));  // in [8, 16]
                if (q == 16) { ++L; q = 8; }
                code = (L > 8 || (L == 8 && q > 14)) ? 0x7Eu : (uint32_t)(((L + 7) << 3) | (int)(q - 8));
            } else {
                code = rne_shift(mant, t + 9);              // subnormal grid 2^-9
            }
        } else {
            if (L >= 0) {
                uint32_t q = rne_shift(mant, t - (L - 1));  // in [2, 4]
                if (q == 4) { ++L; q = 2; }
                code = (L > 2) ? 7u : (uint32_t)(((L + 1) << 1) | (int)(q - 2));
            } else {
                code = rne_shift(mant, t + 1);              // subnormal grid 1/2
            }
        }
    }
    return FMT == 0 ? (sign << 7) | code : (sign << 3) | code;
}

// ------------------------------------------------------------------ scheduler
// Per-workgroup table of the ragged batch, built in LDS from the device-side
// group lengths (no host synchronisation).  For every expert g:
//   row0[g]  first row (clamped into [0, M]),  rows[g] row count (clamped),
//   tile0[g] first linear tile id; tile0[G] = total tiles.
struct GroupTable {
    int *row0;
    int *rows;
    int *tile0;
    int G;
};

// Bytes of LDS the table needs for G experts.
// (3G + 1 ints, then scan scratch for up to 8 waves)
__host__ __device__ constexpr int table_bytes(int G) { return 4 * (3 * G + 1) + 32; }

// Exclusive scan over v (one value per thread) across the NT-thread block;
// returns this thread's exclusive prefix and writes the block total to *total.
template <int NT = kThreads>
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_wave, int *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        int s = s_wave[w];
        before += (w < wave) ? s : 0;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

// Tile counting rule: tiles(rows) for a given expert.
struct TilesFwd {          // fwd/dgrad: ceil(rows / BM) row blocks x column tiles
    int bm, ntiles;
    __device__ int operator()(int rows) const { return ((rows + bm - 1) / bm) * ntiles; }
};
struct TilesWgrad {        // wgrad: the whole output of active experts
    int ntiles, accumulate;
    __device__ int operator()(int rows) const { return (rows > 0 || !accumulate) ? ntiles : 0; }
};

template <class Tiles, int NT = kThreads>
__device__ __forceinline__ int build_group_table(GroupTable &t, const int64_t *lens, const int64_t *offs,
                                 int G, int64_t M, Tiles tiles, uint32_t *err, int *s_scratch)
{
    const int tid = threadIdx.x;
    const int per = (G + NT - 1) / NT;
    const int g0 = tid * per;
    uint32_t flags = 0;
    // pass 1: clamped lengths and (if no offsets) their prefix
    int sum = 0;
    for (int i = 0; i < per; ++i) {
        int g = g0 + i;
        if (g < G) {
            int64_t l = lens[g];
            if (l < 0) { flags |= kErrNegativeLen; l = 0; }
            if (l > M) { flags |= kErrClamped; l = M; }
            t.rows[g] = (int)l;
            sum += (int)l;
        }
    }
    int total_rows;
    int pre = block_exclusive_scan<NT>(sum, s_scratch, &total_rows);
    for (int i = 0; i < per; ++i) {
        int g = g0 + i;
        if (g < G) {
            int64_t start = offs ? offs[g] : (int64_t)pre;
            int64_t l = t.rows[g];
            pre += (int)l;
            if (start < 0 || start > M) { flags |= kErrClamped; start = start < 0 ? 0 : M; }
            if (start + l > M) { flags |= kErrClamped; l = M - start; }
            t.row0[g] = (int)start;
            t.rows[g] = (int)l;
        }
    }
    // pass 2: tile prefix
    int tsum = 0;
    for (int i = 0; i < per; ++i) {
        int g = g0 + i;
        if (g < G) tsum += tiles(t.rows[g]);
    }
    int total_tiles;
    int tpre = block_exclusive_scan<NT>(tsum, s_scratch, &total_tiles);
    for (int i = 0; i < per; ++i) {
        int g = g0 + i;
        if (g < G) {
            t.tile0[g] = tpre;
            tpre += tiles(t.rows[g]);
        }
    }
    if (tid == 0) {
        t.tile0[G] = total_tiles;
        if (!offs && total_rows != M) flags |= kErrSumMismatch;
        if (offs && (offs[G] < 0 || offs[G] > M)) flags |= kErrSumMismatch;
    }
    if (offs) {
        // explicit offsets may leave rows between experts unowned, but the
        // ranges must come in expert order without overlapping:
        // offs[g] + lens[g] <= offs[g + 1]
        for (int i = 0; i < per; ++i) {
            int g = g0 + i;
            if (g < G && offs[g] + lens[g] > offs[g + 1]) flags |= kErrSumMismatch;
        }
    }
    if (flags && err && (blockIdx.x == 0)) atomicOr(err, flags);
    __syncthreads();
    return t.tile0[G];
}

// Split weight gradient (the BF16 and MX kernels).  The weight gradient
// reduces over an expert's tokens.  With a chunk length
// L > 0, an expert is cut into chunks of L consecutive tokens (the last one
// shorter), and every chunk covers the whole output: tiles (expert, chunk,
// K tile, N tile).  Chunk 0 reads-modifies-writes main_grad as an uncut
// expert does; chunk c >= 1 writes its fp32 partial sum to workspace slot
// slot0[g] + c - 1, and launch_wgrad_split_reduce then adds the partials to
// main_grad in chunk order.  The order of every sum is fixed, so the result
// is deterministic.  Experts with no tokens: no tiles when accumulating, one
// zero-writing chunk when not.
struct TilesWgradSplit {
    int ntiles, accumulate, L;
    __device__ int chunks(int rows) const { return rows > 0 ? (L > 0 ? (rows + L - 1) / L : 1) : (accumulate ? 0 : 1); }
    __device__ int operator()(int rows) const { return chunks(rows) * ntiles; }
};

// slot0[g] = sum over earlier experts of (chunks - 1): the first partial
// slot of expert g (needs the table's clamped rows).  NT threads.
template <int NT>
__device__ __forceinline__ void wgrad_slot_table(const GroupTable &tab, const TilesWgradSplit &tw, int *slot0,
                                                 int *s_scan)
{
    const int per = (tab.G + NT - 1) / NT, g0 = (int)threadIdx.x * per;
    int v = 0;
    for (int i = 0; i < per; ++i)
        if (g0 + i < tab.G) v += max(tw.chunks(tab.rows[g0 + i]) - 1, 0);
    int tot;
    int pre = block_exclusive_scan<NT>(v, s_scan, &tot);
    for (int i = 0; i < per; ++i)
        if (g0 + i < tab.G) {
            slot0[g0 + i] = pre;
            pre += max(tw.chunks(tab.rows[g0 + i]) - 1, 0);
        }
    __syncthreads();
}

// Expert owning linear tile id `tile` (the last g with tile0[g] <= tile).
__device__ __forceinline__ int find_group(const GroupTable &t, int tile)
{
    int lo = 0, hi = t.G;          // tile0[lo] <= tile < tile0[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (t.tile0[mid] <= tile) lo = mid; else hi = mid;
    }
    return lo;
}

// Row tile mt and column tile nt of an expert's local tile id (tm row tiles,
// tn column tiles).  Ids walk the row tiles first inside bands of up to 8 row
// tiles, then the column tiles, then the next band: a window of consecutive
// ids (what one XCD runs at a time) then reads a few weight panels and a few
// activation row blocks, each shared by several tiles in the XCD's L2, where
// walking all row tiles of a long expert first would stream its whole
// activation block through L2 once per column tile.  An expert of at most 8
// row tiles keeps the plain row-first order.
__device__ __forceinline__ void grouped_tile_order(int local, int tm, int tn, int &mt, int &nt)
{
    constexpr int GM = 8;
    const int band = local / (GM * tn);
    const int m0 = band * GM;
    const int h = min(GM, tm - m0);
    const int rem = local - band * GM * tn;
    nt = rem / h;
    mt = m0 + rem % h;
}

// Workgroups are dispatched round-robin over the 8 XCDs; renumber them so that
// consecutive logical ids share an XCD (and its L2): tiles that read the same
// weight panel then run on the same XCD at the same time.
__device__ __forceinline__ int xcd_logical_id()
{
    const int n = gridDim.x, b = blockIdx.x;
    if (n % 8) return b;
    return (b % 8) * (n / 8) + b / 8;
}

}  // namespace ptgg
