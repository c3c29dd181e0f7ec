// api.cpp -- the C ABI (include/ptgg.h): host-side argument checks and
// dispatch to the gfx950 kernels.  Nothing here reads device memory,
// allocates or synchronises (except pt_read_error_flags, a test helper).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/ptgg.h"
#include "launch.hpp"

namespace ptgg {

int device_cus()
{
    // per device; concurrent first calls store the same value
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

// 1 when the current device is gfx950, 0 otherwise (cached per device).
bool device_is_gfx950()
{
    static int state[64] = {0};  // 0 unknown, 1 yes, 2 no
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    std::lock_guard<std::mutex> lock(mu);
    if (state[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return state[dev] == 1;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// The kernels address each operand with 32-bit byte offsets (buffer
// resources whose out-of-range offsets start at 2^31).
bool fits31(int64_t bytes) { return bytes < ((int64_t)1 << 31); }

int check_groups(const int64_t *lens, int64_t G, int64_t M)
{
    if (!lens || G < 1 || M < 0) return PT_ERR_INVALID_ARG;
    if (G > PT_MAX_GROUPS) return PT_ERR_UNSUPPORTED;
    if (M > (int64_t)INT32_MAX / 2) return PT_ERR_UNSUPPORTED;
    return PT_OK;
}

uint32_t *error_word(void *ws, size_t bytes) { return (ws && bytes >= 4) ? (uint32_t *)ws : nullptr; }

// The tile-queue counters, when the workspace has room for them; without
// them the persistent kernels take tiles in a static order.
uint32_t *queue_words(void *ws, size_t bytes)
{
    return (ws && bytes >= (size_t)kQueueWsBytes) ? (uint32_t *)((uint8_t *)ws + kQueueWsOffset) : nullptr;
}

// MX forward: the stage-major copies of the A and B scales follow the queues
// in the workspace (256-byte aligned); 0 when the sizes do not allow them.
int64_t round256(int64_t x) { return (x + 255) & ~(int64_t)255; }
int64_t mx_swz_a_bytes(int64_t M, int64_t K, int fmt) { return round256(mx_swizzle_bytes(M, K, fmt)); }
int64_t mx_swz_b_bytes(int64_t G, int64_t N, int64_t K, int fmt) { return round256(mx_swizzle_bytes(G * N, K, fmt)); }
bool mx_swz_possible(int64_t G, int64_t M, int64_t N, int64_t K, int fmt)
{
    return K <= kMxSwzMaxK && fits31(mx_swizzle_bytes(M, K, fmt)) && fits31(mx_swizzle_bytes(G * N, K, fmt));
}

// Split weight gradient: token chunk length and partial slots for a problem
// with M rows and ntl output tiles per expert (256 x 256).  About 4 work units
// per compute unit of the 256 on an MI355X: L = max(512, ceil(M ntl / 1024)),
// so the split only engages where few output tiles per expert leave long
// experts as a serial tail; at most M / L experts are cut, and the chunks
// past each expert's first need at most M / L partial slots.
constexpr int64_t kSplitMinLen = 512;
int64_t wgrad_split_len(int64_t M, int64_t Mout, int64_t Nout)
{
    const int64_t ntl = ((Mout + 255) / 256) * ((Nout + 255) / 256);
    const int64_t L = (M * ntl + 1023) / 1024;
    return L > kSplitMinLen ? L : kSplitMinLen;
}
int64_t wgrad_split_slots(int64_t M, int64_t Mout, int64_t Nout) { return M / wgrad_split_len(M, Mout, Nout); }
int64_t wgrad_split_bytes(int64_t M, int64_t K, int64_t N)
{
    return round256(wgrad_split_slots(M, K, N) * K * N * 4);
}

// Zero the queues (if any) ahead of the launch on the same stream.
template <class Launch>
hipError_t queued(uint32_t *sched, hipStream_t s, Launch launch)
{
    if (sched) {
        hipError_t e = launch_queue_reset(sched, s);
        if (e != hipSuccess) return e;
    }
    return launch();
}

int hip_status(hipError_t e) { return e == hipSuccess ? PT_OK : PT_ERR_HIP; }

// The SwiGLU clamp the kernels apply: +inf (none) for a limit <= 0 or infinite.
float swiglu_clamp(float limit)
{
    return (limit > 0.0f && limit < __builtin_huge_valf()) ? limit : __builtin_huge_valf();
}

// ---------------------------------------------------------------- kernel configurations and tuning
// A configuration of one grouped GEMM call: bit 0 takes tiles in the static
// order even when the workspace holds queues, bit 1 runs the 128 x 256
// kernel.  Every configuration computes the same sums in the same order, so
// results are bit-identical; only speed differs.  The mode is process-wide:
// fixed rules (configuration 0), a forced configuration, or tuning, where
// the first call of each problem class times every configuration that
// applies on the call's own buffers and keeps the fastest.
constexpr int kCfgStatic = 1, kCfgNarrow = 2, kNumCfg = 4;
constexpr int kTuneSlots = 512;
std::atomic<int> g_mode{PT_CONFIG_RULES};

struct TuneKey {
    int dev, op, dtype, epi, trans;
    int64_t G, Mb, N, K;
    bool operator==(const TuneKey &o) const
    {
        return dev == o.dev && op == o.op && dtype == o.dtype && epi == o.epi && trans == o.trans && G == o.G &&
               Mb == o.Mb && N == o.N && K == o.K;
    }
};
struct TuneEntry {
    TuneKey key;
    int cfg;
};
std::mutex g_tune_mu;
TuneEntry g_tune[kTuneSlots];
int g_ntune = 0;

// Problem class: the row count enters rounded up to a power of two.
TuneKey tune_key(int op, int dtype, int epi, int trans, int64_t G, int64_t M, int64_t N, int64_t K)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    int64_t mb = 1;
    while (mb < M) mb <<= 1;
    return TuneKey{dev, op, dtype, epi, trans, G, mb, N, K};
}

int tune_lookup(const TuneKey &k)
{
    std::lock_guard<std::mutex> lock(g_tune_mu);
    for (int i = 0; i < g_ntune; ++i)
        if (g_tune[i].key == k) return g_tune[i].cfg;
    return -1;
}

void tune_store(const TuneKey &k, int cfg)
{
    std::lock_guard<std::mutex> lock(g_tune_mu);
    for (int i = 0; i < g_ntune; ++i)
        if (g_tune[i].key == k) {
            g_tune[i].cfg = cfg;
            return;
        }
    if (g_ntune < kTuneSlots) g_tune[g_ntune++] = TuneEntry{k, cfg};
}

bool tune_full()
{
    std::lock_guard<std::mutex> lock(g_tune_mu);
    return g_ntune >= kTuneSlots;
}

// The applicable configuration nearest to c (dropping what does not apply).
int clamp_cfg(int c, unsigned allowed)
{
    if ((allowed >> c) & 1u) return c;
    if ((allowed >> (c & ~kCfgNarrow)) & 1u) return c & ~kCfgNarrow;
    if ((allowed >> (c & ~kCfgStatic)) & 1u) return c & ~kCfgStatic;
    return 0;
}

// Configurations that apply: the static order only differs when the
// workspace holds queues, the narrow kernel only where one exists.
unsigned cfg_mask(bool queues, bool narrow_ok)
{
    unsigned m = 0;
    for (int c = 0; c < kNumCfg; ++c)
        if ((queues || !(c & kCfgStatic)) && (narrow_ok || !(c & kCfgNarrow))) m |= 1u << c;
    return m;
}

// The rules' configuration: the queued 256 x 256 kernel, except that a
// problem whose every tile can start at once (at most one 256 x 256 tile per
// CU, bounded with M rounded up to a power of two) takes the static order,
// which saves the queue-reset launch and changes nothing else.
int rules_cfg(const TuneKey &key, unsigned allowed)
{
    const int64_t w = key.op == PT_OP_WGRAD ? ((key.K + 255) / 256) * ((key.N + 255) / 256)
                                            : (std::max(key.N, key.K) + 255) / 256;
    const int64_t tiles = key.op == PT_OP_WGRAD ? key.G * w : (key.Mb / 256 + key.G) * w;
    return (tiles <= device_cus() && ((allowed >> kCfgStatic) & 1u)) ? kCfgStatic : 0;
}

// Launch through run(cfg) under the current mode.  A call that must not run
// twice (an accumulating weight gradient) is never timed: it takes a tuned
// choice if its class has one, else the rules.
template <class Run>
int configured(const TuneKey &key, unsigned allowed, bool repeatable, hipStream_t s, Run run)
{
    const int mode = g_mode.load(std::memory_order_relaxed);
    if (mode >= 0) return hip_status(run(clamp_cfg(mode, allowed)));
    if (mode == PT_CONFIG_RULES) return hip_status(run(rules_cfg(key, allowed)));
    const int known = tune_lookup(key);
    if (known >= 0) return hip_status(run(clamp_cfg(known, allowed)));
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (!repeatable || tune_full() || hipStreamIsCapturing(s, &cap) != hipSuccess ||
        cap != hipStreamCaptureStatusNone)
        return hip_status(run(rules_cfg(key, allowed)));
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return PT_ERR_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return PT_ERR_HIP;
    }
    int best = -1;
    float best_ms = 0.0f;
    hipError_t e = hipSuccess;
    for (int c = 0; c < kNumCfg && e == hipSuccess; ++c) {
        if (!((allowed >> c) & 1u)) continue;
        e = run(c);                                       // warm-up (and first-use set-up)
        if (e == hipSuccess) e = hipEventRecord(e0, s);
        for (int i = 0; i < 3 && e == hipSuccess; ++i) e = run(c);
        if (e == hipSuccess) e = hipEventRecord(e1, s);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess && (best < 0 || ms < best_ms)) {
            best = c;
            best_ms = ms;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (e != hipSuccess || best < 0) return PT_ERR_HIP;
    tune_store(key, best);
    return hip_status(run(best));                         // the output comes from the choice
}

}  // namespace
}  // namespace ptgg

using namespace ptgg;

// An MX grouped GEMM out[r, j] = sum_q A[r, q] * B_g[j, q] over a reduction of
// K values (A [M, K] and B [G, N, K], both packed and scaled along K), with
// epilogue `ep` (Nc columns per expert before the epilogue's pairing, output
// row stride ldo).  Shared by the forward and the MX data gradient.
// PT_FP8_E4M3 takes the same path with one fp32 scale for A (a_scale) and
// one per expert for B (b_scale) in place of the E8M0 block scales.
static int mx_gemm(int op, const void *a, const uint8_t *a_scale, const void *b, const uint8_t *b_scale, void *out,
                   uint8_t *out_scale, const int64_t *group_lens, const int64_t *group_offs, int64_t G, int64_t M,
                   int64_t N, int64_t K, int dtype, int ep, int64_t Nc, int64_t ldo, float swiglu_limit,
                   void *workspace, size_t workspace_bytes, hipStream_t s, uint16_t *save = nullptr,
                   bool timing = true, const uint16_t *aux = nullptr, int64_t pitch = 0)
{
    const bool tensor_scales = dtype == PT_FP8_E4M3 || dtype == PT_FP8_E4M3_ROWWISE;
    if (N % 8) return PT_ERR_UNSUPPORTED;              // outputs leave in 16-byte chunks
    if (K % 32) return PT_ERR_UNSUPPORTED;
    if (M > 0 && (!a_scale || !b_scale)) return PT_ERR_INVALID_ARG;
    if (!aligned4(a_scale) || !aligned4(b_scale)) return PT_ERR_MISALIGNED;
    const int64_t kb = dtype == PT_MXFP4_E2M1 ? K / 2 : K;      // code bytes per row
    if (pitch && (pitch < kb || pitch % 16)) return PT_ERR_INVALID_ARG;
    const int64_t rb = pitch ? pitch : kb;                      // bytes between code rows
    if (!fits31(M * rb) || !fits31(N * rb) || !fits31(G * N * (K / 32) + 4)) return PT_ERR_UNSUPPORTED;
    MxParams p = {};
    p.pitch = pitch;
    p.swiglu_limit = swiglu_clamp(swiglu_limit);
    p.save = save;
    p.ldsave = (int)N;
    p.aux = aux;
    p.ldaux = (int)(2 * N);
    p.a = (const uint8_t *)a;
    p.as = a_scale;
    p.b = (const uint8_t *)b;
    p.bs = b_scale;
    p.out = out;
    p.out_scale = out_scale;
    p.lens = group_lens;
    p.offs = group_offs;
    p.err = error_word(workspace, workspace_bytes);
    p.G = (int)G;
    p.M = M;
    p.N = (int)N;
    p.K = (int)K;
    p.ldo = (int)ldo;
    const int tn = epi_glu(ep) ? mx_tile_n() / 2 : mx_tile_n();
    p.tilesN = (int)((Nc + tn - 1) / tn);
    p.sched = queue_words(workspace, workspace_bytes);
    if (tensor_scales) {
        p.sfa = (const float *)a_scale;
        p.sfb = (const float *)b_scale;
        p.sf_rows = dtype == PT_FP8_E4M3_ROWWISE;
        p.as = p.bs = nullptr;
    }
    if (M == 0) return PT_OK;
    const int fmt = dtype == PT_MXFP4_E2M1 ? 1 : 0;
    // a workspace with room for them gets stage-major copies of the scales
    // (read by the 256 x 256 kernel; the 128 x 256 one reads them row-major)
    const bool swz = !tensor_scales && p.sched && mx_swz_possible(G, M, N, K, fmt) &&
                     workspace_bytes >= (size_t)(kQueueWsBytes + mx_swz_a_bytes(M, K, fmt) +
                                                 mx_swz_b_bytes(G, N, K, fmt));
    // the SwiGLU that keeps its input exists for the 256 x 256 kernel only,
    // which E2M1 with K % 256 != 0 reaches through the scale copies alone
    // (and so are code rows with their own pitch)
    const bool wide_only = ep == kEpiSwigluSave || ep == kEpiDSwiglu || pitch != 0;
    if (wide_only && fmt == 1 && K % 256 && !swz) return PT_ERR_UNSUPPORTED;
    uint32_t *queues = p.sched;
    const TuneKey key = tune_key(op, dtype, ep, pitch ? 2 : 0, G, M, N, K);
    return configured(key, cfg_mask(queues != nullptr, !tensor_scales && !wide_only), timing, s, [&](int cfg) {
        p.narrow = (cfg & kCfgNarrow) != 0;
        p.sched = (cfg & kCfgStatic) ? nullptr : queues;
        p.sa = p.sb = nullptr;
        if (swz && !p.narrow) {
            uint32_t *sa = (uint32_t *)((uint8_t *)workspace + kQueueWsBytes);
            uint32_t *sb = (uint32_t *)((uint8_t *)sa + mx_swz_a_bytes(M, K, fmt));
            hipError_t e = launch_mx_scale_swizzle(a_scale, M, K, fmt, sa, s);
            if (e == hipSuccess) e = launch_mx_scale_swizzle(b_scale, G * N, K, fmt, sb, s);
            if (e != hipSuccess) return e;
            p.sa = sa;
            p.sb = sb;
        }
        return queued(p.sched, s, [&] { return launch_mx(p, fmt, ep, s); });
    });
}

// The grouped forward behind pt_grouped_gemm_fwd and
// pt_grouped_gemm_fwd_noalloc; `timing` false never times configurations
// (tuning mode then takes a tuned choice or configuration 0).
static int grouped_fwd(const void *a, const uint8_t *a_scale, const void *b, const uint8_t *b_scale, void *out,
                       uint8_t *out_scale, const int64_t *group_lens, const int64_t *group_offs, int64_t G, int64_t M,
                       int64_t N, int64_t K, int dtype, int trans_b, int epilogue, float swiglu_limit,
                       void *workspace, size_t workspace_bytes, void *stream, bool timing, int64_t pitch = 0)
{
    if (pitch < 0 || (pitch && dtype == PT_BF16)) return pitch < 0 ? PT_ERR_INVALID_ARG : PT_ERR_UNSUPPORTED;
    if (swiglu_limit != swiglu_limit) return PT_ERR_INVALID_ARG;   // NaN
    int st = check_groups(group_lens, G, M);
    if (st) return st;
    if (N < 1 || K < 1 || N > INT32_MAX / 4 || K > INT32_MAX / 4) return PT_ERR_INVALID_ARG;
    if (M > 0 && (!a || !b || !out)) return PT_ERR_INVALID_ARG;
    if (epilogue < PT_EPI_NONE || epilogue > PT_EPI_SWIGLU_MXFP4) return PT_ERR_UNSUPPORTED;
    if (trans_b != 0 && trans_b != 1) return PT_ERR_INVALID_ARG;
    if (epilogue == PT_EPI_SWIGLU && N % 16) return PT_ERR_UNSUPPORTED;
    if (epilogue == PT_EPI_SWIGLU_MXFP4 && !out_scale) return PT_ERR_INVALID_ARG;
    if (epilogue == PT_EPI_SWIGLU_MXFP4 && N % 64) return PT_ERR_UNSUPPORTED;
    if (epilogue != PT_EPI_SWIGLU_MXFP4 && out_scale) return PT_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(b) || !aligned16(out)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const int ep = epilogue == PT_EPI_SWIGLU ? kEpiSwiglu : epilogue == PT_EPI_SWIGLU_MXFP4 ? kEpiSwigluMxfp4 : kEpiNone;
    const int64_t Nc = epilogue == PT_EPI_NONE ? N : N / 2;   // columns per expert tile
    const int64_t ldo = epilogue == PT_EPI_NONE ? N : epilogue == PT_EPI_SWIGLU ? N / 2 : N / 4;
    if (dtype == PT_BF16) {
        if (a_scale || b_scale) return PT_ERR_INVALID_ARG;
        if (K % 8) return PT_ERR_UNSUPPORTED;
        if (!trans_b && N % 8) return PT_ERR_UNSUPPORTED;
        if (!fits31(M * K * 2) || !fits31(N * K * 2)) return PT_ERR_UNSUPPORTED;
        Bf16Params p = {};
        p.swiglu_limit = __builtin_huge_valf();
        p.a = (const uint16_t *)a;
        p.b = (const uint16_t *)b;
        p.out = out;
        p.out_scale = out_scale;
        p.swiglu_limit = swiglu_clamp(swiglu_limit);
        p.lens = group_lens;
        p.offs = group_offs;
        p.err = error_word(workspace, workspace_bytes);
        p.G = (int)G;
        p.M = M;
        p.Kred = (int)K;
        p.Nout = (int)N;
        p.lda = (int)K;
        p.ldb = trans_b ? (int)K : (int)N;
        p.b_gstride = N * K;
        p.ldo = (int)ldo;
        p.tilesN = (int)((Nc + (epilogue == PT_EPI_NONE ? bf16_tile_n() : bf16_tile_n() / 2) - 1) /
                         (epilogue == PT_EPI_NONE ? bf16_tile_n() : bf16_tile_n() / 2));
        p.sched = queue_words(workspace, workspace_bytes);
        if (M == 0) return PT_OK;
        uint32_t *queues = p.sched;
        const TuneKey key = tune_key(PT_OP_FWD, dtype, ep, trans_b, G, M, N, K);
        return configured(key, cfg_mask(queues != nullptr, true), timing, s, [&](int cfg) {
            p.narrow = (cfg & kCfgNarrow) != 0;
            p.sched = (cfg & kCfgStatic) ? nullptr : queues;
            return queued(p.sched, s, [&] { return launch_bf16(p, trans_b ? kFwdKContig : kFwdNContig, ep, s); });
        });
    }
    if (dtype == PT_MXFP8_E4M3 || dtype == PT_MXFP4_E2M1 || dtype == PT_FP8_E4M3 || dtype == PT_FP8_E4M3_ROWWISE) {
        if (!trans_b) return PT_ERR_UNSUPPORTED;           // K-contiguous codes
        return mx_gemm(PT_OP_FWD, a, a_scale, b, b_scale, out, out_scale, group_lens, group_offs, G, M, N, K, dtype,
                       ep, Nc, ldo, swiglu_limit, workspace, workspace_bytes, s, nullptr, timing, nullptr, pitch);
    }
    return PT_ERR_UNSUPPORTED;
}

// ---------------------------------------------------------------- library-held scratch
// pt_grouped_gemm_fwd_noalloc keeps the forward's scratch -- the error word
// and the eight tile-queue counters, kQueueWsBytes bytes whatever the
// problem size -- in this array instead of a caller's workspace.  Every GPU
// the library runs on holds its own copy until the process ends.  The
// array's name is only a host-side stand-in: host code uses the device
// address hipGetSymbolAddress returns, fetched once per device with that
// device current.  The counters are zeroed on the stream at every call; the
// error bits accumulate there and are not reported.
constexpr size_t kScratchBytes = 4096;
static_assert((size_t)kQueueWsBytes <= kScratchBytes, "the forward's scratch must fit the static array");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[64] = {};

// Device address of this device's copy of `scratch` (looked up on the first
// call on each device).
static int scratch_address(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PT_ERR_HIP;
    if (dev < 0 || dev >= 64) return PT_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PT_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PT_OK;
}

extern "C" {

int pt_grouped_gemm_fwd(const void *a, const uint8_t *a_scale, const void *b, const uint8_t *b_scale,
                        void *out, uint8_t *out_scale, const int64_t *group_lens, const int64_t *group_offs,
                        int64_t G, int64_t M, int64_t N, int64_t K, int dtype, int trans_b, int epilogue,
                        float swiglu_limit, void *workspace, size_t workspace_bytes, void *stream)
{
    return grouped_fwd(a, a_scale, b, b_scale, out, out_scale, group_lens, group_offs, G, M, N, K, dtype, trans_b,
                       epilogue, swiglu_limit, workspace, workspace_bytes, stream, true);
}

int pt_grouped_gemm_fwd_pitched(const void *a, const uint8_t *a_scale, const void *b, const uint8_t *b_scale,
                                void *out, uint8_t *out_scale, const int64_t *group_lens,
                                const int64_t *group_offs, int64_t G, int64_t M, int64_t N, int64_t K, int dtype,
                                int epilogue, float swiglu_limit, int64_t code_pitch, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    if (code_pitch <= 0) return PT_ERR_INVALID_ARG;
    return grouped_fwd(a, a_scale, b, b_scale, out, out_scale, group_lens, group_offs, G, M, N, K, dtype, 1, epilogue,
                       swiglu_limit, workspace, workspace_bytes, stream, true, code_pitch);
}

int pt_grouped_gemm_fwd_noalloc(const void *a, const uint8_t *a_scale, const void *b, const uint8_t *b_scale,
                                void *out, uint8_t *out_scale, const int64_t *group_lens,
                                const int64_t *group_offs, int64_t G, int64_t M, int64_t N, int64_t K, int dtype,
                                int trans_b, int epilogue, float swiglu_limit, void *stream)
{
    // the scratch need does not grow with the problem: kQueueWsBytes always
    // fits kScratchBytes (static_assert above), so no size is refused for it
    void *ws = nullptr;
    const int st = scratch_address(&ws);
    if (st) return st;
    return grouped_fwd(a, a_scale, b, b_scale, out, out_scale, group_lens, group_offs, G, M, N, K, dtype, trans_b,
                       epilogue, swiglu_limit, ws, (size_t)kQueueWsBytes, stream, false);
}

int pt_grouped_gemm_dgrad(const void *dy, const uint8_t *dy_scale, const void *b, const uint8_t *b_scale, void *dx,
                          const int64_t *group_lens, const int64_t *group_offs, int64_t G, int64_t M, int64_t N,
                          int64_t K, int dtype, int trans_b, void *workspace, size_t workspace_bytes, void *stream)
{
    int st = check_groups(group_lens, G, M);
    if (st) return st;
    if (N < 1 || K < 1 || N > INT32_MAX / 4 || K > INT32_MAX / 4) return PT_ERR_INVALID_ARG;
    if (M > 0 && (!dy || !b || !dx)) return PT_ERR_INVALID_ARG;
    if (trans_b != 0 && trans_b != 1) return PT_ERR_INVALID_ARG;
    if (dtype == PT_MXFP8_E4M3 || dtype == PT_MXFP4_E2M1 || dtype == PT_FP8_E4M3 || dtype == PT_FP8_E4M3_ROWWISE) {
        // dY packed and scaled along N, and the weight's transposed copy
        // [G, K, N], packed and scaled along N (pt_mx_quantize_t): the MX
        // grouped GEMM with K outputs per row and a reduction over N.  FP8:
        // one factor for dY and one per expert's transposed weight, or one
        // per row of each (per output row and per output column)
        if (trans_b) return PT_ERR_UNSUPPORTED;
        if (!aligned16(dy) || !aligned16(b) || !aligned16(dx)) return PT_ERR_MISALIGNED;
        if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
        return mx_gemm(PT_OP_DGRAD, dy, dy_scale, b, b_scale, dx, nullptr, group_lens, group_offs, G, M, K, N, dtype,
                       kEpiNone, K, K, 0.0f, workspace, workspace_bytes, (hipStream_t)stream);
    }
    if (dtype != PT_BF16) return PT_ERR_UNSUPPORTED;
    if (dy_scale || b_scale) return PT_ERR_INVALID_ARG;
    if (N % 8 || K % 8) return PT_ERR_UNSUPPORTED;
    if (!fits31(M * N * 2) || !fits31(N * K * 2)) return PT_ERR_UNSUPPORTED;
    if (!aligned16(dy) || !aligned16(b) || !aligned16(dx)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    // dX[r, k] = sum_n dY[r, n] B[k, n]: reduction over n, output columns k.
    Bf16Params p = {};
    p.swiglu_limit = __builtin_huge_valf();
    p.a = (const uint16_t *)dy;
    p.b = (const uint16_t *)b;
    p.out = dx;
    p.lens = group_lens;
    p.offs = group_offs;
    p.err = error_word(workspace, workspace_bytes);
    p.G = (int)G;
    p.M = M;
    p.Kred = (int)N;
    p.Nout = (int)K;
    p.lda = (int)N;
    p.ldb = trans_b ? (int)K : (int)N;   // [G,K,N]: row k holds n contiguous
    p.b_gstride = N * K;
    p.ldo = (int)K;
    p.tilesN = (int)((K + bf16_tile_n() - 1) / bf16_tile_n());
    p.sched = queue_words(workspace, workspace_bytes);
    if (M == 0) return PT_OK;
    hipStream_t s = (hipStream_t)stream;
    uint32_t *queues = p.sched;
    const TuneKey key = tune_key(PT_OP_DGRAD, dtype, kEpiNone, trans_b, G, M, N, K);
    return configured(key, cfg_mask(queues != nullptr, true), true, s, [&](int cfg) {
        p.narrow = (cfg & kCfgNarrow) != 0;
        p.sched = (cfg & kCfgStatic) ? nullptr : queues;
        return queued(p.sched, s, [&] { return launch_bf16(p, trans_b ? kFwdNContig : kFwdKContig, kEpiNone, s); });
    });
}

int pt_grouped_gemm_fwd_swiglu_save(const void *a, const uint8_t *a_scale, const void *b, const uint8_t *b_scale,
                                    void *h, void *c, const int64_t *group_lens, const int64_t *group_offs, int64_t G,
                                    int64_t M, int64_t N, int64_t K, int dtype, int trans_b, float swiglu_limit,
                                    void *workspace, size_t workspace_bytes, void *stream)
{
    if (swiglu_limit != swiglu_limit) return PT_ERR_INVALID_ARG;   // NaN
    int st = check_groups(group_lens, G, M);
    if (st) return st;
    if (N < 1 || K < 1 || N > INT32_MAX / 4 || K > INT32_MAX / 4) return PT_ERR_INVALID_ARG;
    if (M > 0 && (!a || !b || !h || !c)) return PT_ERR_INVALID_ARG;
    if (trans_b != 0 && trans_b != 1) return PT_ERR_INVALID_ARG;
    if (N % 16 || K % 8) return PT_ERR_UNSUPPORTED;
    if (!fits31(M * N * 2)) return PT_ERR_UNSUPPORTED;
    if (!aligned16(a) || !aligned16(b) || !aligned16(h) || !aligned16(c)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    if (dtype == PT_MXFP8_E4M3 || dtype == PT_MXFP4_E2M1 || dtype == PT_FP8_E4M3 || dtype == PT_FP8_E4M3_ROWWISE) {
        if (!trans_b) return PT_ERR_UNSUPPORTED;           // K-contiguous codes
        return mx_gemm(PT_OP_FWD, a, a_scale, b, b_scale, h, nullptr, group_lens, group_offs, G, M, N, K, dtype,
                       kEpiSwigluSave, N / 2, N / 2, swiglu_limit, workspace, workspace_bytes, (hipStream_t)stream,
                       (uint16_t *)c);
    }
    if (dtype != PT_BF16) return PT_ERR_UNSUPPORTED;
    if (a_scale || b_scale) return PT_ERR_INVALID_ARG;
    if (!fits31(M * K * 2) || !fits31(N * K * 2)) return PT_ERR_UNSUPPORTED;
    Bf16Params p = {};
    p.swiglu_limit = swiglu_clamp(swiglu_limit);
    p.a = (const uint16_t *)a;
    p.b = (const uint16_t *)b;
    p.out = h;
    p.save = (uint16_t *)c;
    p.ldsave = (int)N;
    p.lens = group_lens;
    p.offs = group_offs;
    p.err = error_word(workspace, workspace_bytes);
    p.G = (int)G;
    p.M = M;
    p.Kred = (int)K;
    p.Nout = (int)N;
    p.lda = (int)K;
    p.ldb = trans_b ? (int)K : (int)N;
    p.b_gstride = N * K;
    p.ldo = (int)(N / 2);
    p.tilesN = (int)((N / 2 + bf16_tile_n() / 2 - 1) / (bf16_tile_n() / 2));
    p.sched = queue_words(workspace, workspace_bytes);
    if (M == 0) return PT_OK;
    hipStream_t s = (hipStream_t)stream;
    uint32_t *queues = p.sched;
    const TuneKey key = tune_key(PT_OP_FWD, PT_BF16, kEpiSwigluSave, trans_b, G, M, N, K);
    return configured(key, cfg_mask(queues != nullptr, false), true, s, [&](int cfg) {
        p.sched = (cfg & kCfgStatic) ? nullptr : queues;
        return queued(p.sched, s, [&] { return launch_bf16(p, trans_b ? kFwdKContig : kFwdNContig, kEpiSwigluSave, s); });
    });
}

int pt_grouped_gemm_dgrad_swiglu(const void *dy, const uint8_t *dy_scale, const void *b, const uint8_t *b_scale,
                                 const void *c_saved, void *dc, const int64_t *group_lens,
                                 const int64_t *group_offs, int64_t G, int64_t M, int64_t N, int64_t K, int dtype,
                                 int trans_b, float swiglu_limit, void *workspace, size_t workspace_bytes,
                                 void *stream)
{
    if (swiglu_limit != swiglu_limit) return PT_ERR_INVALID_ARG;   // NaN
    int st = check_groups(group_lens, G, M);
    if (st) return st;
    if (N < 1 || K < 1 || N > INT32_MAX / 4 || K > INT32_MAX / 8) return PT_ERR_INVALID_ARG;
    if (M > 0 && (!dy || !b || !c_saved || !dc)) return PT_ERR_INVALID_ARG;
    if (trans_b != 0 && trans_b != 1) return PT_ERR_INVALID_ARG;
    if (N % 8 || K % 8) return PT_ERR_UNSUPPORTED;
    if (!fits31(M * N * 2) || !fits31(N * K * 2)) return PT_ERR_UNSUPPORTED;
    if (!aligned16(dy) || !aligned16(b) || !aligned16(c_saved) || !aligned16(dc)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    if (dtype == PT_MXFP8_E4M3 || dtype == PT_MXFP4_E2M1 || dtype == PT_FP8_E4M3 || dtype == PT_FP8_E4M3_ROWWISE) {
        // dH as pt_grouped_gemm_dgrad computes it for the dtype (dY packed
        // and scaled along N, the weight's transposed cache [G, K, N]), then
        // the same SwiGLU-backward epilogue
        if (trans_b) return PT_ERR_UNSUPPORTED;
        return mx_gemm(PT_OP_DGRAD_SWIGLU, dy, dy_scale, b, b_scale, dc, nullptr, group_lens, group_offs, G, M, K, N,
                       dtype, kEpiDSwiglu, K, 2 * K, swiglu_limit, workspace, workspace_bytes, (hipStream_t)stream,
                       nullptr, true, (const uint16_t *)c_saved);
    }
    if (dtype != PT_BF16) return PT_ERR_UNSUPPORTED;
    if (dy_scale || b_scale) return PT_ERR_INVALID_ARG;
    // dH[r, k] = sum_n dY[r, n] B[k, n] as in pt_grouped_gemm_dgrad; the
    // epilogue turns each bf16 dH tile into the [gate | up] gradient.
    Bf16Params p = {};
    p.swiglu_limit = __builtin_huge_valf();
    p.a = (const uint16_t *)dy;
    p.b = (const uint16_t *)b;
    p.out = dc;
    p.lens = group_lens;
    p.offs = group_offs;
    p.err = error_word(workspace, workspace_bytes);
    p.G = (int)G;
    p.M = M;
    p.Kred = (int)N;
    p.Nout = (int)K;
    p.lda = (int)N;
    p.ldb = trans_b ? (int)K : (int)N;
    p.b_gstride = N * K;
    p.ldo = (int)(2 * K);
    p.aux = (const uint16_t *)c_saved;
    p.swiglu_limit = swiglu_clamp(swiglu_limit);
    p.ldaux = (int)(2 * K);
    p.tilesN = (int)((K + bf16_tile_n() - 1) / bf16_tile_n());
    p.sched = queue_words(workspace, workspace_bytes);
    if (M == 0) return PT_OK;
    hipStream_t s = (hipStream_t)stream;
    uint32_t *queues = p.sched;
    const TuneKey key = tune_key(PT_OP_DGRAD_SWIGLU, PT_BF16, kEpiDSwiglu, trans_b, G, M, N, K);
    return configured(key, cfg_mask(queues != nullptr, false), true, s, [&](int cfg) {
        p.sched = (cfg & kCfgStatic) ? nullptr : queues;
        return queued(p.sched, s, [&] { return launch_bf16(p, trans_b ? kFwdNContig : kFwdKContig, kEpiDSwiglu, s); });
    });
}

// The MX weight gradient's workspace: the error word and queues, the
// experts' plan (block and stage starts), both gradients' transposed codes
// and their stage-major scale words.
struct MxWgradWs {
    int64_t pitch, stages, plan, qa, qd, sa, sd, total;
};
MxWgradWs mx_wgrad_ws(int64_t G, int64_t M, int64_t N, int64_t K, int fmt)
{
    MxWgradWs w;
    w.pitch = mx_wgrad_pitch(M, (int)G, fmt);
    w.stages = mx_wgrad_stages(M, (int)G, fmt);
    const int64_t wpr = fmt == 0 ? 1 : 2;
    w.plan = kQueueWsBytes;
    w.qa = w.plan + round256(8 * G);
    w.qd = w.qa + round256(K * w.pitch);
    w.sa = w.qd + round256(N * w.pitch);
    w.sd = w.sa + round256(w.stages * K * wpr * 4);
    w.total = w.sd + round256(w.stages * N * wpr * 4);
    return w;
}

// The BF16 weight gradient (also the second half of the FP8 one);
// its split reduction's partial slots start split_off bytes into the
// workspace.
static int bf16_wgrad(const void *a, const void *dy, float *main_grad, const int64_t *group_lens,
                      const int64_t *group_offs, int64_t G, int64_t M, int64_t N, int64_t K, int trans_out,
                      int accumulate, void *workspace, size_t workspace_bytes, size_t split_off, hipStream_t s)
{
    if (!aligned16(a) || !aligned16(dy) || !aligned16(main_grad)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    Bf16Params p = {};
    p.swiglu_limit = __builtin_huge_valf();
    // trans_out = 0: D[k, n] = sum_r A[r, k] dY[r, n];  1: D^T[n, k] with the
    // operands swapped
    p.a = (const uint16_t *)(trans_out ? dy : a);
    p.b = (const uint16_t *)(trans_out ? a : dy);
    p.lda = (int)(trans_out ? N : K);
    p.ldb = (int)(trans_out ? K : N);
    p.Mout = (int)(trans_out ? N : K);
    p.Nout = (int)(trans_out ? K : N);
    p.out = main_grad;
    p.ldo = p.Nout;
    p.o_gstride = N * K;
    p.lens = group_lens;
    p.offs = group_offs;
    p.err = error_word(workspace, workspace_bytes);
    p.G = (int)G;
    p.M = M;
    p.tilesN = (p.Nout + bf16_tile_n() - 1) / bf16_tile_n();
    p.accumulate = accumulate;
    if (M == 0 && accumulate) return PT_OK;
    uint32_t *queues = queue_words(workspace, workspace_bytes);
    // the split reduction, when the workspace holds its partial slots
    const int64_t split_len = wgrad_split_len(M, p.Mout, p.Nout);
    const int64_t nslots = wgrad_split_slots(M, p.Mout, p.Nout);
    const bool split = queues && aligned16(workspace) && nslots > 0 &&
                       workspace_bytes >= split_off + (size_t)wgrad_split_bytes(M, K, N);
    if (split) {
        p.split_len = (int)split_len;
        p.nslots = (int)nslots;
        p.partials = (float *)((uint8_t *)workspace + split_off);
    }
    const TuneKey key = tune_key(PT_OP_WGRAD, PT_BF16, kEpiNone, trans_out, G, M, N, K);
    return configured(key, cfg_mask(queues != nullptr, !split), !accumulate, s, [&](int cfg) {
        p.narrow = (cfg & kCfgNarrow) != 0;
        p.sched = (cfg & kCfgStatic) ? nullptr : queues;
        p.tilesM = (p.Mout + bf16_tile_m(p.narrow) - 1) / bf16_tile_m(p.narrow);
        hipError_t e = queued(p.sched, s, [&] { return launch_bf16(p, kWgrad, kEpiNone, s); });
        if (e == hipSuccess && split) e = launch_wgrad_split_reduce(p, s);
        return e;
    });
}


// The MX weight gradient on operands already in the workspace (channel rows
// and stage-major scale words of both gradients, and the experts' plan):
// the 256 x 256 MX kernel reduces over each expert's tokens with the block
// scales applied in the matrix cores, optionally split along tokens.
static int mx_wgrad_gemm(const MxWgradWs &w, uint8_t *base, int dtype, float *main_grad, const int64_t *group_lens,
                         const int64_t *group_offs, int64_t G, int64_t M, int64_t N, int64_t K, int trans_out,
                         int accumulate, void *workspace, size_t workspace_bytes, hipStream_t s)
{
    const int fmt = dtype == PT_MXFP8_E4M3 ? 0 : 1;
    int *plan = (int *)(base + w.plan);
    uint8_t *qa = base + w.qa, *qd = base + w.qd;
    uint32_t *sa = (uint32_t *)(base + w.sa), *sd = (uint32_t *)(base + w.sd);
    // trans_out = 0: rows are A's channels (K), columns dY's (N); 1: swapped
    MxParams p = {};
    p.a = trans_out ? qd : qa;
    p.sa = trans_out ? sd : sa;
    p.b = trans_out ? qa : qd;
    p.sb = trans_out ? sa : sd;
    p.wrows = (int)(trans_out ? N : K);
    p.wcols = (int)(trans_out ? K : N);
    p.pitch = w.pitch;
    p.plan = plan;
    p.out = main_grad;
    p.ldo = p.wcols;
    p.o_gstride = N * K;
    p.tilesM = (p.wrows + mx_wide_tile() - 1) / mx_wide_tile();
    p.tilesN = (p.wcols + mx_wide_tile() - 1) / mx_wide_tile();
    p.accumulate = accumulate;
    p.lens = group_lens;
    p.offs = group_offs;
    p.err = error_word(workspace, workspace_bytes);
    p.G = (int)G;
    p.M = M;
    p.K = 32;
    p.N = p.wcols;
    p.swiglu_limit = __builtin_huge_valf();
    uint32_t *queues = queue_words(workspace, workspace_bytes);
    // the split reduction, when the workspace holds its partial slots: the
    // chunk length of the BF16 rule rounded up to whole 256-token stages
    const int64_t split_len = (wgrad_split_len(M, p.wrows, p.wcols) + 255) / 256 * 256;
    const int64_t nslots = M / split_len;
    Bf16Params rp = {};
    if (queues && nslots > 0 && workspace_bytes >= (size_t)(w.total + wgrad_split_bytes(M, K, N))) {
        p.split_len = (int)split_len;
        p.nslots = (int)nslots;
        p.partials = (float *)(base + w.total);
        rp.lens = group_lens;
        rp.offs = group_offs;
        rp.G = (int)G;
        rp.M = M;
        rp.split_len = p.split_len;
        rp.nslots = p.nslots;
        rp.partials = p.partials;
        rp.out = main_grad;
        rp.o_gstride = N * K;
        rp.Mout = p.wrows;
        rp.Nout = p.wcols;
        rp.accumulate = accumulate;
    }
    const TuneKey key = tune_key(PT_OP_WGRAD, dtype, kEpiWgrad, trans_out, G, M, N, K);
    return configured(key, cfg_mask(queues != nullptr, false), false, s, [&](int cfg) {
        p.sched = (cfg & kCfgStatic) ? nullptr : queues;
        hipError_t e2 = queued(p.sched, s, [&] { return launch_mx_wgrad(p, fmt, s); });
        if (e2 == hipSuccess && p.split_len > 0) e2 = launch_wgrad_split_reduce(rp, s);
        return e2;
    });
}

// The FP8 weight gradient with one factor per tensor on operands already in
// the workspace (both gradients' codes as channel rows, the experts' plan);
// fa, fd: the two dequantisation factors (device).
static int fp8_wgrad_gemm(const MxWgradWs &w, uint8_t *base, const float *fa, const float *fd, float *main_grad,
                          const int64_t *group_lens, const int64_t *group_offs, int64_t G, int64_t M, int64_t N,
                          int64_t K, int trans_out, int accumulate, void *workspace, size_t workspace_bytes,
                          hipStream_t s)
{
    int *plan = (int *)(base + w.plan);
    uint8_t *qa = base + w.qa, *qd = base + w.qd;
    MxParams p = {};
    p.a = trans_out ? qd : qa;
    p.b = trans_out ? qa : qd;
    p.sfa = fa;
    p.sfb = fd;
    p.wrows = (int)(trans_out ? N : K);
    p.wcols = (int)(trans_out ? K : N);
    p.pitch = w.pitch;
    p.plan = plan;
    p.out = main_grad;
    p.ldo = p.wcols;
    p.o_gstride = N * K;
    p.tilesM = (p.wrows + mx_wide_tile() - 1) / mx_wide_tile();
    p.tilesN = (p.wcols + mx_wide_tile() - 1) / mx_wide_tile();
    p.accumulate = accumulate;
    p.lens = group_lens;
    p.offs = group_offs;
    p.err = error_word(workspace, workspace_bytes);
    p.G = (int)G;
    p.M = M;
    p.K = 32;
    p.N = p.wcols;
    p.swiglu_limit = __builtin_huge_valf();
    uint32_t *queues = queue_words(workspace, workspace_bytes);
    const TuneKey key = tune_key(PT_OP_WGRAD, PT_FP8_E4M3, kEpiWgrad, trans_out, G, M, N, K);
    return configured(key, cfg_mask(queues != nullptr, false), false, s, [&](int cfg) {
        p.sched = (cfg & kCfgStatic) ? nullptr : queues;
        return queued(p.sched, s, [&] { return launch_mx_wgrad(p, 2, s); });
    });
}

int pt_grouped_gemm_wgrad(const void *a, const uint8_t *a_scale, const void *dy, const uint8_t *dy_scale,
                          float *main_grad, const int64_t *group_lens, const int64_t *group_offs, int64_t G,
                          int64_t M, int64_t N, int64_t K, int dtype, int trans_out, int accumulate,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    int st = check_groups(group_lens, G, M);
    if (st) return st;
    if (N < 8 || K < 8 || N > INT32_MAX / 4 || K > INT32_MAX / 4) return PT_ERR_INVALID_ARG;
    if (!main_grad || (M > 0 && (!a || !dy))) return PT_ERR_INVALID_ARG;
    if (trans_out != 0 && trans_out != 1) return PT_ERR_INVALID_ARG;
    if (accumulate != 0 && accumulate != 1) return PT_ERR_INVALID_ARG;
    if (N % 8 || K % 8) return PT_ERR_UNSUPPORTED;
    if (!fits31(M * K * 2) || !fits31(M * N * 2)) return PT_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == PT_MXFP8_E4M3 || dtype == PT_MXFP4_E2M1) {
        // codes blocked along tokens (pt_mx_quantize_tokens): both are
        // transposed into the workspace (channel rows, each expert's tokens
        // padded to whole blocks; stage-major scales), and the 256 x 256 MX
        // kernel reduces over each expert's tokens with the block scales
        // applied in the matrix cores
        const int fmt = dtype == PT_MXFP8_E4M3 ? 0 : 1;
        if (M > 0 && (!a_scale || !dy_scale)) return PT_ERR_INVALID_ARG;
        if (!aligned16(a) || !aligned16(dy) || !aligned16(main_grad) || !aligned16(a_scale) || !aligned16(dy_scale))
            return PT_ERR_MISALIGNED;
        if (M == 0 && accumulate) return PT_OK;
        if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
        const MxWgradWs w = mx_wgrad_ws(G, M, N, K, fmt);
        if (!fits31(K * w.pitch) || !fits31(N * w.pitch) || !fits31(w.stages * (K + N) * 8))
            return PT_ERR_UNSUPPORTED;
        if (!workspace || !aligned16(workspace) || workspace_bytes < (size_t)w.total) return PT_ERR_WORKSPACE;
        uint8_t *base = (uint8_t *)workspace;
        int *plan = (int *)(base + w.plan);
        uint8_t *qa = base + w.qa, *qd = base + w.qd;
        uint32_t *sa = (uint32_t *)(base + w.sa), *sd = (uint32_t *)(base + w.sd);
        hipError_t e = launch_mx_tokens_transpose((const uint8_t *)a, a_scale, group_lens, group_offs, (int)G, M, K,
                                                  fmt, qa, w.pitch, sa, plan, s);
        if (e == hipSuccess)
            e = launch_mx_tokens_transpose((const uint8_t *)dy, dy_scale, group_lens, group_offs, (int)G, M, N, fmt,
                                           qd, w.pitch, sd, plan, s);
        if (e != hipSuccess) return PT_ERR_HIP;
        return mx_wgrad_gemm(w, base, dtype, main_grad, group_lens, group_offs, G, M, N, K, trans_out, accumulate,
                             workspace, workspace_bytes, s);
    }
    if (dtype == PT_FP8_E4M3) {
        // one factor per tensor: both gradients' codes are transposed into
        // the workspace as for MXFP8 (channel rows, each expert's tokens
        // padded to whole 32-token blocks, no block scales), the MX kernel
        // sums exact code products in fp32 (unit block scales), and its
        // epilogue adds fp32(d_a * d_dy) * sum into main_grad by one fused
        // multiply-add per element.  Experts are not split along tokens here:
        // the factor scales each expert's whole sum before main_grad is added.
        if (M == 0) return bf16_wgrad(nullptr, nullptr, main_grad, group_lens, group_offs, G, M, N, K, trans_out,
                                      accumulate, workspace, workspace_bytes, kQueueWsBytes, s);
        if (!a_scale || !dy_scale) return PT_ERR_INVALID_ARG;
        if (!aligned16(a) || !aligned16(dy) || !aligned16(main_grad) || !aligned4(a_scale) || !aligned4(dy_scale))
            return PT_ERR_MISALIGNED;
        if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
        const MxWgradWs w = mx_wgrad_ws(G, M, N, K, 0);
        if (!fits31(K * w.pitch) || !fits31(N * w.pitch)) return PT_ERR_UNSUPPORTED;
        if (!workspace || !aligned16(workspace) || workspace_bytes < (size_t)w.sa) return PT_ERR_WORKSPACE;
        uint8_t *base = (uint8_t *)workspace;
        int *plan = (int *)(base + w.plan);
        uint8_t *qa = base + w.qa, *qd = base + w.qd;
        hipError_t e = launch_mx_tokens_transpose((const uint8_t *)a, nullptr, group_lens, group_offs, (int)G, M, K,
                                                  0, qa, w.pitch, nullptr, plan, s);
        if (e == hipSuccess)
            e = launch_mx_tokens_transpose((const uint8_t *)dy, nullptr, group_lens, group_offs, (int)G, M, N, 0, qd,
                                           w.pitch, nullptr, plan, s);
        if (e != hipSuccess) return PT_ERR_HIP;
        return fp8_wgrad_gemm(w, base, (const float *)a_scale, (const float *)dy_scale, main_grad, group_lens,
                              group_offs, G, M, N, K, trans_out, accumulate, workspace, workspace_bytes, s);
    }
    if (dtype != PT_BF16) return PT_ERR_UNSUPPORTED;
    if (a_scale || dy_scale) return PT_ERR_INVALID_ARG;
    return bf16_wgrad(a, dy, main_grad, group_lens, group_offs, G, M, N, K, trans_out, accumulate, workspace,
                      workspace_bytes, kQueueWsBytes, s);
}

// Bytes the FP8 weight gradient with tensor factors keeps after its
// operands: the two amax words and the two dequantisation factors.
constexpr int64_t kFp8WgradTail = 256;

int pt_grouped_gemm_wgrad_quantize(const void *a, const void *dy, float *main_grad, const int64_t *group_lens,
                                   const int64_t *group_offs, int64_t G, int64_t M, int64_t N, int64_t K, int dtype,
                                   int trans_out, int accumulate, void *workspace, size_t workspace_bytes,
                                   void *stream)
{
    int st = check_groups(group_lens, G, M);
    if (st) return st;
    if (N < 8 || K < 8 || N > INT32_MAX / 4 || K > INT32_MAX / 4) return PT_ERR_INVALID_ARG;
    if (!main_grad || (M > 0 && (!a || !dy))) return PT_ERR_INVALID_ARG;
    if (trans_out != 0 && trans_out != 1) return PT_ERR_INVALID_ARG;
    if (accumulate != 0 && accumulate != 1) return PT_ERR_INVALID_ARG;
    if (dtype != PT_MXFP8_E4M3 && dtype != PT_MXFP4_E2M1 && dtype != PT_FP8_E4M3) return PT_ERR_UNSUPPORTED;
    if (N % 8 || K % 8) return PT_ERR_UNSUPPORTED;
    if (!fits31(M * K * 2) || !fits31(M * N * 2)) return PT_ERR_UNSUPPORTED;
    if (!aligned16(a) || !aligned16(dy) || !aligned16(main_grad)) return PT_ERR_MISALIGNED;
    if (M == 0 && accumulate) return PT_OK;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const bool fp8 = dtype == PT_FP8_E4M3;
    if (fp8 && M == 0)
        return bf16_wgrad(nullptr, nullptr, main_grad, group_lens, group_offs, G, M, N, K, trans_out, accumulate,
                          workspace, workspace_bytes, kQueueWsBytes, s);
    const int fmt = dtype == PT_MXFP4_E2M1 ? 1 : 0;
    const MxWgradWs w = mx_wgrad_ws(G, M, N, K, fmt);
    if (!fits31(K * w.pitch) || !fits31(N * w.pitch) || (!fp8 && !fits31(w.stages * (K + N) * 8)))
        return PT_ERR_UNSUPPORTED;
    const int64_t need = fp8 ? w.sa + kFp8WgradTail : w.total;
    if (!workspace || !aligned16(workspace) || workspace_bytes < (size_t)need) return PT_ERR_WORKSPACE;
    uint8_t *base = (uint8_t *)workspace;
    int *plan = (int *)(base + w.plan);
    // both gradients quantised along tokens straight into the operand layout
    // of the weight gradient (the GEMM validates the lengths itself); FP8:
    // each tensor's amax first, then its codes with the factor of
    // pt_fp8_quantize
    uint32_t *amax = fp8 ? (uint32_t *)(base + w.sa) : nullptr;
    float *deq = fp8 ? (float *)(base + w.sa + 16) : nullptr;
    hipError_t e = hipSuccess;
    if (fp8) {
        e = launch_fp8_amax((const uint16_t *)a, amax, M * K, s);
        if (e == hipSuccess) e = launch_fp8_amax((const uint16_t *)dy, amax + 1, M * N, s);
    }
    if (e == hipSuccess)
        e = launch_mx_tokens_quant_t((const uint16_t *)a, group_lens, group_offs, (int)G, M, K, fp8 ? 2 : fmt,
                                     base + w.qa, w.pitch, fp8 ? nullptr : (uint32_t *)(base + w.sa), plan, nullptr,
                                     amax, deq, s);
    if (e == hipSuccess)
        e = launch_mx_tokens_quant_t((const uint16_t *)dy, group_lens, group_offs, (int)G, M, N, fp8 ? 2 : fmt,
                                     base + w.qd, w.pitch, fp8 ? nullptr : (uint32_t *)(base + w.sd), plan, nullptr,
                                     fp8 ? amax + 1 : nullptr, fp8 ? deq + 1 : nullptr, s);
    if (e != hipSuccess) return PT_ERR_HIP;
    if (fp8)
        return fp8_wgrad_gemm(w, base, deq, deq + 1, main_grad, group_lens, group_offs, G, M, N, K, trans_out,
                              accumulate, workspace, workspace_bytes, s);
    return mx_wgrad_gemm(w, base, dtype, main_grad, group_lens, group_offs, G, M, N, K, trans_out, accumulate,
                         workspace, workspace_bytes, s);
}

int pt_mx_quantize(const void *x, void *q, uint8_t *scales, int64_t rows, int64_t cols, int dtype, int axis,
                   void *stream)
{
    if (rows < 0 || cols < 0) return PT_ERR_INVALID_ARG;
    if (axis != 0 && axis != 1) return PT_ERR_INVALID_ARG;
    if (dtype != PT_MXFP8_E4M3 && dtype != PT_MXFP4_E2M1) return PT_ERR_UNSUPPORTED;
    if (axis == 1 && cols % 32) return PT_ERR_UNSUPPORTED;
    if (axis == 0 && (rows % 32 || cols % 8)) return PT_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return PT_OK;
    if (!x || !q || !scales) return PT_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q)) return PT_ERR_MISALIGNED;
    if (axis == 0 && !aligned4(scales)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    const int fmt = dtype == PT_MXFP8_E4M3 ? 0 : 1;
    if (axis == 0)
        return hip_status(launch_quantize_cols((const uint16_t *)x, (uint8_t *)q, scales, rows, cols, fmt,
                                               (hipStream_t)stream));
    return hip_status(launch_quantize((const uint16_t *)x, (uint8_t *)q, scales, rows, cols, fmt,
                                      (hipStream_t)stream));
}

int pt_mx_quantize_pitched(const void *x, void *q, uint8_t *scales, int64_t rows, int64_t cols, int dtype,
                           int64_t q_pitch, void *stream)
{
    if (rows < 0 || cols < 0) return PT_ERR_INVALID_ARG;
    if (dtype != PT_MXFP8_E4M3 && dtype != PT_MXFP4_E2M1) return PT_ERR_UNSUPPORTED;
    if (cols % 32) return PT_ERR_UNSUPPORTED;
    const int fmt = dtype == PT_MXFP8_E4M3 ? 0 : 1;
    if (q_pitch < (fmt == 0 ? cols : cols / 2) || q_pitch % 16) return PT_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return PT_OK;
    if (!x || !q || !scales) return PT_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    return hip_status(launch_quantize((const uint16_t *)x, (uint8_t *)q, scales, rows, cols, fmt,
                                      (hipStream_t)stream, q_pitch));
}

int pt_fp8_quantize(const void *x, void *q, float *amax, float *dequant, int64_t batch, int64_t rows, int64_t cols,
                    void *stream)
{
    if (batch < 0 || rows < 0 || cols < 0 || batch > 65535) return PT_ERR_INVALID_ARG;
    if (cols % 8) return PT_ERR_UNSUPPORTED;
    if (batch == 0) return PT_OK;
    if (!amax || !dequant || ((rows > 0 && cols > 0) && (!x || !q))) return PT_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q) || !aligned4(amax) || !aligned4(dequant)) return PT_ERR_MISALIGNED;
    if (!fits31(rows * cols / 8)) return PT_ERR_UNSUPPORTED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    return hip_status(launch_fp8_quantize((const uint16_t *)x, (uint8_t *)q, amax, dequant, batch, rows * cols,
                                          (hipStream_t)stream));
}

int pt_mx_quantize_tokens(const void *x, const int64_t *group_lens, const int64_t *group_offs, void *q,
                          uint8_t *scales, int64_t G, int64_t M, int64_t cols, int dtype, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    int st = check_groups(group_lens, G, M);
    if (st) return st;
    if (cols < 0) return PT_ERR_INVALID_ARG;
    if (dtype != PT_MXFP8_E4M3 && dtype != PT_MXFP4_E2M1) return PT_ERR_UNSUPPORTED;
    if (cols % 8 || M / 32 + G > INT32_MAX) return PT_ERR_UNSUPPORTED;
    if (M == 0 || cols == 0) return PT_OK;
    if (!x || !q || !scales) return PT_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q) || !aligned16(scales)) return PT_ERR_MISALIGNED;
    if (!fits31(M * cols)) return PT_ERR_UNSUPPORTED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    return hip_status(launch_mx_quantize_tokens((const uint16_t *)x, group_lens, group_offs, (int)G, M, cols,
                                                dtype == PT_MXFP8_E4M3 ? 0 : 1, (uint8_t *)q, scales,
                                                error_word(workspace, workspace_bytes), (hipStream_t)stream));
}

int pt_fp8_quantize_rows(const void *x, void *q, float *amax, float *dequant, int64_t rows, int64_t cols,
                         void *stream)
{
    if (rows < 0 || cols < 0) return PT_ERR_INVALID_ARG;
    if (cols % 8) return PT_ERR_UNSUPPORTED;
    if (rows == 0) return PT_OK;
    if (!amax || !dequant || (cols > 0 && (!x || !q))) return PT_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q) || !aligned4(amax) || !aligned4(dequant)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    if (cols == 0) return PT_OK;
    return hip_status(launch_fp8_quantize_rows((const uint16_t *)x, (uint8_t *)q, amax, dequant, rows, cols,
                                               (hipStream_t)stream));
}

int pt_mx_quantize_t(const void *x, void *q, uint8_t *scales, int64_t batch, int64_t rows, int64_t cols, int dtype,
                     void *stream)
{
    if (batch < 0 || rows < 0 || cols < 0 || batch > 65535) return PT_ERR_INVALID_ARG;
    if (dtype != PT_MXFP8_E4M3 && dtype != PT_MXFP4_E2M1) return PT_ERR_UNSUPPORTED;
    if (rows % 32 || cols % 8) return PT_ERR_UNSUPPORTED;
    if (batch == 0 || rows == 0 || cols == 0) return PT_OK;
    if (!x || !q || !scales) return PT_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    return hip_status(launch_quantize_t((const uint16_t *)x, (uint8_t *)q, scales, batch, rows, cols,
                                        dtype == PT_MXFP8_E4M3 ? 0 : 1, (hipStream_t)stream));
}

int pt_stack_experts(const void *const *experts, void *out, int64_t G, int64_t rows, int64_t cols, int transpose,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    if (G < 0 || rows < 0 || cols < 0 || (transpose != 0 && transpose != 1)) return PT_ERR_INVALID_ARG;
    if (G > 65535 || rows % 8 || cols % 8) return PT_ERR_UNSUPPORTED;
    if (G == 0 || rows == 0 || cols == 0) return PT_OK;
    if (!experts || !out) return PT_ERR_INVALID_ARG;
    if (!aligned16(out) || ((uintptr_t)experts & 7)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    return hip_status(launch_stack_experts(experts, (uint16_t *)out, (int)G, rows, cols, transpose,
                                           error_word(workspace, workspace_bytes), (hipStream_t)stream));
}

int pt_mx_quantize_experts(const void *const *experts, void *q, uint8_t *scales, void *q_t, uint8_t *scales_t,
                           int64_t G, int64_t rows, int64_t cols, int dtype, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    if (G < 0 || rows < 0 || cols < 0) return PT_ERR_INVALID_ARG;
    if ((q == nullptr) != (scales == nullptr) || (q_t == nullptr) != (scales_t == nullptr)) return PT_ERR_INVALID_ARG;
    if (!q && !q_t) return PT_ERR_INVALID_ARG;
    if (dtype != PT_MXFP8_E4M3 && dtype != PT_MXFP4_E2M1) return PT_ERR_UNSUPPORTED;
    if (G > 65535 || rows % 8 || cols % 8 || (q && cols % 32) || (q_t && rows % 32)) return PT_ERR_UNSUPPORTED;
    if (G == 0 || rows == 0 || cols == 0) return PT_OK;
    if (!experts) return PT_ERR_INVALID_ARG;
    if ((q && !aligned16(q)) || (q_t && !aligned16(q_t)) || ((uintptr_t)experts & 7)) return PT_ERR_MISALIGNED;
    if (!device_is_gfx950()) return PT_ERR_UNSUPPORTED;
    return hip_status(launch_mx_quantize_experts(experts, (uint8_t *)q, scales, (uint8_t *)q_t, scales_t, (int)G,
                                                 rows, cols, dtype == PT_MXFP8_E4M3 ? 0 : 1,
                                                 error_word(workspace, workspace_bytes), (hipStream_t)stream));
}

size_t pt_grouped_gemm_workspace_size(int op, int64_t G, int64_t M, int64_t N, int64_t K, int dtype)
{
    // the error word and the tile-queue counters; for an MX forward also the
    // stage-major copies of the A and B scales
    if (op == PT_OP_FWD && (dtype == PT_MXFP8_E4M3 || dtype == PT_MXFP4_E2M1) && G > 0 && M >= 0 && N > 0 &&
        K > 0 && K % 32 == 0) {
        const int fmt = dtype == PT_MXFP8_E4M3 ? 0 : 1;
        if (mx_swz_possible(G, M, N, K, fmt))
            return (size_t)(kQueueWsBytes + mx_swz_a_bytes(M, K, fmt) + mx_swz_b_bytes(G, N, K, fmt));
    }
    // the weight gradients: the split reduction's partial slots last; before
    // them the experts' plan and both gradients' transposed codes and
    // stage-major scale words (MX)
    if (op == PT_OP_WGRAD && (dtype == PT_MXFP8_E4M3 || dtype == PT_MXFP4_E2M1) && M >= 0 && N > 0 && K > 0 &&
        G > 0)
        return (size_t)(mx_wgrad_ws(G, M, N, K, dtype == PT_MXFP8_E4M3 ? 0 : 1).total + wgrad_split_bytes(M, K, N));
    // FP8 with tensor factors: the plan and both gradients' transposed codes
    if (op == PT_OP_WGRAD && dtype == PT_FP8_E4M3 && M > 0 && N > 0 && K > 0 && G > 0)
        return (size_t)(mx_wgrad_ws(G, M, N, K, 0).sa + kFp8WgradTail);
    if (op == PT_OP_WGRAD && M > 0 && N > 0 && K > 0 && G > 0)
        return (size_t)(kQueueWsBytes + wgrad_split_bytes(M, K, N));
    // the MX data gradient: K outputs per row, a reduction over N
    if ((op == PT_OP_DGRAD || op == PT_OP_DGRAD_SWIGLU) && (dtype == PT_MXFP8_E4M3 || dtype == PT_MXFP4_E2M1) &&
        G > 0 && M >= 0 && N > 0 &&
        K > 0 && N % 32 == 0) {
        const int fmt = dtype == PT_MXFP8_E4M3 ? 0 : 1;
        if (mx_swz_possible(G, M, K, N, fmt))
            return (size_t)(kQueueWsBytes + mx_swz_a_bytes(M, N, fmt) + mx_swz_b_bytes(G, K, N, fmt));
    }
    return kQueueWsBytes;
}

int pt_set_gemm_config(int config)
{
    if (config != PT_CONFIG_RULES && config != PT_CONFIG_TUNE && (config < 0 || config >= kNumCfg)) return -3;
    return g_mode.exchange(config);
}

int pt_gemm_config_of(int op, int dtype, int epilogue, int trans, int64_t G, int64_t M, int64_t N, int64_t K)
{
    // the classes as the entry points record them
    switch (op) {
    case PT_OP_FWD: {
        const int ep =
            epilogue == PT_EPI_SWIGLU ? kEpiSwiglu : epilogue == PT_EPI_SWIGLU_MXFP4 ? kEpiSwigluMxfp4 : kEpiNone;
        return tune_lookup(tune_key(op, dtype, ep, dtype == PT_BF16 ? trans : 0, G, M, N, K));
    }
    case PT_OP_DGRAD:      // the MX / FP8 data gradient runs as a GEMM with K outputs over N
        if (dtype == PT_BF16) return tune_lookup(tune_key(op, dtype, kEpiNone, trans, G, M, N, K));
        return tune_lookup(tune_key(op, dtype, kEpiNone, 0, G, M, K, N));
    case PT_OP_WGRAD:      // the MX weight gradient has its own class; the others run the BF16 kernel
        if (dtype == PT_MXFP8_E4M3 || dtype == PT_MXFP4_E2M1)
            return tune_lookup(tune_key(op, dtype, kEpiWgrad, trans, G, M, N, K));
        return tune_lookup(tune_key(op, PT_BF16, kEpiNone, trans, G, M, N, K));
    case PT_OP_DGRAD_SWIGLU:
        if (dtype == PT_BF16) return tune_lookup(tune_key(op, PT_BF16, kEpiDSwiglu, trans, G, M, N, K));
        return tune_lookup(tune_key(op, dtype, kEpiDSwiglu, 0, G, M, K, N));
    default:
        return -1;
    }
}

void pt_clear_gemm_tuning(void)
{
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_ntune = 0;
}

int pt_read_error_flags(const void *workspace, void *stream, uint32_t *flags)
{
    if (!workspace || !flags) return PT_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (hipStreamSynchronize(s) != hipSuccess) return PT_ERR_HIP;
    if (hipMemcpy(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return PT_ERR_HIP;
    return PT_OK;
}

const char *pt_status_string(int status)
{
    switch (status) {
    case PT_OK: return "PT_OK";
    case PT_ERR_INVALID_ARG: return "PT_ERR_INVALID_ARG";
    case PT_ERR_UNSUPPORTED: return "PT_ERR_UNSUPPORTED";
    case PT_ERR_MISALIGNED: return "PT_ERR_MISALIGNED";
    case PT_ERR_WORKSPACE: return "PT_ERR_WORKSPACE";
    case PT_ERR_HIP: return "PT_ERR_HIP";
    default: return "PT_ERR_UNKNOWN";
    }
}

const char *pt_version(void) { return "ptgg 0.1.0 (gfx950)"; }

}  // extern "C"
