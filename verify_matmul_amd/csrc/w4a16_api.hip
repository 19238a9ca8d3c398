// C ABI of libw4a16.so: argument checks, kernel choice, split-K factor and per-stream scratch.
// The declarations and the contract live in include/w4a16.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <utility>
#include <vector>

#include "w4a16.h"
#include "w4a16_launch.h"

using namespace w4a16;

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(W4A16_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ---- per-(device, stream) scratch -------------------------------------------------------------
// One block per (device, stream) in four regions:
//   [0] control words: split-K tile counters, the decode kernel's slice flags, the fused pick's
//       row keys and the argmax counters. Zeroed when the block is allocated; every kernel leaves
//       them zero, so they are zero between calls whatever the previous call was.
//   [1] the small-row kernel's split-K exchange: fp32 slots for its slices, every word
//       kSliceEmpty when the block is allocated. Each reducer writes the pattern back into the
//       slots it took, so the region is all kSliceEmpty between calls whatever the previous call
//       was. Nothing else is stored there.
//   [2] data written before it is read within a call: the decode kernel's fp32 slices (read only
//       after their flags are raised) and fused k-best slots, the many-row GEMM's K slices.
//   [3] prepared activations, rewritten by every call that reads them.
// When a call needs a larger block, a new one is allocated and set up and the old one is kept
// (a graph captured earlier may still use it) until w4a16_release_scratch. A call that would
// allocate while its stream is being captured fails instead (allocation and zeroing are not
// captured): warm the stream up with the same shapes before capturing it.
constexpr int kRegions = 4;
struct Scratch {
    void *base = nullptr;
    size_t bytes[kRegions] = {0, 0, 0, 0};
    std::vector<void *> retired;
};

struct Key {
    int device;
    hipStream_t stream;
    bool operator<(const Key &o) const
    {
        return device != o.device ? device < o.device : (uintptr_t)stream < (uintptr_t)o.stream;
    }
};

std::mutex g_scratch_mu;
std::map<Key, Scratch> g_scratch;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct ScratchView {
    uint32_t *control;
    float *exchange;
    float *partials;
    void *act;
};

__global__ void fill_words_kernel(uint32_t *p, size_t n, uint32_t value)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = value;
}

hipError_t fill_words(uint32_t *p, size_t n, uint32_t value, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_words_kernel, dim3(256), dim3(256), 0, stream, p, n, value);
    return hipGetLastError();
}

// Returns W4A16_OK and fills `view` with pointers into a block whose regions hold at least the
// requested bytes, allocating a larger block for the stream when needed.
int get_scratch(hipStream_t stream, size_t control_bytes, size_t exchange_bytes, size_t partial_bytes,
                size_t act_bytes, ScratchView *view)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    Scratch &s = g_scratch[Key{dev, stream}];
    const size_t need[kRegions] = {std::max(control_bytes, (size_t)4096), exchange_bytes, partial_bytes, act_bytes};
    if (s.base == nullptr || s.bytes[0] < need[0] || s.bytes[1] < need[1] || s.bytes[2] < need[2] ||
        s.bytes[3] < need[3]) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
        if (cap != hipStreamCaptureStatusNone)
            return fail(W4A16_ERR_UNSUPPORTED,
                        "this call needs more scratch than its stream holds, and the stream is being captured: "
                        "run the same calls on the stream once before capturing it");
        size_t nb[kRegions], total = 0;
        for (int r = 0; r < kRegions; ++r) {
            nb[r] = round_up(std::max(need[r], s.bytes[r]), 256);
            total += nb[r];
        }
        void *p = nullptr;
        e = hipMalloc(&p, total);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(W4A16_ERR_NO_MEMORY, "hipMalloc of %zu scratch bytes: %s", total, hipGetErrorString(e));
        }
        e = hipMemsetAsync(p, 0, total, stream);
        if (e == hipSuccess)
            e = fill_words(reinterpret_cast<uint32_t *>(static_cast<char *>(p) + nb[0]), nb[1] / sizeof(uint32_t),
                           kSliceEmpty, stream);
        if (e != hipSuccess) {
            (void)hipFree(p);
            return hip_fail(e, "setting up scratch");
        }
        if (s.base) s.retired.push_back(s.base);
        s.base = p;
        for (int r = 0; r < kRegions; ++r) s.bytes[r] = nb[r];
    }
    char *b = static_cast<char *>(s.base);
    view->control = reinterpret_cast<uint32_t *>(b);
    view->exchange = reinterpret_cast<float *>(b + s.bytes[0]);
    view->partials = reinterpret_cast<float *>(b + s.bytes[0] + s.bytes[1]);
    view->act = b + s.bytes[0] + s.bytes[1] + s.bytes[2];
    return W4A16_OK;
}

// ---- the no-allocation scratch (w4a16_gemm_noalloc) -------------------------------------------
// For callers that cannot allocate: one fixed array in device memory per GPU, `scratch`, laid out
// as [control words (kNoAllocControl bytes)][split-K exchange (kNoAllocExchange bytes)][data:
// the decode kernel's slices, prepared activations (kNoAllocData bytes)]. Its address is taken with hipGetSymbolAddress once
// per device (with that device current) and kept; host code passes that address, never the
// array's name, to kernels. At that set-up fill kernels zero the control words and set every
// word of the exchange to kSliceEmpty; every kernel leaves them so from then on. Every call on a
// GPU shares its array: calls that overlap on one GPU race.
constexpr size_t kNoAllocBytes = 16u << 20;
constexpr size_t kNoAllocControl = 1u << 20;
constexpr size_t kNoAllocExchange = 6u << 20;
constexpr size_t kNoAllocData = kNoAllocBytes - kNoAllocControl - kNoAllocExchange;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

std::mutex g_noalloc_mu;
std::map<int, char *> g_noalloc_ptr;   // device -> address of its `scratch`

// Whether a call's scratch fits the no-allocation array's regions.
bool noalloc_fits(size_t control_bytes, size_t exchange_bytes, size_t partial_bytes, size_t act_bytes)
{
    return control_bytes <= kNoAllocControl && exchange_bytes <= kNoAllocExchange &&
           round_up(partial_bytes, 256) + act_bytes <= kNoAllocData;
}

int noalloc_scratch(hipStream_t stream, size_t control_bytes, size_t exchange_bytes, size_t partial_bytes,
                    size_t act_bytes, ScratchView *view)
{
    if (!noalloc_fits(control_bytes, exchange_bytes, partial_bytes, act_bytes))
        return fail(W4A16_ERR_UNSUPPORTED,
                    "the call needs %zu control, %zu exchange and %zu data bytes of scratch; the no-allocation "
                    "buffer holds %zu, %zu and %zu",
                    control_bytes, exchange_bytes, round_up(partial_bytes, 256) + act_bytes, kNoAllocControl,
                    kNoAllocExchange, kNoAllocData);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    char *base = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_noalloc_mu);
        auto it = g_noalloc_ptr.find(dev);
        if (it == g_noalloc_ptr.end()) {
            void *ptr = nullptr;
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
            uint32_t *words = static_cast<uint32_t *>(ptr);
            e = fill_words(words, kNoAllocControl / sizeof(uint32_t), 0u, stream);
            if (e == hipSuccess)
                e = fill_words(words + kNoAllocControl / sizeof(uint32_t), kNoAllocExchange / sizeof(uint32_t),
                               kSliceEmpty, stream);
            if (e != hipSuccess) return hip_fail(e, "setting up the no-allocation scratch");
            it = g_noalloc_ptr.emplace(dev, static_cast<char *>(ptr)).first;
        }
        base = it->second;
    }
    view->control = reinterpret_cast<uint32_t *>(base);
    view->exchange = reinterpret_cast<float *>(base + kNoAllocControl);
    view->partials = reinterpret_cast<float *>(base + kNoAllocControl + kNoAllocExchange);
    view->act = base + kNoAllocControl + kNoAllocExchange + round_up(partial_bytes, 256);
    return W4A16_OK;
}

// The launch plan of a shape. Measured on MI355X, the weights stream best from many short
// waves (5-20 K steps each) with a shallow ring, 4-16 thousand waves in all: they keep HBM
// busy from the first microsecond. Each column tile is cut into pieces along K, `waves_k` of
// them inside one workgroup (summed in LDS) and `splits` workgroups (summed through scratch).
// Matrices of at most one tile per compute unit take the splits that balance the CUs' work
// (below); wider ones 4 waves per workgroup up to 32 pieces, 8 beyond and for more than 8 rows.
// `splits` / `wk` > 0 override the choice (tuning and tests).
int make_plan(int M, int N, int K, int g, ZeroMode zm, int splits, int wk, int tile_cols, bool argmax,
              GemmPlan *plan)
{
    const int steps = K / kStepK;
    if (tile_cols != 0 && tile_cols != 64 && tile_cols != 128)
        return fail(W4A16_ERR_INVALID_ARG, "tile_cols=%d is not 0, 64 or 128", tile_cols);
    // 128-column tiles for wide matrices: each wave then converts its activation slice once
    // for twice the columns (measured on the 248320-column output layer: 148 -> 130 us at
    // M = 5); narrower matrices keep 64-column tiles and the larger wave count they give.
    // Affine codes above 8 rows take them too: the product against ones that forms the group
    // sums of the activations is then shared by twice the columns (affine-4 FFN 5120 x 17408,
    // groups of 64, M = 12 / 16: 28.4 -> 25.7 / 30.6 -> 27.9 us; at M <= 8 no gain).
    const int cols = tile_cols != 0 ? tile_cols / 16 : (N >= kWideTileMinN || (zm == kAffine && M > 8) ? 8 : 4);
    const int tiles = (N + tile_columns(cols) - 1) / tile_columns(cols);
    if ((splits == 0 || wk == 0) && tiles <= kCus) {
        // At most one column tile per compute unit: the launch is balanced by its workgroup
        // count, not its wave count. `s` workgroups per tile put ceil(tiles * s / kCus) of them on
        // the busiest CU, each with 1/s of the tile's work: take the s (up to two workgroups per
        // CU) that minimises that, the fewest on a tie (each slice more adds to the exchange),
        // and 16 waves per workgroup (8 for up to 8 rows when the pieces would be shorter than 8
        // steps, and 8 on 128-column tiles, whose registers already hold a CU to 4 waves per SIMD:
        // affine-4 FFN 5120 x 17408, 136 tiles, M = 9 / 12 / 16 24.0 / 24.7 / 27.2 us with 4 x 8,
        // 24.9 / 25.8 / 27.1 with 3 x 16, 21.4 / 23.0 / 25.2 with 3 x 8). Measured on MI355X, back
        // to back, us: attention 5120 x 5120 (80 tiles) M = 1 / 8 / 16 9.4 / 10.6 / 13.4 -> 8.5 /
        // 9.2 / 10.6 (3 workgroups per tile, 4 before); FFN down 17408 x 5120 M = 1 / 4 / 8 / 16
        // 16.5 / 18.8 / 21.2 / 25.4 -> 14.7 / 15.3 / 17.5 / 23.1;
        // 5120 x 4096 (64 tiles) M = 1 / 16 8.3 / 9.9 -> 7.6 / 8.8; 5120 x 13824 (216 tiles) M = 1
        // / 16 12.4 / 20.4 -> 11.1 / 18.5 (whole K in a workgroup); 5120 x 8192 (128 tiles) M = 16
        // 13.6 -> 12.4. Matrices of more tiles keep the wave-count rule below.
        int s = 1;
        for (int c = 2; c <= std::min(16, 2 * kCus / tiles); ++c)
            if ((long long)((tiles * c + kCus - 1) / kCus) * s < (long long)((tiles * s + kCus - 1) / kCus) * c) s = c;
        int w = cols == 4 && (M > 8 || steps / (s * 16) >= 8) ? 16 : 8;
        while (w > 1 && s * w > steps) w /= 2;
        s = std::max(1, std::min(s, steps / w));
        if (wk == 0) wk = w;
        if (splits == 0) splits = std::max(1, std::min(s, steps / wk));
    }
    if (splits == 0 || wk == 0) {
        // P pieces per tile: about 4352 waves in all, at least 8 pieces, of at least 10 steps
        // up to 4 rows (attention, M = 1: 16 pieces of 10 steps 10.2 us, 32 of 5 10.6 us) and
        // at least 5 steps beyond (attention, M = 8: 11.9 us with 5 steps, 12.6 with 10); for
        // more than 8 rows 8192 waves, at most 64 pieces, whose shorter pieces keep their
        // activation slices within the LDS staging budget. The workgroups per tile are rounded
        // up to a power of two (FFN down, M = 1..8: 8 beat 7 by 0.5-1.2 us).
        const int want = M > 8 ? 8192 : 4352;
        const int cap = M > 8 ? std::min(64, steps / 5) : M > 4 ? steps / 5 : steps / 10;
        const int P = std::max(8, std::min(cap, (want + tiles - 1) / tiles));
        int w = P <= 8 ? P : (P < 32 && M <= 8 ? 4 : 8);
        while (w > 1 && w > steps) w /= 2;
        int s = 1;
        while (s < (P + w - 1) / w) s *= 2;
        s = std::max(1, std::min(s, steps / w));
        if (wk == 0) wk = w;
        if (splits == 0) splits = std::max(1, std::min(s, steps / wk));
    }
    if (wk != 1 && wk != 2 && wk != 4 && wk != 8 && wk != 16)
        return fail(W4A16_ERR_INVALID_ARG, "waves_k=%d is not 1, 2, 4, 8 or 16", wk);
    if (splits < 1 || splits > 65535 || (long long)splits * wk > steps)
        return fail(W4A16_ERR_INVALID_ARG, "splits=%d x waves_k=%d exceeds the %d K-steps of 32", splits, wk, steps);
    // One row takes the dot-product GEMV on 64-column tiles. On 128-column tiles its eight
    // columns per lane make the VALU the tighter resource, and the matrix cores (16 rows of which
    // one is used) measure faster: 248320-column output layer, 120.3 -> 116.1 us.
    plan->mfma = M > 1 || cols == 8;
    plan->cols = cols;
    plan->wk = wk;
    plan->splits = splits;
    // Stage activations in LDS when a wave's slice fits the per-wave budget: then they arrive by
    // direct loads issued with the weights and are converted once. Past the budget the LDS a
    // workgroup needs would cut the waves per CU; those slices are prepared once per call
    // instead (below). The GEMV always stages.
    // On 128-column tiles, whose registers already limit the waves per CU, the test is whether the
    // staged workgroups still fit that many waves (output layer, M = 5: 134.4 -> 127.7 us).
    GemmPlan staged{};
    const size_t lds_staged = gemm_lds_layout(M, K, g, splits, wk, cols, true, zm, argmax, &staged);
    const bool fits = cols == 8 ? (size_t)kLdsPerCu / lds_staged >= (size_t)std::max(1, kWideTileWavesPerCu / wk)
                                : (size_t)staged.wave_lds <= (size_t)kLdsStageBudget;
    plan->lds_a = !plan->mfma || (fits && lds_staged <= (size_t)kMaxLds);
    // Activations a wave cannot stage are prepared once per call by a separate kernel: without
    // it each wave would run an exponent pass over its slice and convert every fragment as it
    // streams in. Staged slices are converted in the wave (cheaper than the extra launch).
    plan->prep_a = plan->mfma && !plan->lds_a;
    plan->lds = gemm_lds_layout(M, K, g, splits, wk, cols, plan->lds_a, zm, argmax, plan);
    if (plan->lds > (size_t)kMaxLds)
        return fail(W4A16_ERR_INVALID_ARG, "plan needs %zu bytes of LDS per workgroup (max %d): use more splits",
                    plan->lds, kMaxLds);
    return W4A16_OK;
}

// The decode kernel's launch (w4a16_decode.hip). A workgroup is `tiles` x `kw` waves on adjacent
// column tiles over one K slice; `slices` workgroups per group of columns. Defaults: 4 tiles of 64
// columns, one wave each; slices for about 512 workgroups (at most 16, at least 4 K steps per
// slice, more while the slice's activations would not fit in LDS). `slices`, `tiles`, `kw`,
// `tile_cols` and `ring` > 0 override the defaults (tuning and tests).
// `bits`: 0 for GPTQ codes, else the width of affine codes (64-column tiles, a ring of 4)
int make_decode_plan(int M, int N, int K, int g, bool packed, int slices, int tiles, int kw, int tile_cols, int ring,
                     bool pick, DecodePlan *pl, int bits = 0)
{
    const bool affine = bits > 0;
    if (tile_cols != 0 && tile_cols != 64 && tile_cols != 128)
        return fail(W4A16_ERR_INVALID_ARG, "tile_cols=%d is not 0, 64 or 128", tile_cols);
    if (affine && tile_cols == 128)
        return fail(W4A16_ERR_INVALID_ARG, "affine codes run on 64-column tiles (tile_cols=%d)", tile_cols);
    // 1- and 2-bit codes: a word per lane, blocks of 4 / bits steps, where the quantisation groups
    // hold whole blocks (otherwise the 8-row reader, 2 or 4 lanes per word)
    pl->sub = affine && bits <= 2 && g % (kStepK * 4 / bits) == 0 ? 4 / bits : 1;
    const int steps = K / kStepK / pl->sub;   // in blocks: slices and pieces take whole ones
    pl->mfma = M > 1;
    pl->cols = tile_cols ? tile_cols / 16 : 4;
    pl->one_round = false;
    // GPTQ codes, 9-16 rows, fewer than kDecodeMinN columns: 4 tiles x 2 K pieces per workgroup, a
    // ring of 4, and the fewest K slices that give at least kDecodeMidWgs workgroups which all run
    // at once (measured on MI355X, back to back, at 16 rows: FFN 5120 x 17408 3 slices 20.5-20.7
    // us against 21.8-23.4 for the small-row kernel, 8 tiles x 1 piece 23.1-23.4, ring 8 21.6;
    // 5120 x 32768 2 slices 25.5 against 29.6; 8192 x 28672 with 3 slices, one and a third rounds
    // of workgroups, 48.4 against 41.9)
    // Affine codes from kDecodeMidN to kDecodeMinN columns take the same launch at every row count
    // (affine FFN 5120 x 17408, groups of 64, us back to back, 6 slices of 4 tiles x 1 piece ->
    // 3 slices of 4 x 2: 4-bit M = 1 / 8 / 16 18.0 / 20.9 / 22.7 -> 16.7 / 19.4 / 21.1; 8-bit
    // 21.9 / 25.0 / 26.5 -> 20.5 / 23.0 / 24.9; 2-bit 18.2 / 21.4 / 22.6 -> 17.0 / 20.0 / 21.9).
    const bool mid = N < kDecodeMinN && (affine ? N >= kDecodeMidN : M > 8);
    // more rows stage more activations per workgroup, which leaves room for fewer workgroups per
    // CU: give each workgroup more waves
    // (narrower affine matrices: 4 tiles at every row count; on the 5120 x 17408 projection at
    // 2, 4 and 8 bits 8 tiles with more K slices lost 10-30%)
    pl->tiles = tiles ? tiles : (pl->mfma && (!affine || N >= kDecodeMinN) && !mid ? 8 : 4);
    pl->kw = kw ? kw : mid ? 2 : 1;
    if (pl->tiles < 1 || pl->kw < 1 || pl->tiles * pl->kw > kDecMaxWaves)
        return fail(W4A16_ERR_INVALID_ARG, "tiles=%d x kw=%d waves outside 1..%d", pl->tiles, pl->kw, kDecMaxWaves);
    const long long wc = (long long)pl->tiles * 16 * pl->cols;
    const int groups = (int)((N + wc - 1) / wc);
    if (slices == 0 && mid) {
        // workgroups per CU: by waves (3 with the 77 registers of the ring-4 instance) and by LDS
        const int by_waves = 3 * 8 / (pl->tiles * pl->kw);
        for (int s = std::max(1, (kDecodeMidWgs + groups - 1) / groups);
             s <= std::min(kDecMaxSlices, steps / pl->kw); ++s) {
            const size_t lds =
                decode_lds_layout(M, K, g, pl->mfma, pl->cols, pl->tiles, pl->kw, s, packed, pick, nullptr, false);
            const long long per_cu = std::min<long long>(by_waves, (long long)(kLdsPerCu / lds));
            if (lds <= (size_t)kMaxLds && (long long)groups * s <= (long long)kCus * per_cu) {
                slices = s;
                pl->one_round = true;
                break;
            }
        }
    }
    if (slices == 0) {
        // about 512 workgroups (affine codes: 400, which measured 8-10% faster than 512)
        const int target = affine ? 400 : 512;
        slices = (int)std::min<long long>(kDecMaxSlices, (target + groups - 1) / groups);
        slices = std::max(1, std::min(slices, steps / (4 * pl->kw)));
        // long K: more slices until the slice's activations fit in LDS; past 8 rows (affine codes:
        // past one row, whose scales and biases of groups of 64 take 4x the LDS of GPTQ's groups
        // of 128), until two workgroups fit on a CU (one workgroup of 16 rows per CU leaves the CU
        // too few waves)
        const size_t lds_cap = M > 8 || (affine && M > 1) ? (size_t)kMaxLds / 2 : (size_t)kMaxLds;
        while (slices < std::min(kDecMaxSlices, steps / pl->kw) &&
               decode_lds_layout(M, K, g, pl->mfma, pl->cols, pl->tiles, pl->kw, slices, packed, pick, nullptr, affine,
                                 pl->sub) > lds_cap)
            ++slices;
    }
    if (slices < 1 || slices > kDecMaxSlices || (long long)slices * pl->kw > steps)
        return fail(W4A16_ERR_INVALID_ARG, "slices=%d outside 1..%d, or slices x kw=%d above the %d K-%s",
                    slices, kDecMaxSlices, pl->kw, steps, pl->sub > 1 ? "blocks" : "steps of 32");
    pl->slices = slices;
    // the kernel addresses a slice's codes (plus the ring's reads past its end) with 32-bit byte
    // offsets
    const long long smax = (long long)(steps + slices - 1) / slices * pl->sub;
    const long long step_bytes = 4LL * (affine ? bits : 4) * N;   // a step's codes over all columns
    if ((smax + 8LL * pl->sub) * step_bytes >= (1LL << 31))
        return fail(W4A16_ERR_UNSUPPORTED, "a K slice of %lld steps over %d columns exceeds 2 GiB of codes: use more slices",
                    smax, N);
    pl->ring = ring ? ring : affine || mid ? 4 : (pl->cols == 8 ? 2 : M == 1 ? 3 : M <= 8 ? 4 : 8);
    const bool ring_ok = affine ? pl->ring == 4
                         : pl->cols == 8 ? (pl->ring == 2 || pl->ring == 4)
                                         : (pl->ring == 2 || pl->ring == 3 || pl->ring == 4 || pl->ring == 6 || pl->ring == 8);
    if (!ring_ok)
        return fail(W4A16_ERR_INVALID_ARG, "ring=%d is not available for %s", pl->ring,
                    affine ? "affine codes (4)" : pl->cols == 8 ? "128-column tiles" : "64-column tiles");
    pl->lds = decode_lds_layout(M, K, g, pl->mfma, pl->cols, pl->tiles, pl->kw, slices, packed, pick, pl, affine, pl->sub);
    if (pl->lds > (size_t)kMaxLds)
        return fail(W4A16_ERR_INVALID_ARG, "decode plan needs %zu bytes of LDS per workgroup (max %d): use more slices",
                    pl->lds, kMaxLds);
    return W4A16_OK;
}

int check_gemm_args(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                    int g, int M, int N, int K, void *out, int out_dtype, int max_m = 16)
{
    if (!A || !qweight || !scales || !out)
        return fail(W4A16_ERR_INVALID_ARG, "null pointer (A=%p qweight=%p scales=%p out=%p)", A,
                    (const void *)qweight, (const void *)scales, out);
    if (M < 1 || M > max_m) return fail(W4A16_ERR_INVALID_ARG, "M=%d outside 1..%d", M, max_m);
    if (N <= 0 || K <= 0 || g <= 0)
        return fail(W4A16_ERR_INVALID_ARG, "sizes must be positive (N=%d K=%d group_size=%d)", N, K, g);
    if (g % 32) return fail(W4A16_ERR_INVALID_ARG, "group_size=%d is not a multiple of 32", g);
    if (K % g) return fail(W4A16_ERR_INVALID_ARG, "K=%d is not a multiple of group_size=%d", K, g);
    if (N % 8) return fail(W4A16_ERR_INVALID_ARG, "N=%d is not a multiple of 8", N);
    if ((long long)(K / 8) * N > 0xFFFFFFFFLL)   // the kernels address qweight with 32-bit word offsets
        return fail(W4A16_ERR_UNSUPPORTED, "qweight of %lld words exceeds 2^32 words", (long long)(K / 8) * N);
    if (!aligned16(A) || !aligned16(qweight) || !aligned16(scales) || (qzeros && !aligned16(qzeros)) ||
        !aligned16(out))
        return fail(W4A16_ERR_UNSUPPORTED, "every pointer must be 16-byte aligned");
    if (out_dtype != W4A16_OUT_F32 && out_dtype != W4A16_OUT_BF16)
        return fail(W4A16_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
    return W4A16_OK;
}


// One stored matrix: packed codes, scales, packed zeros (nullptr: symmetric), or for affine
// codes bf16 scales and bf16 biases (no zeros).
struct Matrix {
    const uint32_t *qweight;
    const uint16_t *scales;
    const uint32_t *qzeros;
    const uint16_t *biases = nullptr;
};

// One GEMM call: check, plan, take scratch, launch. `idx` non-null adds the fused greedy pick;
// `up` non-null makes it a gated pair (w is the gate): out = silu(A x w) * (A x up), planned as
// one 2N-column problem on 128-column tiles (64 output columns of each matrix). `pair_sum` adds
// the pair's two products instead: out = (A x w) + (A x up).
int decode_call(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                int group_size, int M, int N, int K, void *out, int out_dtype, int slices, int tiles, int kw,
                int tile_cols, int ring, int topk, int32_t *idx, int pick_none, hipStream_t stream, bool noalloc,
                const uint16_t *biases = nullptr, int bits = 0);

// Whether a plain GPTQ call takes the decode kernel by default: for matrices of at least
// kDecodeMinN columns, wide enough to fill the chip with whole-K (or few-slice) workgroups, such
// as the 248320-column output layer (MI355X, back-to-back launches: 101 against 115 us at one row,
// 111 against 124 at five, 137 against 163 at sixteen); and for 9-16 rows on matrices of
// kDecodeMidN columns or more when its launch for them runs in one round (see make_decode_plan).
// Narrower matrices, and fewer rows, need more K slices, whose exchange costs the decode kernel
// more than the small-row kernel's split-K (FFN 5120 x 17408: 17 against 14 us at one row, 18.0
// against 16.7 at eight; attention 5120 x 5120 at sixteen: 17.2 against 13.6).
bool decode_by_default(int M, int N, int K, int g, bool packed, bool pick)
{
    if (N < kDecodeMidN || (N < kDecodeMinN && M <= 8)) return false;
    DecodePlan pl{};
    if (make_decode_plan(M, N, K, g, packed, 0, 0, 0, 0, 0, pick, &pl) != W4A16_OK) return false;
    return N >= kDecodeMinN || pl.one_round;
}

int gemm_call(const void *A, Matrix w, const Matrix *up, int group_size, int M, int N, int K, void *out,
              int out_dtype, int splits, int waves_k, int tile_cols, int32_t *idx, hipStream_t stream,
              bool pair_sum = false, bool noalloc = false)
{
    if (!up && !w.biases && splits == 0 && waves_k == 0 && tile_cols == 0 && M >= 1 && M <= 16 && N > 0 && K > 0 &&
        group_size > 0 && group_size % 32 == 0 && K % group_size == 0 && N % 8 == 0 &&
        decode_by_default(M, N, K, group_size, w.qzeros != nullptr, idx != nullptr))
        return decode_call(A, w.qweight, w.scales, w.qzeros, group_size, M, N, K, out, out_dtype, 0, 0, 0, 0, 0,
                           idx ? 1 : 0, idx, 0, stream, noalloc);
    const uint32_t *qweight = w.qweight;
    const uint16_t *scales = w.scales;
    const uint32_t *qzeros = w.qzeros;
    int rc = check_gemm_args(A, qweight, scales, qzeros, group_size, M, N, K, out, out_dtype);
    if (rc != W4A16_OK) return rc;
    if (w.biases && (qzeros || idx || (up && (up->qzeros || !up->biases))))
        return fail(W4A16_ERR_INVALID_ARG, "affine codes take no zero points or fused pick, and pair only with affine codes");
    if (!w.biases && up && up->biases)
        return fail(W4A16_ERR_INVALID_ARG, "a GPTQ matrix does not pair with affine codes");
    if ((w.biases && !aligned16(w.biases)) || (up && up->biases && !aligned16(up->biases)))
        return fail(W4A16_ERR_UNSUPPORTED, "every pointer must be 16-byte aligned");
    const ZeroMode zm = w.biases ? kAffine : qzeros ? kZeroPacked : kZeroSym;
    if (up) {
        rc = check_gemm_args(A, up->qweight, up->scales, up->qzeros, group_size, M, N, K, out, out_dtype);
        if (rc != W4A16_OK) return rc;
        if ((qzeros == nullptr) != (up->qzeros == nullptr))
            return fail(W4A16_ERR_INVALID_ARG, "qzeros_gate and qzeros_up must both be NULL or both be given");
    }
    if (splits < 0 || waves_k < 0)
        return fail(W4A16_ERR_INVALID_ARG, "splits=%d waves_k=%d must be >= 0", splits, waves_k);
    const int NV = up ? 2 * N : N;   // columns of the planned problem
    if (up) tile_cols = 128;
    GemmPlan plan{};
    rc = make_plan(M, NV, K, group_size, zm, splits, waves_k, tile_cols, idx != nullptr, &plan);
    if (rc != W4A16_OK) return rc;
    // scratch of a plan: control words [tile counters][fused pick's row keys, one slot of 16 x 64
    // bit per tile], the split-K exchange [splits, M, NV], prepared activations [M, K] and their
    // shifts
    const size_t tile = (size_t)tile_columns(plan.cols);
    const size_t tiles = ((size_t)NV + tile - 1) / tile;
    const size_t a16_bytes = round_up((size_t)M * K * sizeof(uint16_t), 256);
    auto needs = [&](const GemmPlan &pl, size_t *control, size_t *exch, size_t *act) {
        *control = round_up(tiles * sizeof(uint32_t), 8) + (idx ? tiles * 16 * sizeof(unsigned long long) : 0);
        *exch = pl.splits > 1 ? (size_t)pl.splits * M * NV * sizeof(float) : 0;
        *act = pl.prep_a ? a16_bytes + (size_t)pl.splits * pl.wk * M * sizeof(int) : 0;
    };
    size_t control_bytes, exchange_bytes, act_bytes;
    needs(plan, &control_bytes, &exchange_bytes, &act_bytes);
    // the no-allocation buffer: a default plan that does not fit takes fewer workgroups per tile
    // (fewer partial slices), down to one
    // (down to one, or to the last launch that still fits in LDS; what still does not fit is refused
    // by noalloc_scratch)
    while (noalloc && splits == 0 && plan.splits > 1 && !noalloc_fits(control_bytes, exchange_bytes, 0, act_bytes)) {
        GemmPlan fewer{};
        if (make_plan(M, NV, K, group_size, zm, std::max(1, plan.splits / 2), plan.wk, tile_cols, idx != nullptr,
                      &fewer) != W4A16_OK)
            break;
        plan = fewer;
        needs(plan, &control_bytes, &exchange_bytes, &act_bytes);
    }

    GemmArgs a{};
    a.A = static_cast<const uint16_t *>(A);
    a.qweight = qweight;
    a.scales = scales;
    a.qzeros = qzeros;
    a.biases = w.biases;
    if (up) {
        a.qweight2 = up->qweight;
        a.scales2 = up->scales;
        a.qzeros2 = up->qzeros;
        a.biases2 = up->biases;
        a.pair_sum = pair_sum ? 1 : 0;
    }
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.g = group_size;
    a.splits = plan.splits;
    a.out_bf16 = out_dtype == W4A16_OUT_BF16;
    a.wave_lds = plan.wave_lds;
    a.scale_off = plan.scale_off;
    a.zero_off = plan.zero_off;
    const bool split_k = plan.splits > 1;
    if (split_k || plan.prep_a || idx) {
        const size_t key_off = round_up(tiles * sizeof(uint32_t), 8);
        ScratchView v{};
        rc = noalloc ? noalloc_scratch(stream, control_bytes, exchange_bytes, 0, act_bytes, &v)
                     : get_scratch(stream, control_bytes, exchange_bytes, 0, act_bytes, &v);
        if (rc != W4A16_OK) return rc;
        char *c = reinterpret_cast<char *>(v.control);
        a.counters = v.control;
        a.partials = v.exchange;
        a.A16 = static_cast<uint16_t *>(v.act);
        a.ashift = reinterpret_cast<int *>(static_cast<char *>(v.act) + a16_bytes);
        if (idx) {
            a.amax_keys = reinterpret_cast<unsigned long long *>(c + key_off);
            a.amax_idx = idx;
        }
    }
    const hipError_t e = launch_gemm(a, plan, stream);
    if (e != hipSuccess) return hip_fail(e, "GEMM launch");
    return W4A16_OK;
}

// Affine codes read at their own width: column bit streams [K * bits / 32, N] (addressed with
// 32-bit word offsets), bf16 scales and biases, no zero points.
int check_affine_bits_args(const uint32_t *qzeros, const uint16_t *biases, int bits, int N, int K)
{
    if (!biases) return fail(W4A16_ERR_INVALID_ARG, "null pointer (biases)");
    if (qzeros) return fail(W4A16_ERR_INVALID_ARG, "affine codes take no zero points");
    if (!(bits >= 1 && bits <= 6) && bits != 8)
        return fail(W4A16_ERR_INVALID_ARG, "bits=%d is not 1, 2, 3, 4, 5, 6 or 8 (7-bit codes: w4a16_affine_split)",
                    bits);
    if (!aligned16(biases)) return fail(W4A16_ERR_UNSUPPORTED, "every pointer must be 16-byte aligned");
    if ((long long)(K / 32) * bits * N > 0xFFFFFFFFLL)
        return fail(W4A16_ERR_UNSUPPORTED, "codes of %lld words exceed 2^32 words", (long long)(K / 32) * bits * N);
    return W4A16_OK;
}

// A decode-kernel call: check, plan, take scratch, launch.
int decode_call(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                int group_size, int M, int N, int K, void *out, int out_dtype, int slices, int tiles, int kw,
                int tile_cols, int ring, int topk, int32_t *idx, int pick_none, hipStream_t stream, bool noalloc,
                const uint16_t *biases, int bits)
{
    int rc = check_gemm_args(A, qweight, scales, qzeros, group_size, M, N, K, out, out_dtype);
    if (rc != W4A16_OK) return rc;
    if (bits) {
        rc = check_affine_bits_args(qzeros, biases, bits, N, K);
        if (rc != W4A16_OK) return rc;
    }
    if (slices < 0 || tiles < 0 || kw < 0 || ring < 0)
        return fail(W4A16_ERR_INVALID_ARG, "slices=%d tiles=%d kw=%d ring=%d must be >= 0", slices, tiles, kw, ring);
    if (topk < 0 || topk > kDecMaxTopK || (topk > 0) != (idx != nullptr))
        return fail(W4A16_ERR_INVALID_ARG, "k=%d outside 1..%d, or idx %s", topk, kDecMaxTopK,
                    idx ? "given without k" : "missing (null pointer)");
    DecodePlan plan{};
    rc = make_decode_plan(M, N, K, group_size, qzeros != nullptr, slices, tiles, kw, tile_cols, ring, topk > 0, &plan,
                          bits);
    if (rc != W4A16_OK) return rc;
    const long long wc = (long long)plan.tiles * 16 * plan.cols;
    const int groups = (int)((N + wc - 1) / wc);
    // the data a launch keeps in scratch: fp32 slices, then the fused pick's slots
    auto data_need = [&](int sl) {
        const size_t part = sl > 1 ? (size_t)sl * M * N * sizeof(float) : 0;
        return round_up(part, 256) + (size_t)groups * M * topk * sizeof(unsigned long long);
    };
    // the no-allocation array: a default launch whose slices do not fit takes fewer slices while
    // its activation slice still fits in LDS (what still does not fit is refused below)
    while (noalloc && slices == 0 && plan.slices > 1 && !noalloc_fits(0, 0, data_need(plan.slices), 0)) {
        DecodePlan fewer{};
        if (make_decode_plan(M, N, K, group_size, qzeros != nullptr, plan.slices - 1, tiles, kw, tile_cols, ring,
                             topk > 0, &fewer, bits) != W4A16_OK)
            break;
        plan = fewer;
    }
    DecodeArgs a{};
    a.A = static_cast<const uint16_t *>(A);
    a.qweight = qweight;
    a.scales = scales;
    a.qzeros = qzeros;
    a.biases = bits ? biases : nullptr;
    a.bits = bits;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.g = group_size;
    a.tiles = plan.tiles;
    a.kw = plan.kw;
    a.slices = plan.slices;
    a.groups = groups;
    a.out_bf16 = out_dtype == W4A16_OUT_BF16;
    a.a_off = plan.a_off;
    a.s_off = plan.s_off;
    a.z_off = plan.z_off;
    a.r_off = plan.r_off;
    a.mp_log2 = decode_mp_log2(M);
    if (plan.slices > 1 || topk > 0) {
        // control words: [counters, one per group of columns][flags, groups x slices][the fused
        // pick's counter]; data: [fp32 partials, slices x M x N][the fused pick's slots, groups x
        // M x k keys]. (The decode kernel keeps per-slice flags: the small-row kernel's exchange,
        // whose reducer writes the empty pattern back, would add the slices' bytes again in
        // writes, 2.2 MB per call at 16 rows on FFN 5120 x 17408, for no measured gain here.)
        const size_t control_bytes = (size_t)groups * (1 + plan.slices) * sizeof(uint32_t) + sizeof(uint32_t);
        const size_t part_bytes = plan.slices > 1 ? (size_t)plan.slices * M * N * sizeof(float) : 0;
        if (part_bytes >= (1ull << 31))
            return fail(W4A16_ERR_UNSUPPORTED, "%zu bytes of partial sums exceed the 2 GiB the kernel addresses",
                        part_bytes);
        const size_t slot_off = round_up(part_bytes, 256);
        const size_t data_bytes = slot_off + (size_t)groups * M * topk * sizeof(unsigned long long);
        ScratchView v{};
        rc = noalloc ? noalloc_scratch(stream, control_bytes, 0, data_bytes, 0, &v)
                     : get_scratch(stream, control_bytes, 0, data_bytes, 0, &v);
        if (rc != W4A16_OK) return rc;
        a.counters = v.control;
        a.flags = v.control + groups;
        a.partials = v.partials;
        a.part_bytes = (uint32_t)part_bytes;
        if (topk > 0) {
            a.topk = topk;
            a.pick_none = pick_none;
            a.pick_counter = v.control + (size_t)groups * (1 + plan.slices);
            a.pick_slots = reinterpret_cast<unsigned long long *>(reinterpret_cast<char *>(v.partials) + slot_off);
            a.pick_idx = idx;
        }
    }
    const hipError_t e = launch_decode(a, plan, stream);
    if (e != hipSuccess) return hip_fail(e, "decode GEMM launch");
    return W4A16_OK;
}

// A many-row call (prompt processing): check, choose the K slices, take scratch, prepare the
// activations, launch. `up` non-null makes it a gated pair (w is the gate); bits > 0 makes w
// affine codes of that width (w.biases given), a single matrix.
int prefill_call(const void *A, Matrix w, const Matrix *up, int group_size, int M, int N, int K, void *out,
                 int out_dtype, hipStream_t stream, int bits = 0)
{
    int rc = check_gemm_args(A, w.qweight, w.scales, w.qzeros, group_size, M, N, K, out, out_dtype, W4A16_PREFILL_MAX_M);
    if (rc != W4A16_OK) return rc;
    if (bits) {
        rc = check_affine_bits_args(w.qzeros, w.biases, bits, N, K);
        if (rc != W4A16_OK) return rc;
    }
    if (up) {
        rc = check_gemm_args(A, up->qweight, up->scales, up->qzeros, group_size, M, N, K, out, out_dtype,
                             W4A16_PREFILL_MAX_M);
        if (rc != W4A16_OK) return rc;
        if ((w.qzeros == nullptr) != (up->qzeros == nullptr))
            return fail(W4A16_ERR_INVALID_ARG, "qzeros_gate and qzeros_up must both be NULL or both be given");
    }
    const int out_cols = up ? kPrefillTileN / 2 : kPrefillTileN;   // output columns per tile
    // K slices when the tiles cannot fill the compute units: about two 4-wave workgroups per CU
    // run at once (`slots`), so fewer tiles than that are cut into S = slots / tiles whole-group
    // K ranges (at most 16) whose fp32 sums are added in slice order. Measured on MI355X: FFN
    // down 17408 x 5120 at M = 512, 160 tiles, 371 -> 207 us with 3 slices; at M = 128 12 slices
    // 80 us. From one full round of tiles on, the slices' extra fp32 traffic costs more than
    // the idle tail (attention 5120 x 5120 at M = 2048: 177 us whole, 213 us in 4 slices).
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    const long long tiles = (long long)((M + kPrefillTileM - 1) / kPrefillTileM) * ((N + out_cols - 1) / out_cols);
    const long long slots = 2LL * std::max(cus, 1);
    // Workgroups a CU holds at once: 3 for GPTQ codes with symmetric zero points, 2 otherwise.
    const bool three = w.qzeros == nullptr && bits == 0;
    const long long resident = (three ? 3LL : 2LL) * std::max(cus, 1);
    int splits = tiles >= slots ? 1 : (int)std::min<long long>({16LL, (long long)(K / group_size), slots / tiles});
    // The symmetric kernel, which holds 3 workgroups a CU, takes up to that many when the count
    // above is 1 or 2, or while each slice keeps at least 8 quantisation groups (FFN up 5120 x
    // 17408 at M = 256, 272 tiles: 107.5 us whole, 89.4 in 2 slices; at M = 128, 136 tiles, 57.0
    // in 3 slices, 53.3 in 5; attention at M = 1024, 320 tiles: 111 -> 93). Shorter slices past
    // the 2-a-CU count lost on attention at M = 128 and 256 (12 -> 16 slices 32.4 -> 34.6 us,
    // 6 -> 9 40.2 -> 41.3).
    if (three && tiles < resident)
        splits = (int)std::min<long long>({16LL, (long long)(K / group_size), resident / tiles,
                                           std::max<long long>({2LL, (long long)splits,
                                                                (long long)(K / group_size) / 8})});
    // From one round on, the 2-workgroup kernels take two slices when they cut the rounds the tiles
    // need by a fifth or more: FFN down 17408 x 5120 (stored zero points) at M = 2048, 640 tiles,
    // 1.25 rounds of 512: 750-767 us whole, 632 in 2 slices (659 in 3, 651 in 4). The symmetric
    // kernel, whose third workgroup a CU makes the last round cheaper, stays whole (FFN up at M =
    // 1024, 1088 tiles: 259 us whole, 281 in 2 slices; at M = 2048 469 -> 528).
    if (!three && tiles >= slots && K / group_size >= 2) {
        const long long whole = (tiles + resident - 1) / resident;        // rounds, in whole-K tiles
        const long long halves = (2 * tiles + resident - 1) / resident;   // rounds of half-K tiles
        if (5 * halves <= 8 * whole) splits = 2;                          // halves / 2 <= 0.8 whole
    }
    // scratch: the prepared activations (fp16, [M, K]), one rescale per row, the K slices
    const size_t a16_bytes = round_up((size_t)M * K * sizeof(uint16_t), 256);
    const size_t part_bytes = splits > 1 ? (size_t)splits * M * N * (up ? 2 : 1) * sizeof(float) : 0;
    ScratchView v{};
    rc = get_scratch(stream, 0, 0, part_bytes, a16_bytes + (size_t)M * sizeof(int), &v);
    if (rc != W4A16_OK) return rc;
    uint16_t *a16 = static_cast<uint16_t *>(v.act);
    int *shifts = reinterpret_cast<int *>(static_cast<char *>(v.act) + a16_bytes);
    e = launch_act_prep(ActPrepArgs{static_cast<const uint16_t *>(A), a16, shifts, M, K, 1, 1}, stream);
    if (e != hipSuccess) return hip_fail(e, "activation preparation launch");
    PrefillArgs pa{};
    pa.A16 = a16;
    pa.shifts = shifts;
    pa.qweight = w.qweight;
    pa.scales = w.scales;
    pa.qzeros = w.qzeros;
    if (up) {
        pa.qweight2 = up->qweight;
        pa.scales2 = up->scales;
        pa.qzeros2 = up->qzeros;
    }
    pa.biases = bits ? w.biases : nullptr;
    pa.bits = bits;
    pa.out = out;
    pa.partials = v.partials;
    pa.M = M;
    pa.N = N;
    pa.K = K;
    pa.g = group_size;
    pa.out_bf16 = out_dtype == W4A16_OUT_BF16;
    pa.splits = splits;
    e = launch_prefill(pa, stream);
    if (e != hipSuccess) return hip_fail(e, "prefill GEMM launch");
    return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_gemm_ex(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                  int group_size, int M, int N, int K, void *out, int out_dtype, int splits, int waves_k,
                  int tile_cols, hipStream_t stream)
{
    return gemm_call(A, Matrix{qweight, scales, qzeros}, nullptr, group_size, M, N, K, out, out_dtype, splits,
                     waves_k, tile_cols, nullptr, stream);
}

int w4a16_gemm_decode_ex(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                         int group_size, int M, int N, int K, void *out, int out_dtype, int slices, int tiles, int kw,
                         int tile_cols, int ring, int topk, int32_t *idx, hipStream_t stream)
{
    return decode_call(A, qweight, scales, qzeros, group_size, M, N, K, out, out_dtype, slices, tiles, kw, tile_cols,
                       ring, topk, idx, -1, stream, false);
}

int w4a16_gemm_affine_bits_ex(const void *A, const uint32_t *packed, int bits, const uint16_t *scales,
                              const uint16_t *biases, int group_size, int M, int N, int K, void *out, int out_dtype,
                              int slices, int tiles, int kw, int ring, hipStream_t stream)
{
    if (bits == 0) return fail(W4A16_ERR_INVALID_ARG, "bits=0 is not 1, 2, 3, 4, 5, 6 or 8");
    return decode_call(A, packed, scales, nullptr, group_size, M, N, K, out, out_dtype, slices, tiles, kw, 0, ring, 0,
                       nullptr, 0, stream, false, biases, bits);
}

int w4a16_gemm_affine_bits(const void *A, const uint32_t *packed, int bits, const uint16_t *scales,
                           const uint16_t *biases, int group_size, int M, int N, int K, void *out, int out_dtype,
                           hipStream_t stream)
{
    return w4a16_gemm_affine_bits_ex(A, packed, bits, scales, biases, group_size, M, N, K, out, out_dtype, 0, 0, 0, 0,
                                     stream);
}

int w4a16_gemm_affine_bits_prefill(const void *A, const uint32_t *packed, int bits, const uint16_t *scales,
                                   const uint16_t *biases, int group_size, int M, int N, int K, void *out,
                                   int out_dtype, hipStream_t stream)
{
    if (bits == 0) return fail(W4A16_ERR_INVALID_ARG, "bits=0 is not 1, 2, 3, 4, 5, 6 or 8");
    Matrix w{packed, scales, nullptr};
    w.biases = biases;
    return prefill_call(A, w, nullptr, group_size, M, N, K, out, out_dtype, stream, bits);
}

int w4a16_gemm_topk(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                    int group_size, int M, int N, int K, void *out, int out_dtype, int k, int32_t *idx,
                    hipStream_t stream)
{
    if (!idx) return fail(W4A16_ERR_INVALID_ARG, "null pointer (idx)");
    if (k < 1 || k > kDecMaxTopK) return fail(W4A16_ERR_INVALID_ARG, "k=%d outside 1..%d", k, kDecMaxTopK);
    return decode_call(A, qweight, scales, qzeros, group_size, M, N, K, out, out_dtype, 0, 0, 0, 0, 0, k, idx, -1,
                       stream, false);
}

int w4a16_gemm_argmax(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                      int group_size, int M, int N, int K, void *out, int out_dtype, int32_t *idx,
                      hipStream_t stream)
{
    if (!idx) return fail(W4A16_ERR_INVALID_ARG, "null pointer (idx)");
    return gemm_call(A, Matrix{qweight, scales, qzeros}, nullptr, group_size, M, N, K, out, out_dtype, 0, 0, 0, idx,
                     stream);
}

int w4a16_gemm_prefill(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                       int group_size, int M, int N, int K, void *out, int out_dtype, hipStream_t stream)
{
    return prefill_call(A, Matrix{qweight, scales, qzeros}, nullptr, group_size, M, N, K, out, out_dtype, stream);
}

int w4a16_gemm_gate_up_prefill(const void *A, const uint32_t *qweight_gate, const uint16_t *scales_gate,
                               const uint32_t *qzeros_gate, const uint32_t *qweight_up, const uint16_t *scales_up,
                               const uint32_t *qzeros_up, int group_size, int M, int N, int K, void *out,
                               int out_dtype, hipStream_t stream)
{
    const Matrix up{qweight_up, scales_up, qzeros_up};
    return prefill_call(A, Matrix{qweight_gate, scales_gate, qzeros_gate}, &up, group_size, M, N, K, out, out_dtype,
                        stream);
}

int w4a16_gemm_gate_up_ex(const void *A, const uint32_t *qweight_gate, const uint16_t *scales_gate,
                          const uint32_t *qzeros_gate, const uint32_t *qweight_up, const uint16_t *scales_up,
                          const uint32_t *qzeros_up, int group_size, int M, int N, int K, void *out, int out_dtype,
                          int splits, int waves_k, hipStream_t stream)
{
    const Matrix up{qweight_up, scales_up, qzeros_up};
    return gemm_call(A, Matrix{qweight_gate, scales_gate, qzeros_gate}, &up, group_size, M, N, K, out, out_dtype,
                     splits, waves_k, 0, nullptr, stream);
}

int w4a16_gemm_gate_up(const void *A, const uint32_t *qweight_gate, const uint16_t *scales_gate,
                       const uint32_t *qzeros_gate, const uint32_t *qweight_up, const uint16_t *scales_up,
                       const uint32_t *qzeros_up, int group_size, int M, int N, int K, void *out, int out_dtype,
                       hipStream_t stream)
{
    return w4a16_gemm_gate_up_ex(A, qweight_gate, scales_gate, qzeros_gate, qweight_up, scales_up, qzeros_up,
                                 group_size, M, N, K, out, out_dtype, 0, 0, stream);
}

int w4a16_gemm(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
               int group_size, int M, int N, int K, void *out, int out_dtype, hipStream_t stream)
{
    return w4a16_gemm_ex(A, qweight, scales, qzeros, group_size, M, N, K, out, out_dtype, 0, 0, 0, stream);
}

int w4a16_gemm_noalloc(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                       int group_size, int M, int N, int K, void *out, int out_dtype, hipStream_t stream)
{
    return gemm_call(A, Matrix{qweight, scales, qzeros}, nullptr, group_size, M, N, K, out, out_dtype, 0, 0, 0, nullptr,
                     stream, false, true);
}

int w4a16_gemm_affine_ex(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint16_t *biases,
                         int group_size, int M, int N, int K, void *out, int out_dtype, int splits, int waves_k,
                         int tile_cols, hipStream_t stream)
{
    if (!biases) return fail(W4A16_ERR_INVALID_ARG, "null pointer (biases)");
    Matrix w{qweight, scales, nullptr};
    w.biases = biases;
    return gemm_call(A, w, nullptr, group_size, M, N, K, out, out_dtype, splits, waves_k, tile_cols, nullptr, stream);
}

int w4a16_gemm_affine(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint16_t *biases,
                      int group_size, int M, int N, int K, void *out, int out_dtype, hipStream_t stream)
{
    return w4a16_gemm_affine_ex(A, qweight, scales, biases, group_size, M, N, K, out, out_dtype, 0, 0, 0, stream);
}

int w4a16_affine_split(const uint32_t *packed, int bits, const uint16_t *scales, const uint16_t *biases,
                       int group_size, int K, int N, uint32_t *qweight_out, uint16_t *scales_out, uint16_t *biases_out,
                       hipStream_t stream)
{
    if (!packed || !scales || !biases || !qweight_out || !scales_out || !biases_out)
        return fail(W4A16_ERR_INVALID_ARG, "null pointer");
    if (bits < 5 || bits > 8) return fail(W4A16_ERR_INVALID_ARG, "bits=%d outside 5..8", bits);
    if (K <= 0 || N <= 0 || K % 32 || N % 8 || K > (1 << 29))
        return fail(W4A16_ERR_INVALID_ARG, "K=%d N=%d", K, N);
    if (group_size <= 0 || group_size % 32 || K % group_size)
        return fail(W4A16_ERR_INVALID_ARG, "group_size=%d with K=%d", group_size, K);
    if ((long long)(2 * (long long)K / 8) * N > 0xFFFFFFFFLL)
        return fail(W4A16_ERR_UNSUPPORTED, "split planes of %lld words exceed 2^32 words", (long long)(K / 4) * N);
    if (!aligned16(packed) || !aligned16(scales) || !aligned16(biases) || !aligned16(qweight_out) ||
        !aligned16(scales_out) || !aligned16(biases_out))
        return fail(W4A16_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
    const hipError_t e =
        launch_affine_split(packed, bits, scales, biases, group_size, K, N, qweight_out, scales_out, biases_out, stream);
    if (e != hipSuccess) return hip_fail(e, "split launch");
    return W4A16_OK;
}

int w4a16_gemm_affine_split(const void *A, const uint32_t *qweight, const uint16_t *scales, const uint16_t *biases,
                            int group_size, int M, int N, int K, void *out, int out_dtype, hipStream_t stream)
{
    if (!qweight || !scales || !biases) return fail(W4A16_ERR_INVALID_ARG, "null pointer (qweight, scales or biases)");
    if (N <= 0 || K <= 0 || group_size <= 0 || group_size % 32 || K % group_size)
        return fail(W4A16_ERR_INVALID_ARG, "N=%d K=%d group_size=%d", N, K, group_size);
    // the two planes as a pair of matrices over the same activations, summed per column
    const size_t plane = (size_t)(K / 8) * N, groups = (size_t)(K / group_size) * N;
    Matrix lo{qweight, scales, nullptr};
    lo.biases = biases;
    Matrix hi{qweight + plane, scales + groups, nullptr};
    hi.biases = biases + groups;
    return gemm_call(A, lo, &hi, group_size, M, N, K, out, out_dtype, 0, 0, 0, nullptr, stream, true);
}

int w4a16_gemm_affine_gate_up(const void *A, const uint32_t *qweight_gate, const uint16_t *scales_gate,
                              const uint16_t *biases_gate, const uint32_t *qweight_up, const uint16_t *scales_up,
                              const uint16_t *biases_up, int group_size, int M, int N, int K, void *out,
                              int out_dtype, hipStream_t stream)
{
    if (!biases_gate || !biases_up) return fail(W4A16_ERR_INVALID_ARG, "null pointer (biases)");
    Matrix gate{qweight_gate, scales_gate, nullptr};
    gate.biases = biases_gate;
    Matrix up{qweight_up, scales_up, nullptr};
    up.biases = biases_up;
    return gemm_call(A, gate, &up, group_size, M, N, K, out, out_dtype, 0, 0, 0, nullptr, stream);
}

int w4a16_affine_widen(const uint32_t *packed, int bits, int K, int N, uint32_t *qweight, hipStream_t stream)
{
    if (!packed || !qweight) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
    if (bits < 1 || bits > 4) return fail(W4A16_ERR_INVALID_ARG, "bits=%d outside 1..4", bits);
    if (K <= 0 || N <= 0 || K % 32 || N % 8) return fail(W4A16_ERR_INVALID_ARG, "K=%d N=%d", K, N);
    if ((long long)(K / 8) * N > 0xFFFFFFFFLL)
        return fail(W4A16_ERR_UNSUPPORTED, "qweight of %lld words exceeds 2^32 words", (long long)(K / 8) * N);
    if (!aligned16(packed) || !aligned16(qweight)) return fail(W4A16_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
    const hipError_t e = launch_affine_widen(packed, bits, K, N, qweight, stream);
    if (e != hipSuccess) return hip_fail(e, "widen launch");
    return W4A16_OK;
}

int w4a16_plan(int M, int N, int K, int group_size, int *kernel, int *splits, int *waves_k, int *tile_cols)
{
    if (M < 1 || M > 16 || N <= 0 || K <= 0 || group_size <= 0 || group_size % 32 || K % group_size || N % 8)
        return fail(W4A16_ERR_INVALID_ARG, "invalid shape M=%d N=%d K=%d group_size=%d", M, N, K, group_size);
    if (decode_by_default(M, N, K, group_size, false, false)) {
        DecodePlan dp{};
        const int rc = make_decode_plan(M, N, K, group_size, false, 0, 0, 0, 0, 0, false, &dp);
        if (rc != W4A16_OK) return rc;
        if (kernel) *kernel = dp.mfma ? 3 : 2;
        if (splits) *splits = dp.slices;
        if (waves_k) *waves_k = dp.kw;
        if (tile_cols) *tile_cols = 16 * dp.cols;
        return W4A16_OK;
    }
    GemmPlan plan{};
    const int rc = make_plan(M, N, K, group_size, kZeroSym, 0, 0, 0, false, &plan);
    if (rc != W4A16_OK) return rc;
    if (kernel) *kernel = plan.mfma ? 1 : 0;
    if (splits) *splits = plan.splits;
    if (waves_k) *waves_k = plan.wk;
    if (tile_cols) *tile_cols = tile_columns(plan.cols);
    return W4A16_OK;
}

int w4a16_decode_plan(int M, int N, int K, int group_size, int packed_zeros, int slices, int tiles, int kw,
                      int tile_cols, int ring, int topk, int affine_bits, int *plan_out)
{
    if (affine_bits && ((!(affine_bits >= 1 && affine_bits <= 6) && affine_bits != 8) || packed_zeros))
        return fail(W4A16_ERR_INVALID_ARG, "affine_bits=%d is not 0, 1, 2, 3, 4, 5, 6 or 8, or comes with zero points",
                    affine_bits);
    if (M < 1 || M > 16 || N <= 0 || K <= 0 || group_size <= 0 || group_size % 32 || K % group_size || N % 8)
        return fail(W4A16_ERR_INVALID_ARG, "invalid shape M=%d N=%d K=%d group_size=%d", M, N, K, group_size);
    if (slices < 0 || tiles < 0 || kw < 0 || ring < 0)
        return fail(W4A16_ERR_INVALID_ARG, "slices=%d tiles=%d kw=%d ring=%d must be >= 0", slices, tiles, kw, ring);
    if (topk < 0 || topk > kDecMaxTopK) return fail(W4A16_ERR_INVALID_ARG, "k=%d outside 0..%d", topk, kDecMaxTopK);
    DecodePlan plan{};
    const int rc = make_decode_plan(M, N, K, group_size, packed_zeros != 0, slices, tiles, kw, tile_cols, ring,
                                    topk > 0, &plan, affine_bits);
    if (rc != W4A16_OK) return rc;
    if (plan_out) {
        plan_out[0] = plan.slices;
        plan_out[1] = plan.tiles;
        plan_out[2] = plan.kw;
        plan_out[3] = 16 * plan.cols;
        plan_out[4] = plan.ring;
        plan_out[6] = plan.sub;
        plan_out[5] = (int)plan.lds;
    }
    return W4A16_OK;
}

int w4a16_argmax_rows(const float *logits, int M, int N, int32_t *idx, hipStream_t stream)
{
    if (!logits || !idx) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
    if (M < 1 || M > 65535 || N < 1) return fail(W4A16_ERR_INVALID_ARG, "M=%d or N=%d out of range", M, N);
    if (!aligned16(logits)) return fail(W4A16_ERR_UNSUPPORTED, "logits must be 16-byte aligned");
    ArgmaxArgs a{};
    a.logits = logits;
    a.idx = idx;
    a.M = M;
    a.N = N;
    a.chunks = (int)(((long long)N + kArgmaxChunk - 1) / kArgmaxChunk);
    // counters: M uint32 counters followed by M 64-bit keys, all zero between calls
    const size_t need = round_up((size_t)M * 4, 8) + (size_t)M * 8;
    ScratchView v{};
    int rc = get_scratch(stream, need, 0, 0, 0, &v);
    if (rc != W4A16_OK) return rc;
    uint32_t *ctr = v.control;
    a.counters = ctr;
    a.keys = reinterpret_cast<unsigned long long *>(reinterpret_cast<char *>(ctr) + round_up((size_t)M * 4, 8));
    const hipError_t e = launch_argmax(a, stream);
    if (e != hipSuccess) return hip_fail(e, "argmax launch");
    return W4A16_OK;
}

int w4a16_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (!buf || !sink) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
    if (bytes == 0 || bytes % 16) return fail(W4A16_ERR_INVALID_ARG, "bytes=%zu is not a positive multiple of 16", bytes);
    if (bytes / (16 * 1024) >= 0x7FFFFFFFull)
        return fail(W4A16_ERR_UNSUPPORTED, "bytes=%zu needs more than 2^31 - 1 workgroups", bytes);
    if (!aligned16(buf)) return fail(W4A16_ERR_UNSUPPORTED, "buf must be 16-byte aligned");
    const hipError_t e = launch_stream_read(buf, (long long)bytes, sink, stream);
    if (e != hipSuccess) return hip_fail(e, "stream read launch");
    return W4A16_OK;
}

int w4a16_unpack_u8(const uint32_t *qweight, int K, int N, uint8_t *q_out, hipStream_t stream)
{
    if (!qweight || !q_out) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
    if (K <= 0 || N <= 0 || K % 8 || N % 4) return fail(W4A16_ERR_INVALID_ARG, "K=%d N=%d", K, N);
    if (!aligned16(qweight) || !aligned16(q_out)) return fail(W4A16_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
    const hipError_t e = launch_unpack_u8(qweight, K, N, q_out, stream);
    if (e != hipSuccess) return hip_fail(e, "unpack launch");
    return W4A16_OK;
}

int w4a16_dequant_f32(const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros, int group_size,
                      int K, int N, float *w_out, hipStream_t stream)
{
    if (!qweight || !scales || !w_out) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
    if (K <= 0 || N <= 0 || group_size <= 0 || group_size % 32 || K % group_size || N % 8)
        return fail(W4A16_ERR_INVALID_ARG, "K=%d N=%d group_size=%d", K, N, group_size);
    if (!aligned16(qweight) || !aligned16(scales) || (qzeros && !aligned16(qzeros)) || !aligned16(w_out))
        return fail(W4A16_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
    const hipError_t e = launch_dequant_f32(qweight, scales, qzeros, group_size, K, N, w_out, stream);
    if (e != hipSuccess) return hip_fail(e, "dequant launch");
    return W4A16_OK;
}

int w4a16_release_scratch(void)
{
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    int rc = W4A16_OK;
    for (auto &kv : g_scratch) {
        std::vector<void *> blocks = kv.second.retired;
        if (kv.second.base) blocks.push_back(kv.second.base);
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(kv.first.device);
        for (void *b : blocks) {
            const hipError_t e = hipFree(b);
            if (e != hipSuccess) rc = hip_fail(e, "hipFree");
        }
        (void)hipSetDevice(cur);
    }
    g_scratch.clear();
    return rc;
}

const char *w4a16_status_string(int status)
{
    switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_INVALID_ARG: return "invalid argument";
    case W4A16_ERR_UNSUPPORTED: return "unsupported (alignment, size, or scratch during capture)";
    case W4A16_ERR_HIP: return "HIP runtime error";
    case W4A16_ERR_NO_MEMORY: return "out of device memory";
    default: return "unknown status";
    }
}

const char *w4a16_last_error(void) { return g_last_error; }

int w4a16_version(void) { return 200; }

#ifndef W4A16_SOURCE_HASH
#define W4A16_SOURCE_HASH "unknown"
#endif
const char *w4a16_source_hash(void) { return W4A16_SOURCE_HASH; }

}  // extern "C"
