// W4A16 GEMV (M = 1) and small-M MFMA GEMM (M = 1..16) for gfx950.
//
// Work layout
//   * A column tile is one wave wide: 64 columns (4 adjacent columns per lane), or 128 (8 per
//     lane) for wide matrices. Lane l owns its columns' 16-byte loads of word row l / 16 of
//     every 4-row step, so one wave-wide load fetches 4 rows x 256 contiguous bytes.
//   * The `wk` waves of a workgroup share one column tile and split its K range into contiguous
//     pieces; their sums meet in LDS at the end.
//   * `splits` workgroups per tile split K further. Their fp32 partials are written with
//     agent-scope atomic stores and the workgroup that started last adds them in slice order,
//     so results are bit-identical from run to run. Because the partials are themselves
//     coherent atomic stores, publishing them needs no L2 write-back. The pages reduce split-K
//     through per-slice partials too on GPUs without thread-block clusters (TensorFold PR #859,
//     commit messages).
//
// Latency first. A wave lives for a few microseconds, only a handful of HBM round trips, so it
// starts all its memory traffic at once:
//   1. its activation slice into registers (or, for a long one-row slice, straight into LDS),
//      and the scales and zero points of its groups straight into LDS (global_load_lds);
//   2. a ring of kPf steps of packed weights into registers;
//   3. a wait for (1) only: loads retire in order, so "at most the ring outstanding" suffices;
//   4. the activations are rescaled and converted to fp16 and written to LDS once, while the
//      weights are still in flight.
// The ring then issues exactly one step per iteration (clamped past the wave's end), so the
// compiler waits for the oldest step only.
//
// Per step (32 K rows x one tile per wave)
//   * each packed word becomes 8 exact fp16 values (q - z) (w4a16_device.h);
//   * GEMV (one row, 64-column tiles): v_dot2c_f32_f16 into one fp32 sum per column; the four
//     word rows of a step are added across lanes at the end. Otherwise one
//     v_mfma_f32_16x16x32_f16 per word column (16 rows x 16 columns x 32 K), activations padded
//     with zero rows up to 16;
//   * sums are kept per quantisation group and scaled once at the group's end.
//
// Activations are fp16 after an exact per-row power-of-two rescale chosen from the row's largest
// exponent over the wave's K range. A slice too large to stage without costing waves per CU is
// prepared once per call by act_prep_kernel instead, and its fragments stream in with the
// weights.
//
// Why this shape (GRIMOIRE v1.7 release notes, 'What changed': a GEMV for one user and a
// matrix-engine GEMM for 2-16 rows; GRIMOIRE v1.8, 'What changed': the small-row kernel got
// faster from register budgeting and from splitting work over more threads): every
// configuration is bound by streaming the packed weights from HBM, so the VALU work is only
// the exact dequantisation and the weight loads stay in flight from the first instructions on.
#include <type_traits>

#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {
namespace {

// Activation items (16 bytes) a lane may stage through registers: 8 KB per wave.
constexpr int kHeld = 8;

// The K range [wb, we) (in steps) of piece `wave` of split `split`: splits cut K into
// contiguous slices, the waves of a workgroup cut each slice again. The activation preparation
// kernel and the GEMM compute the same ranges.
__device__ __forceinline__ void piece_range(int steps, int splits, int wk, int split, int wave, int &wb, int &we)
{
    const int sb = (int)((long long)split * steps / splits);
    const int se = (int)((long long)(split + 1) * steps / splits);
    wb = sb + (int)((long long)wave * (se - sb) / wk);
    we = sb + (int)((long long)(wave + 1) * (se - sb) / wk);
}

// Activation preparation for the matrix-core path, once per call instead of once per column
// tile: for each K piece of the launch and each row, the largest bf16 exponent gives the
// power-of-two rescale (see act_shift), and the piece's activations are stored as fp16 in the
// packed-word slot order with that rescale applied. One wave per (piece, row): its items stay
// in registers, the row maximum is a wave reduction, and no LDS or barrier is involved.
constexpr int kPrepWaves = 4;   // rows per workgroup
constexpr int kPrepHeld = 4;    // items (16 bytes) a lane keeps in registers between the passes

__global__ __launch_bounds__(kPrepWaves * 64) void act_prep_kernel(ActPrepArgs p)
{
    const int piece = blockIdx.x;
    const int m = blockIdx.y * kPrepWaves + (int)(threadIdx.x >> 6);
    if (m >= p.M) return;   // whole waves: no barrier follows
    const int lane = threadIdx.x & 63;
    const int split = piece / p.wk;
    const int wave = piece - split * p.wk;
    int wb, we;
    piece_range(p.K / kStepK, p.splits, p.wk, split, wave, wb, we);
    const int nwr = (we - wb) * 4;   // word rows (16-byte items) of the row in this piece
    const size_t base = (size_t)m * p.K + (size_t)wb * 4 * 8;
    // Largest magnitude: the first kPrepHeld x 64 items stay in registers for the conversion;
    // a longer piece reads the rest twice.
    uint4 held[kPrepHeld];
    uint32_t mag = 0;
#pragma unroll
    for (int u = 0; u < kPrepHeld; ++u) {
        const int it = lane + 64 * u;
        held[u] = uint4{0u, 0u, 0u, 0u};
        if (it < nwr) {
            held[u] = *reinterpret_cast<const uint4 *>(p.A + base + (size_t)it * 8);
            mag = max(mag, max_mag8(held[u]));
        }
    }
    for (int it = lane + 64 * kPrepHeld; it < nwr; it += 64)
        mag = max(mag, max_mag8(*reinterpret_cast<const uint4 *>(p.A + base + (size_t)it * 8)));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, o));
    const int sh = act_shift(mag >> 7);
    if (lane == 0) p.shifts[(size_t)piece * p.M + m] = sh;
    const float mul = pow2_neg(sh);
#pragma unroll
    for (int u = 0; u < kPrepHeld; ++u) {
        const int it = lane + 64 * u;
        if (it < nwr)
            *reinterpret_cast<uint4 *>(p.A16 + base + (size_t)it * 8) = __builtin_bit_cast(uint4, act8_to_slots(held[u], mul));
    }
    for (int it = lane + 64 * kPrepHeld; it < nwr; it += 64) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(p.A + base + (size_t)it * 8);
        *reinterpret_cast<uint4 *>(p.A16 + base + (size_t)it * 8) = __builtin_bit_cast(uint4, act8_to_slots(raw, mul));
    }
}

// Occupancy the register allocator must keep (waves per SIMD; 1 = no constraint). Left to
// itself it moves the 64-column matrix-core kernels' accumulators into AGPRs whenever a
// workgroup has at most 4 waves, which costs two waves per SIMD. Affine codes hold one more
// accumulator and the biases: at 7 they would spill.
template <bool kMfma, int kZM, int kC>
constexpr int gemm_min_waves()
{
    return kMfma && kC == 4 ? (kZM == kZeroPacked ? 5 : kZM == kAffine ? 6 : 7) : 1;
}

// kLdsA: the wave stages its activation slice in LDS and converts it itself. Otherwise (a
// slice too large to stage) the activations come prepared by act_prep_kernel -- fp16, slot
// order, rescaled per piece and row -- and stream in with the weights, one fragment per step.
// kDual: a gated pair (gate in qweight, up in qweight2, same shape). A lane's 8 columns are 4
// output columns of the gate followed by the same 4 of the up projection, so a tile covers 64
// output columns of both, the activations are staged and converted once for the two, and the
// epilogue writes silu(gate) * up. Internally the pair is a 2N-column problem whose column c of
// a tile is output column (c / 8) * 4 + c % 4 of matrix (c / 4) % 2. With p.pair_sum the pair is
// summed instead, out = (A x W) + (A x W2): the low and high 4-bit planes of wider affine codes.
// kZM (ZeroMode): for affine codes, w = s * q + b, the sum of a group is
// s * sum(a * q) + b * sum(a): the codes go through the same exact conversion with zero point
// 0, and sum(a) over the group comes from one more product per step against a fragment of ones
// (the matrix cores are not the bound at these row counts).
template <bool kMfma, int kZM, bool kLdsA, int kWK, int kPf, int kC, bool kDual = false>
__global__ __launch_bounds__(kWK * 64)
__attribute__((amdgpu_waves_per_eu(gemm_min_waves<kMfma, kZM, kC>()))) void w4a16_gemm_kernel(GemmArgs p)
{
    static_assert(!kDual || (kMfma && kC == 8), "gated pairs run on the matrix cores, 8 columns per lane");
    constexpr bool kAff = kZM == kAffine;
    // how a pair's two sums of one output column meet (uniform over the launch)
    const bool pair_sum = p.pair_sum != 0;
    auto combine = [pair_sum](float g, float u) { return pair_sum ? g + u : silu_f32(g) * u; };
    constexpr bool kPreA = !kLdsA;
    constexpr int kTile = 16 * kC;      // columns per tile: kC adjacent columns per lane
    constexpr int kOutTile = kDual ? kTile / 2 : kTile;   // output columns per tile
    constexpr int kV = kC / 4;          // 16-byte weight loads per lane per step
    constexpr int kZW = kTile / 8;      // zero words (and 8-scale items) per group
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_last;
    __shared__ unsigned long long s_rowkey[16];   // fused argmax: best key per row of the tile

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: K-range math stays scalar
    const int cl = lane & 15;   // column block (and MFMA A row) of this lane
    const int rl = lane >> 4;   // word row within the step
    const int M = p.M;
    const int N = p.N;
    const int K = p.K;
    const int spg = p.g / kStepK;   // steps per quantisation group
    const int tile = blockIdx.x;
    const int split = blockIdx.y;
    // Split-K: count this workgroup in at the start; the answer is needed only at the end, and
    // the workgroup that starts last becomes the one that adds the slices.
    uint32_t arrival = 0;
    if (p.splits > 1 && tid == 0)
        arrival = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int steps = K / kStepK;
    int wb, we;   // we > wb (host)
    piece_range(steps, p.splits, kWK, split, wave, wb, we);
    const int piece = split * kWK + wave;
    const int g0 = wb / spg;                  // first group of the wave
    const int ng = (we - 1) / spg - g0 + 1;   // groups touched by the wave

    // LDS: [kWK x (16 row shifts, 16 row multipliers)][per wave: activations | scales | zeros]
    int *shift_lds = reinterpret_cast<int *>(smem) + wave * kRowHeader;
    float *mul_lds = reinterpret_cast<float *>(shift_lds + 16);
    unsigned char *region = smem + kWK * kRowHeader * sizeof(int);
    unsigned char *wreg = region + (size_t)wave * p.wave_lds;
    uint4 *a_lds = reinterpret_cast<uint4 *>(wreg);                                // [word row][M]
    uint16_t *sc_lds = reinterpret_cast<uint16_t *>(wreg + p.scale_off);           // [group][64]
    uint32_t *z_lds = reinterpret_cast<uint32_t *>(wreg + p.zero_off);             // [group][8]
    uint16_t *b_lds = reinterpret_cast<uint16_t *>(wreg + p.zero_off);             // affine: [group][64]

    const int n0 = tile * kOutTile + cl * (kDual ? 4 : kC);   // the lane's first output column
    const bool col_ok = n0 < N;
    const int nc = col_ok ? n0 : 0;       // clamped column for loads of dead lanes
    const int arow = cl < M ? cl : 0;     // clamped activation row (MFMA fragments)
    const uint32_t *qw_lane = p.qweight + (size_t)rl * N + nc;
    const uint32_t *qw2_lane = kDual ? p.qweight2 + (size_t)rl * N + nc : qw_lane;   // up columns
    const uint16_t *asrc = kPreA ? p.A16 : p.A;   // prepared fp16 or raw bf16
    const uint16_t *a_lane = asrc + (size_t)arow * K + rl * 8;
    int pre_shift = 0;   // prepared path: this piece's rescale of row `lane`
    if (kPreA && lane < M) pre_shift = p.ashift[(size_t)piece * M + lane];

    const int nwr = (we - wb) * 4;   // packed word rows in the wave's range
    const int items = M * nwr;       // 16-byte activation items, item = word row * M + row
    int pre_loads = 0;               // vector memory operations issued before the ring
    // 64 items are dq word rows and dr rows: the register path gives each lane the fixed row
    // m_l (below); the direct-to-LDS path walks the items 64 at a time and tracks each item's
    // (word row, row) with adds. Neither divides by M per item.
    const int dq = 64 / M;
    const int dr = 64 - dq * M;
    const int wr_l = lane / M;
    const int m_l = lane - wr_l * M;

    // ---- 1. small operands: activations into registers, scales and zeros straight into LDS ---
    // A slice of at most kHeld items per lane is loaded into registers, reduced and converted
    // there, and written to LDS once as fp16. There every lane keeps one row: lane l takes row
    // l % M and word rows l / M + i * dq, so item l + i * dq * M (lanes from dq * M on idle when M
    // does not divide 64). A longer slice (long one-row pieces) goes into LDS by direct loads
    // and is reduced and converted in place.
    const bool held = (nwr + dq - 1) / dq <= kHeld;   // uniform
    const bool lane_on = lane < dq * M;
    uint4 held_a[kHeld];
    auto held_ok = [&](int i) { return lane_on && wr_l + i * dq < nwr; };
    if (kLdsA) {
        int wr = wb * 4 + wr_l, m = m_l;
        if (held) {
#pragma unroll
            for (int i = 0; i < kHeld; ++i) {
                held_a[i] = uint4{0u, 0u, 0u, 0u};
                if (i * dq < nwr && held_ok(i))   // (uniform, then per lane)
                    held_a[i] = *reinterpret_cast<const uint4 *>(asrc + (size_t)m_l * K + (size_t)(wr + i * dq) * 8);
            }
        } else {
            for (int b = 0; b < items; b += 64) {
                if (b + lane < items) load_to_lds16(asrc + (size_t)m * K + (size_t)wr * 8, a_lds + b);
                ++pre_loads;
                wr += dq;
                m += dr;
                if (m >= M) {
                    m -= M;
                    ++wr;
                }
            }
        }
    }
    if constexpr (kDual) {   // scales: 64 pairs per group, in lane order [cl][gate 4 | up 4]
        const int sitems = ng * 64;
        for (int b = 0; b < sitems; b += 64) {
            const int gi = g0 + b / 64;
            const int j = (2 * lane) & 7;   // first slot of the pair within the lane's 8
            int c = tile * kOutTile + (lane >> 2) * 4 + (j & 3);
            if (c >= N) c = 0;
            load_to_lds4((j < 4 ? p.scales : p.scales2) + (size_t)gi * N + c, sc_lds + (size_t)b * 2);
            ++pre_loads;
            if constexpr (kAff) {   // the biases in the same order
                load_to_lds4((j < 4 ? p.biases : p.biases2) + (size_t)gi * N + c, b_lds + (size_t)b * 2);
                ++pre_loads;
            }
        }
    } else {   // scales (affine: and biases): kZW items of 8 columns per group (lanes past the last
        // item stay idle, so the LDS area holds exactly the wave's groups)
        const int sitems = ng * kZW;
        for (int b = 0; b < sitems; b += 64) {
            const int it = b + lane;
            const int gi = g0 + it / kZW;
            int c = tile * kTile + (it % kZW) * 8;
            if (c >= N) c = 0;
            if (it < sitems) load_to_lds16(p.scales + (size_t)gi * N + c, sc_lds + (size_t)b * 8);
            ++pre_loads;
            if constexpr (kAff) {
                if (it < sitems) load_to_lds16(p.biases + (size_t)gi * N + c, b_lds + (size_t)b * 8);
                ++pre_loads;
            }
        }
    }
    if constexpr (kZM == kZeroPacked) {   // zero words: kZW per group (8 columns each; a pair: 8 gate words, 8 up words)
        const int zitems = ng * kZW;
        for (int b = 0; b < zitems; b += 64) {
            const int it = b + lane;
            const int gi = g0 + it / kZW;
            const int w = it % kZW;
            int c = kDual ? tile * kOutTile + (w & 7) * 8 : tile * kTile + w * 8;
            if (c >= N) c = 0;
            const uint32_t *zsrc = kDual && w >= 8 ? p.qzeros2 : p.qzeros;
            if (it < zitems) load_to_lds4(zsrc + (size_t)gi * (N / 8) + c / 8, z_lds + b);
            ++pre_loads;
        }
    }

    if (lane < 16) shift_lds[lane] = 0;
    asm volatile("" ::: "memory");

    // ---- 2. the weight ring -------------------------------------------------------------------
    uint4 ring_w[kPf][kV];
    uint4 ring_a[kLdsA ? 1 : kPf];
    auto load_w = [&](uint4 *dst, int t) {
#pragma unroll
        for (int v = 0; v < kV; ++v)   // word offsets fit 32 bits (checked on the host)
            dst[v] = kDual ? *reinterpret_cast<const uint4 *>((v ? qw2_lane : qw_lane) + (uint32_t)t * 4u * (uint32_t)N)
                           : *reinterpret_cast<const uint4 *>(qw_lane + (uint32_t)t * 4u * (uint32_t)N + 4 * v);
    };
#pragma unroll
    for (int u = 0; u < kPf; ++u) {
        const int t = min(wb + u, we - 1);
        load_w(ring_w[u], t);
        if (!kLdsA) ring_a[u] = *reinterpret_cast<const uint4 *>(a_lane + (size_t)t * kStepK);
    }
    asm volatile("" ::: "memory");

    // ---- 3./4. wait for the staged operands only, then rescale and convert the activations -------
    // (the ring holds kPf steps of kV weight loads, plus one activation fragment each when unstaged)
    if (pre_loads) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPf * (kV + (kLdsA ? 0 : 1))));
    asm volatile("" ::: "memory");
    if (kLdsA) {   // each row's largest magnitude (its largest exponent), then its rescale
        uint32_t run = 0;
        int m = m_l;
        auto fold = [&](uint32_t mag) {
            run = max(run, mag);
            if (dr) {   // the row changes from one item of the lane to the next
                if (run) atomicMax(&shift_lds[m], (int)run);
                run = 0;
                m += dr;
                if (m >= M) m -= M;
            }
        };
        if (held) {   // the lane's row is fixed: a packed running maximum, its halves folded once
            uint32_t pk = 0;
#pragma unroll
            for (int i = 0; i < kHeld; ++i)
                if (i * dq < nwr && held_ok(i)) pk = max_mag8_packed(held_a[i], pk);
            run = max(pk & 0xFFFFu, pk >> 16);
        } else {
            for (int it = lane; it < items; it += 64) fold(max_mag8(a_lds[it]));
        }
        if (run) atomicMax(&shift_lds[m], (int)run);
    }
    if (lane < M) {
        const int sh = kPreA ? pre_shift : act_shift((uint32_t)shift_lds[lane] >> 7);
        shift_lds[lane] = sh;
        mul_lds[lane] = pow2_neg(sh);
    }
    if (kLdsA) {
        int m = m_l;
        if (held) {   // one multiplier per lane (its row)
            const float mul = lane_on ? mul_lds[m_l] : 0.f;
#pragma unroll
            for (int i = 0; i < kHeld; ++i)
                if (i * dq < nwr && held_ok(i))
                    a_lds[lane + i * dq * M] = __builtin_bit_cast(uint4, act8_to_slots(held_a[i], mul));
        } else {
            for (int it = lane; it < items; it += 64) {
                a_lds[it] = __builtin_bit_cast(uint4, act8_to_slots(a_lds[it], mul_lds[m]));
                m += dr;
                if (m >= M) m -= M;
            }
        }
    }

    // ---- stream ------------------------------------------------------------------------
    const Masks mk = make_masks();
    const half8_t zero8 = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    float4_t acc[kC];
    float4_t tot[kC];
#pragma unroll
    for (int j = 0; j < kC; ++j) {
        acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
        tot[j] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    ZeroSub zs[kC];
#pragma unroll
    for (int j = 0; j < kC; ++j) zs[j] = kAff ? zero_sub(0u) : zero_sub_sym();
    float4_t acc1 = float4_t{0.f, 0.f, 0.f, 0.f};   // affine: the group's activation sums per row
    const half8_t ones = half8_t{1, 1, 1, 1, 1, 1, 1, 1};
    // Position in the quantisation groups, kept by counting (all wave-uniform): step t is step
    // gpos of group gi, and `first` marks the first step of the wave's part of a group.
    int gi = g0;
    int gpos = wb - g0 * spg;
    bool first = true;

    // One step: dequantise the ring slot's words, multiply, and scale at a group's end.
    auto step = [&](int t, const uint4 *wv, const uint4 av) {
        const bool last = gpos == spg - 1 || t + 1 == we;
        half8_t a;
        if (kLdsA) {
            const int wrow = (t - wb) * 4 + rl;
            if (kMfma) {
                a = zero8;
                if (cl < M) a = __builtin_bit_cast(half8_t, a_lds[wrow * M + cl]);
            } else {
                a = __builtin_bit_cast(half8_t, a_lds[wrow]);
            }
        } else {
            a = __builtin_bit_cast(half8_t, av);   // prepared fragment
            if (cl >= M) a = zero8;
        }
        if (kZM == kZeroPacked && first) {   // zero points change once per group (uniform)
            if constexpr (kDual) {
                const uint32_t *zg = z_lds + (gi - g0) * kZW + (cl >> 1);
                const uint32_t zw0 = zg[0], zw1 = zg[8];   // gate, up
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    zs[j] = zero_sub(zero_of(zw0, (uint32_t)(nc + j)));
                    zs[4 + j] = zero_sub(zero_of(zw1, (uint32_t)(nc + j)));
                }
            } else {
                const uint32_t zw = z_lds[(gi - g0) * kZW + (cl * kC) / 8];
#pragma unroll
                for (int j = 0; j < kC; ++j) zs[j] = zero_sub(zero_of(zw, (uint32_t)(nc + j)));
            }
        }
        uint32_t words[kC];
#pragma unroll
        for (int v = 0; v < kV; ++v) {
            words[4 * v] = wv[v].x;
            words[4 * v + 1] = wv[v].y;
            words[4 * v + 2] = wv[v].z;
            words[4 * v + 3] = wv[v].w;
        }
#pragma unroll
        for (int j = 0; j < kC; ++j) {
            const half8_t b = dequant_word(words[j], kZM == kZeroSym ? zero_sub_sym() : zs[j], mk);
            if (kMfma) {
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
            } else {
                float s = acc[j][0];
                s = __builtin_amdgcn_fdot2(b.lo.lo, a.lo.lo, s, false);
                s = __builtin_amdgcn_fdot2(b.lo.hi, a.lo.hi, s, false);
                s = __builtin_amdgcn_fdot2(b.hi.lo, a.hi.lo, s, false);
                s = __builtin_amdgcn_fdot2(b.hi.hi, a.hi.hi, s, false);
                acc[j][0] = s;
            }
        }
        if constexpr (kAff) {
            if (kMfma) {
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, acc1, 0, 0, 0);
            } else {
                float s = acc1[0];
                s = __builtin_amdgcn_fdot2(ones.lo.lo, a.lo.lo, s, false);
                s = __builtin_amdgcn_fdot2(ones.lo.hi, a.lo.hi, s, false);
                s = __builtin_amdgcn_fdot2(ones.hi.lo, a.hi.lo, s, false);
                s = __builtin_amdgcn_fdot2(ones.hi.hi, a.hi.hi, s, false);
                acc1[0] = s;
            }
        }
        if (last) {
            const uint16_t *sp = sc_lds + (gi - g0) * kTile + cl * kC;
            uint32_t sw[kC / 2];
            if constexpr (kC == 4) {
                const uint2 v = *reinterpret_cast<const uint2 *>(sp);
                sw[0] = v.x;
                sw[1] = v.y;
            } else {   // the lane's 8 scales
                const uint4 q = *reinterpret_cast<const uint4 *>(sp);
                sw[0] = q.x;
                sw[1] = q.y;
                sw[2] = q.z;
                sw[3] = q.w;
            }
            float s4[kC];
#pragma unroll
            for (int j = 0; j < kC; ++j) {
                const uint32_t bits = (sw[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
                s4[j] = kAff ? bf16_bits_to_float(bits) : half_bits_to_float(bits);
            }
            if constexpr (kAff) {   // the bias term first: b * sum(a), per row
                const uint16_t *bp = b_lds + (gi - g0) * kTile + cl * kC;
                uint32_t bw[kC / 2];
#pragma unroll
                for (int i = 0; i < kC / 2; ++i) bw[i] = reinterpret_cast<const uint32_t *>(bp)[i];
#pragma unroll
                for (int j = 0; j < kC; ++j) {
                    const float bj = bf16_bits_to_float((bw[j / 2] >> (16 * (j & 1))) & 0xFFFFu);
#pragma unroll
                    for (int r = 0; r < (kMfma ? 4 : 1); ++r) tot[j][r] = __builtin_fmaf(acc1[r], bj, tot[j][r]);
                }
                acc1 = float4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < kC; ++j) {
                if (kMfma) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) tot[j][r] = __builtin_fmaf(acc[j][r], s4[j], tot[j][r]);
                    acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
                } else {
                    tot[j][0] = __builtin_fmaf(acc[j][0], s4[j], tot[j][0]);
                    acc[j][0] = 0.f;
                }
            }
        }
        first = last;
        if (++gpos == spg) {
            gpos = 0;
            ++gi;
        }
    };

    // Whole rounds of the ring: every step computes and reissues its slot unconditionally, so
    // the compiler's wait before each step covers exactly that slot (a skipped step would leave
    // a load in flight into the registers being reloaded and force a full wait).
    const int full_end = wb + (we - wb) / kPf * kPf;
    int t0 = wb;
    for (; t0 < full_end; t0 += kPf) {
#pragma unroll
        for (int u = 0; u < kPf; ++u) {
            const int t = t0 + u;
            step(t, ring_w[u], ring_a[kLdsA ? 0 : u]);
            const int tn = min(t + kPf, we - 1);
            load_w(ring_w[u], tn);
            if (!kLdsA) ring_a[u] = *reinterpret_cast<const uint4 *>(a_lane + (size_t)tn * kStepK);
        }
    }
    // The last (we - wb) % kPf steps are already in the ring's first slots.
#pragma unroll
    for (int u = 0; u + 1 < kPf; ++u)
        if (t0 + u < we) step(t0 + u, ring_w[u], ring_a[kLdsA ? 0 : u]);

    // ---- this wave's sums: add the word rows (GEMV), undo the activation rescale ---------------
    // GEMM: lane holds rows 4*rl + r of its 4 columns. GEMV: lanes with rl == 0 hold row 0.
    constexpr int kRows = kMfma ? 4 : 1;
    if (!kMfma) {
#pragma unroll
        for (int j = 0; j < kC; ++j) {
            float v = tot[j][0];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            tot[j][0] = v;
        }
    }
    const int row_base = kMfma ? 4 * rl : 0;
    const bool holder = kMfma || rl == 0;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int m = row_base + r;
        const int sh = m < M ? shift_lds[m] : 0;
#pragma unroll
        for (int j = 0; j < kC; ++j) tot[j][r] = __builtin_amdgcn_ldexpf(tot[j][r], sh);
    }

    auto store_out = [&](int m, int n, float v) {
        if (p.out_bf16)
            static_cast<uint16_t *>(p.out)[(size_t)m * N + n] = (uint16_t)float_to_bf16_bits(v);
        else
            static_cast<float *>(p.out)[(size_t)m * N + n] = v;
    };

    const bool amax = p.amax_keys != nullptr;   // fused greedy pick (output layer)
    if (kWK == 1 && p.splits == 1 && !amax) {
        if (!holder || !col_ok) return;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int m = row_base + r;
            if (m >= M) break;
            const size_t o = (size_t)m * N + n0;
#pragma unroll
            for (int v = 0; v < (kDual ? 1 : kV); ++v) {
                float x0 = tot[4 * v][r], x1 = tot[4 * v + 1][r], x2 = tot[4 * v + 2][r], x3 = tot[4 * v + 3][r];
                if constexpr (kDual) {   // silu(gate) * up, or the sum of an affine pair
                    x0 = combine(x0, tot[4][r]);
                    x1 = combine(x1, tot[5][r]);
                    x2 = combine(x2, tot[6][r]);
                    x3 = combine(x3, tot[7][r]);
                }
                if (p.out_bf16) {
                    uint2 q;
                    q.x = float_to_bf16_bits(x0) | (float_to_bf16_bits(x1) << 16);
                    q.y = float_to_bf16_bits(x2) | (float_to_bf16_bits(x3) << 16);
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + o + 4 * v) = q;
                } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o + 4 * v) = make_float4(x0, x1, x2, x3);
                }
            }
        }
        return;
    }

    // ---- cross-wave reduction in LDS, in wave order ---------------------------------------
    float *red = reinterpret_cast<float *>(region);   // [kWK][M][kTile] over the dead staging areas
    __syncthreads();
    if (holder) {
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int m = row_base + r;
            if (m < M) {
                float *dst = red + ((size_t)wave * M + m) * kTile + cl * kC;
#pragma unroll
                for (int v = 0; v < kV; ++v)
                    *reinterpret_cast<float4_t *>(dst + 4 * v) =
                        float4_t{tot[4 * v][r], tot[4 * v + 1][r], tot[4 * v + 2][r], tot[4 * v + 3][r]};
            }
        }
    }
    if (p.splits > 1 && tid == 0) s_last = arrival == (uint32_t)(p.splits - 1);
    if (tid < 16) s_rowkey[tid] = 0;
    __syncthreads();
    constexpr int kThreads = kWK * 64;
    auto wg_sum = [&](int m, int c) {
        float v = red[(size_t)m * kTile + c];
#pragma unroll
        for (int w = 1; w < kWK; ++w) v += red[((size_t)w * M + m) * kTile + c];
        return v;
    };
    // Fused greedy pick: every finished output of the tile folds into its row's key in LDS, and
    // the tile stores its keys to its own slot of the call's keys (plain stores: no atomics on
    // shared words, which serialise when many tiles merge into the same few rows); the finishing
    // kernel next on the stream takes each row's largest key over the slots (the keys of
    // argmax_rows_kernel, so the pick equals its pick over the fp32 outputs). All lanes of a wave
    // hold outputs of one row (a tile's width is a multiple of 64), so the keys are first reduced
    // across the wave and one LDS atomic per wave folds them in: emit is called by every lane of
    // the wave together, with `ok` false for columns past N.
    auto emit = [&](int m, int n, float v, bool ok) {
        if (ok) store_out(m, n, v);
        if (amax) {
            unsigned long long k = ok && v == v ? argmax_key(v, (uint32_t)n) : 0ull;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const unsigned long long other = shfl_xor_u64(k, o);
                k = other > k ? other : k;
            }
            if (lane == 0 && k) atomicMax(&s_rowkey[m], k);
        }
    };
    auto finish_argmax = [&]() {
        __syncthreads();
        if (tid < M) p.amax_keys[(size_t)tile * 16 + tid] = s_rowkey[tid];
    };
    // Column c of the tile: its place in the split-K partials (2N wide for a gated pair),
    // whether it holds an output, and where its finished sum goes -- out, or for a gated pair
    // into LDS over the thread's own slot of wave 0's sums (only that thread reads the slot)
    // until silu(gate) * up is formed.
    const size_t NV = kDual ? 2 * (size_t)N : (size_t)N;
    auto col_valid = [&](int c) { return kDual ? tile * kOutTile + (c >> 3) * 4 < N : tile * kTile + c < N; };
    auto put = [&](int m, int c, float v, bool ok) {
        if constexpr (kDual)
            red[(size_t)m * kTile + c] = v;
        else
            emit(m, tile * kTile + c, v, ok);
    };
    auto finish_pair = [&]() {
        __syncthreads();
        for (int idx = tid; idx < M * kOutTile; idx += kThreads) {
            const int m = idx / kOutTile;
            const int oc = idx - m * kOutTile;
            const int n = tile * kOutTile + oc;
            const float *fin = red + (size_t)m * kTile + (oc >> 2) * 8 + (oc & 3);   // gate; up 4 further
            if (n < N) store_out(m, n, combine(fin[0], fin[4]));
        }
    };
    if (p.splits == 1) {
        for (int idx = tid; idx < M * kTile; idx += kThreads) {
            const int m = idx / kTile;
            const int c = idx - m * kTile;
            put(m, c, wg_sum(m, c), col_valid(c));
        }
        if (kDual) finish_pair();
        if (amax) finish_argmax();
        return;
    }

    // ---- split-K across workgroups ---------------------------------------------------------
    // Every workgroup of the tile counted itself in on the tile's counter when it started; the
    // last one to start adds the slices. The others store their slice into the split-K
    // exchange as fp32 with agent-scope atomic stores and are done: nothing to wait for, no
    // flag. The reducer reads each other slice's slot again until it no longer holds
    // kSliceEmpty, adds the slices in slice order (bit-identical results from run to run), writes
    // kSliceEmpty back into every slot it took and lowers the counter. The exchange and the
    // counters are therefore as they were before the call whatever the call was: no state
    // carries from one call to the next, so a call replayed from a captured graph runs exactly as
    // it ran when it was captured.
    const size_t slice = (size_t)M * NV;
    uint32_t *const ex = reinterpret_cast<uint32_t *>(p.partials);   // slots as bits
    if (!s_last) {
        for (int idx = tid; idx < M * kTile; idx += kThreads) {
            const int m = idx / kTile;
            const int c = idx - m * kTile;
            if (col_valid(c))
                __hip_atomic_store(ex + (size_t)split * slice + (size_t)m * NV + tile * kTile + c,
                                   __builtin_bit_cast(uint32_t, wg_sum(m, c)), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    constexpr int kBatch = 8;
    for (int idx = tid; idx < M * kTile; idx += kThreads) {
        const int m = idx / kTile;
        const int c = idx - m * kTile;
        const bool in = col_valid(c);
        const float own = wg_sum(m, c);
        uint32_t *const col = ex + (size_t)m * NV + tile * kTile + c;
        float v = 0.f;
        bool failed = false;
        for (int sp0 = 0; in && sp0 < p.splits; sp0 += kBatch) {
            auto taken = [&](int i) { return sp0 + i < p.splits && sp0 + i != split; };
            uint32_t x[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                x[i] = taken(i) ? __hip_atomic_load(col + (size_t)(sp0 + i) * slice, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : __builtin_bit_cast(uint32_t, own);
            for (uint32_t spins = 0;;) {   // until every slot of the batch has arrived
                bool wait = false;
#pragma unroll
                for (int i = 0; i < kBatch; ++i) wait |= taken(i) && x[i] == kSliceEmpty;
                if (!wait) break;
                if (++spins == kSpinLimit) {   // cannot happen while every workgroup runs to its end
                    failed = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
                    if (taken(i) && x[i] == kSliceEmpty)
                        x[i] = __hip_atomic_load(col + (size_t)(sp0 + i) * slice, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                if (sp0 + i < p.splits) v += __builtin_bit_cast(float, x[i]);
#pragma unroll
            for (int i = 0; i < kBatch; ++i)   // the slots are empty again
                if (taken(i))
                    __hip_atomic_store(col + (size_t)(sp0 + i) * slice, kSliceEmpty, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
        put(m, c, failed ? __builtin_nanf("") : v, in);
    }
    if (kDual) finish_pair();
    if (amax) finish_argmax();
    if (tid == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Ends a fused greedy pick: one workgroup per row takes the largest key over the slots of the
// tiles (or column groups), turns it into an index (0 when the row held no number), and clears
// the row's slots (the control words are zero between calls). Runs after the GEMM on its stream,
// so every slot has been stored.
constexpr int kFinishThreads = 256;
constexpr int kFinishBatch = 8;
__global__ __launch_bounds__(kFinishThreads) void argmax_slots_finish_kernel(unsigned long long *keys, int slots,
                                                                            int32_t *idx)
{
    __shared__ unsigned long long s_best[kFinishThreads / 64];
    const int m = blockIdx.x;
    unsigned long long best = 0ull;
    // each thread reads its own slots, kFinishBatch loads in flight, then clears them
    for (int s0 = threadIdx.x; s0 < slots; s0 += kFinishBatch * kFinishThreads) {
        unsigned long long k[kFinishBatch];
#pragma unroll
        for (int b = 0; b < kFinishBatch; ++b) {
            const int s = s0 + b * kFinishThreads;
            k[b] = s < slots ? keys[(size_t)s * 16 + m] : 0ull;
        }
#pragma unroll
        for (int b = 0; b < kFinishBatch; ++b) {
            const int s = s0 + b * kFinishThreads;
            best = k[b] > best ? k[b] : best;
            if (s < slots) keys[(size_t)s * 16 + m] = 0ull;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long other = shfl_xor_u64(best, o);
        best = other > best ? other : best;
    }
    if ((threadIdx.x & 63) == 0) s_best[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kFinishThreads / 64; ++w) best = s_best[w] > best ? s_best[w] : best;
        idx[m] = best ? (int32_t)(0xFFFFFFFFu - (uint32_t)best) : 0;
    }
}

}  // namespace
hipError_t launch_act_prep(const ActPrepArgs &pa, hipStream_t stream);
namespace {

template <bool kMfma, int kZM, bool kLdsA, int kWK, int kC, bool kDual>
hipError_t launch_one(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream)
{
    constexpr int kPf = kLdsA ? kRingStaged : ring_unstaged<kZM, kC>();
    constexpr int kOutTile = kDual ? 8 * kC : 16 * kC;
    const auto kern = w4a16_gemm_kernel<kMfma, kZM, kLdsA, kWK, kPf, kC, kDual>;
    if (!kLdsA) {
        const hipError_t e = launch_act_prep(ActPrepArgs{a.A, a.A16, a.ashift, a.M, a.K, a.splits, kWK}, stream);
        if (e != hipSuccess) return e;
    }
    if (plan.lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)((a.N + kOutTile - 1) / kOutTile), (unsigned)a.splits);
    hipLaunchKernelGGL(kern, grid, dim3(kWK * 64), plan.lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.amax_keys) return e;
    return launch_argmax_finish(a.amax_keys, (int)grid.x, a.amax_idx, a.M, stream);
}

template <bool kMfma, int kZM, bool kLdsA, int kC, bool kDual = false>
hipError_t launch_wk(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream)
{
    switch (plan.wk) {
    case 1: return launch_one<kMfma, kZM, kLdsA, 1, kC, kDual>(a, plan, stream);
    case 2: return launch_one<kMfma, kZM, kLdsA, 2, kC, kDual>(a, plan, stream);
    case 4: return launch_one<kMfma, kZM, kLdsA, 4, kC, kDual>(a, plan, stream);
    case 8: return launch_one<kMfma, kZM, kLdsA, 8, kC, kDual>(a, plan, stream);
    case 16: return launch_one<kMfma, kZM, kLdsA, 16, kC, kDual>(a, plan, stream);
    default: return hipErrorInvalidValue;
    }
}

// The GEMV runs on 64-column tiles only (128-column tiles go to the matrix cores).
template <bool kMfma, int kZM, bool kLdsA>
hipError_t launch_cols(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream)
{
    if constexpr (kMfma)
        return plan.cols == 8 ? launch_wk<kMfma, kZM, kLdsA, 8>(a, plan, stream)
                              : launch_wk<kMfma, kZM, kLdsA, 4>(a, plan, stream);
    else
        return plan.cols == 4 ? launch_wk<kMfma, kZM, kLdsA, 4>(a, plan, stream) : hipErrorInvalidValue;
}

template <bool kMfma, bool kLdsA>
hipError_t launch_sym(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream)
{
    if (a.biases) return launch_cols<kMfma, kAffine, kLdsA>(a, plan, stream);
    return a.qzeros == nullptr ? launch_cols<kMfma, kZeroSym, kLdsA>(a, plan, stream)
                               : launch_cols<kMfma, kZeroPacked, kLdsA>(a, plan, stream);
}

// A gated pair: matrix cores on 8 columns per lane (4 of each matrix).
template <bool kLdsA>
hipError_t launch_pair(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream)
{
    if (plan.cols != 8 || !plan.mfma) return hipErrorInvalidValue;
    if (a.biases) return launch_wk<true, kAffine, kLdsA, 8, true>(a, plan, stream);
    return a.qzeros == nullptr ? launch_wk<true, kZeroSym, kLdsA, 8, true>(a, plan, stream)
                               : launch_wk<true, kZeroPacked, kLdsA, 8, true>(a, plan, stream);
}

}  // namespace

hipError_t launch_act_prep(const ActPrepArgs &pa, hipStream_t stream)
{
    hipLaunchKernelGGL(act_prep_kernel, dim3((unsigned)(pa.splits * pa.wk), (unsigned)((pa.M + kPrepWaves - 1) / kPrepWaves)),
                       dim3(kPrepWaves * 64), 0, stream, pa);
    return hipGetLastError();
}

hipError_t launch_argmax_finish(unsigned long long *keys, int slots, int32_t *idx, int M, hipStream_t stream)
{
    hipLaunchKernelGGL(argmax_slots_finish_kernel, dim3((unsigned)M), dim3(kFinishThreads), 0, stream, keys, slots,
                       idx);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream)
{
    if (a.qweight2) return plan.lds_a ? launch_pair<true>(a, plan, stream) : launch_pair<false>(a, plan, stream);
    if (!plan.mfma) return launch_sym<false, true>(a, plan, stream);   // GEMV: always staged
    return plan.lds_a ? launch_sym<true, true>(a, plan, stream) : launch_sym<true, false>(a, plan, stream);
}

}  // namespace w4a16
