// W4A16 GEMM for many rows (prompt processing) on gfx950's matrix cores.
//
// The GRIMOIRE v1.8 release notes ('What changed', INT4 prompt processing) route GPTQ int4
// weights through a fast prompt path. With hundreds of rows every packed weight feeds hundreds
// of multiply-adds, so the bound is the matrix cores, not HBM, and the shape is a tiled GEMM:
//   * a workgroup owns a 64 x 256 output tile; each of its 4 waves owns 64 x 64 (4 x 4 blocks of
//     one v_mfma_f32_16x16x32_f16 each per 32-row K step). The tile is wide because a step moves
//     2 / width bytes of activations (re-read by every column tile) per multiply-add against
//     0.5 / height of packed weights, and the global->LDS traffic is what bounds the kernel
//     (64 x 256 measured 18% faster than 128 x 128 at 512 rows; 128 x 256 with 8 waves slower,
//     one such workgroup per CU leaving no second one to run while it waits);
//   * the activations come prepared once per call (act_prep_kernel with one piece per row):
//     fp16 in the packed-word slot order after an exact power-of-two rescale of each row, so a
//     16-byte read is an MFMA A fragment as is;
//   * every operand of a step -- the 128 x 32 activation tile, the 32 x 128 packed weights, and
//     the scales and zero words of the step's group -- is staged in LDS by direct global->LDS
//     loads, kStages steps ahead, so the loads cost no registers and each step waits for its
//     own stage only; one barrier per step both publishes a stage and frees the one before;
//   * each wave dequantises its columns' packed words exactly in registers (w4a16_device.h)
//     into the B fragments of its 4 column blocks;
//   * sums are kept per quantisation group and scaled once at the group's end in fp32, so the
//     exact (q - z) * scale product never rounds before accumulation.
#include <type_traits>

#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {
namespace {

constexpr int kStages = 4;   // LDS ring depth in steps
constexpr int kXcds = 8;     // gfx950 dies; workgroups are dispatched to them round-robin
constexpr int kRowGroup = 4; // row tiles that visit the column tiles together

// One stage of LDS: the activation tile [64 rows][4 chunks of 16 B] (a row's chunk c sits in
// slot c ^ ((row / 4) % 4): the 16 rows a wave reads at once then fall into 16 different bank
// groups), the codes [R word rows][256 columns], then for GPTQ codes 256 fp16 scales and 32 zero
// words, for affine codes per wave w the bf16 scales of columns [64 w, 64 w + 64) followed by
// their bf16 biases. R = 4 for GPTQ words; R = the code width for affine bit streams (a step's
// 32 rows of a column are that many words).
template <int kBits>
struct Stage {
    static constexpr int R = kBits ? kBits : 4;
    static constexpr int A = kPrefillTileM * 64;
    static constexpr int B = R * kPrefillTileN * 4;
    static constexpr int S = kPrefillTileN * 2;
    static constexpr int Z = kBits ? kPrefillTileN * 2 : kPrefillTileN / 8 * 4;
    static constexpr int bytes = A + B + S + Z;
};

// Waves per SIMD the register allocator must keep: 3 for symmetric zero points (the gated pair
// needs it: FFN 5120 x 17408 at M = 2048, 852 us against 985 with 2), 2 with stored zero
// points, whose extra registers would spill at 3 (FFN down 17408 x 5120 at M = 2048: 1158 us
// at 3 against 772 at 2), and 2 for affine codes (16 more accumulators: the bias sums).
template <bool kSym, int kBits>
constexpr int prefill_min_waves() { return kSym && !kBits ? 3 : 2; }

// kDual: a gated pair (gate in qweight, up in qweight2). The tile's 256 columns are then 128
// output columns of the gate followed by the same 128 of the up projection: waves 0 and 1
// compute the gate, waves 2 and 3 the up projection, and the up waves hand their sums to the
// gate waves through LDS, which write silu(gate) * up. Everything up to the epilogue is the
// single-matrix kernel over those 256 columns.
//
// kBits > 0: affine codes w = s * q + b (MLX affine checkpoints, TensorFold PR #859, commit
// messages and PR description: codes of their own width, and a prompt GEMM for them), stored as
// column bit streams [K * kBits / 32, N] with bf16 scales and biases [K / g, N]. A step stages
// its kBits word rows; each lane pulls its column's 8 codes out of one or two words as exact
// fp16 values (affine_codes), and one more matrix-core product per row block against ones gives
// the activations' own sums, so every group adds s * sum(a q) + b * sum(a) in fp32.
template <bool kSym, bool kDual, int kBits = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(prefill_min_waves<kSym, kBits>()))) void
w4a16_prefill_kernel(PrefillArgs p)
{
    constexpr bool kAff = kBits > 0;
    static_assert(!(kAff && kDual), "the affine prompt GEMM is a single matrix");
    using St = Stage<kBits>;
    constexpr int kStA = St::A;
    constexpr int kStB = St::B;
    constexpr int kStS = St::S;
    constexpr int kStBytes = St::bytes;
    constexpr int R = St::R;
    // codes staged with 16-byte loads (word rows w, w + 4 of the step by wave w: GPTQ words and
    // 4- and 8-bit streams) or 4-byte loads (column t of every word row by thread t: widths 1, 2,
    // 3, 5 and 6), so that every wave issues the same number of loads per stage
    constexpr bool kWide = !kAff || kBits % 4 == 0;
    constexpr int kWLoads = !kAff ? 1 : kWide ? kBits / 4 : kBits;
    constexpr int kOutCols = kDual ? kPrefillTileN / 2 : kPrefillTileN;   // output columns per tile
    __shared__ __align__(16) unsigned char lds[kStages * kStBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS and load bases stay scalar
    const int cl = lane & 15;   // A row / B column of the lane within a 16 x 16 block
    const int rl = lane >> 4;   // word row (8 K rows) of the lane within a 32-row step
    const int wn = wave;   // the wave's 64 columns of the tile
    const int M = p.M;
    const int N = p.N;
    const int K = p.K;
    // A contiguous range of tiles per die: workgroup w runs on die w % 8 (the dispatch order is a
    // matter of speed only; any mapping is correct).
    // Work units are (tile, K slice) pairs, the slices of a tile adjacent.
    const int row_tiles = (M + kPrefillTileM - 1) / kPrefillTileM;
    const int col_tiles = (N + kOutCols - 1) / kOutCols;
    const int units = row_tiles * col_tiles * p.splits;
    const int per_die = (units + kXcds - 1) / kXcds;
    const int unit = (int)(blockIdx.x % kXcds) * per_die + (int)(blockIdx.x / kXcds);
    if (unit >= units) return;   // padding of the grid to a multiple of 8
    const int tile = unit / p.splits;
    const int slice = unit - tile * p.splits;
    // Within that order, kRowGroup row tiles take each column tile in turn, so the row tiles of
    // a group share a weight tile in L2 while their activations stay there.
    const int grp = tile / (kRowGroup * col_tiles);
    const int g_rows = min(kRowGroup, row_tiles - grp * kRowGroup);
    const int idx = tile - grp * kRowGroup * col_tiles;
    const int tm = (grp * kRowGroup + idx % g_rows) * kPrefillTileM;   // the tile's first row
    const int tn = (idx / g_rows) * kOutCols;                          // the tile's first column
    const int spg = p.g / kStepK;
    // the slice's K range: whole quantisation groups [gb, ge), so every group is scaled once
    const int groups = K / p.g;
    const int gb = (int)((long long)slice * groups / p.splits);
    const int ge = (int)((long long)(slice + 1) * groups / p.splits);
    const int s0 = gb * spg;              // first step of the slice
    const int steps = (ge - gb) * spg;    // steps of the slice (>= 1: splits <= groups)

    // ---- loads of one stage: every wave issues the same kLoads direct loads -------------------
    constexpr int kLoads = 2 + kWLoads + (!kAff && !kSym ? 1 : 0);
    // activation tile: wave w fills slots [64 w, 64 w + 64), rows 16 w .. 16 w + 15
    // (all operands of a single GPTQ matrix, and the activations of every instance, load from a
    // wave-uniform base in scalar registers plus a byte offset per lane; the gated pair and affine
    // codes pick between two arrays per lane, and those loads keep a full address per lane)
    constexpr bool kSBase = !kDual && !kAff;
    const uint16_t *const a_base = p.A16 + (size_t)tm * K;   // the tile's first row
    uint32_t a_off_b;                                         // bytes (< 64 rows x K x 2)
    {
        const int slot = wave * 64 + lane;
        const int row = slot >> 2;
        const int chunk = (slot & 3) ^ ((row >> 2) & 3);
        a_off_b = (uint32_t)(((min(tm + row, M - 1) - tm) * K + chunk * 8) * 2);   // rows past M: the last row
    }
    auto col = [&](int c) { return c < N ? c : 0; };   // columns past N read column 0, never stored
    // Column c of the tile (0..255) is output column tn + c of the single matrix, or for a pair
    // output column tn + c % 128 of the gate (c < 128) or of the up projection.
    auto in_up = [&](int c) { return kDual && c >= kOutCols; };
    auto out_col = [&](int c) { return col(tn + (kDual ? c % kOutCols : c)); };
    // packed weights: wave w loads word row w of the step (and w + 4 of an 8-bit stream), four
    // columns per lane; or thread t loads column t of every word row of the step
    const uint32_t *w_src = kWide ? (in_up(lane * 4) ? p.qweight2 : p.qweight) + (size_t)wave * N + out_col(lane * 4)
                                  : p.qweight + out_col(tid);
    // scales: wave w loads columns [64 w, 64 w + 64) as 32 pairs; zero words: wave w loads 8;
    // affine biases: lanes 32..63 load the same columns' biases right after the scales
    const int sc_c = wave * 64 + (lane & 31) * 2;
    const uint16_t *s_src = kAff ? (lane < 32 ? p.scales : p.biases) + out_col(sc_c)
                                 : (in_up(sc_c) ? p.scales2 : p.scales) + out_col(sc_c);
    const int zc_c = (wave * 8 + (lane & 7)) * 8;
    const uint32_t *z_src = kSym ? nullptr : (in_up(zc_c) ? p.qzeros2 : p.qzeros) + out_col(zc_c) / 8;
    // their byte offsets from the matrices' starts, for the scalar-base loads
    const uint32_t w_off_b = (uint32_t)(((size_t)wave * N + out_col(lane * 4)) * 4);
    const uint32_t s_off_b = (uint32_t)out_col(sc_c) * 2;
    const uint32_t z_off_b = (uint32_t)(out_col(zc_c) / 8) * 4;
    int lt = s0, lg = gb, lpos = 0;   // next step to stage, its group and position in the group
    auto issue = [&](int buf) {
        unsigned char *st = lds + buf * kStBytes;
        load_to_lds16_s(a_base + (size_t)lt * kStepK, a_off_b, st + wave * 64 * 16);
        // word offsets < 2^32 (host)
#pragma unroll
        for (int j = 0; j < kWLoads; ++j) {
            if constexpr (kSBase)
                load_to_lds16_s(p.qweight + (size_t)((uint32_t)lt * (uint32_t)R + 4u * (uint32_t)j) * (uint32_t)N,
                                w_off_b, st + kStA + (wave + 4 * j) * 1024);
            else if constexpr (kWide)
                load_to_lds16(w_src + ((uint32_t)lt * (uint32_t)R + 4u * (uint32_t)j) * (uint32_t)N,
                              st + kStA + (wave + 4 * j) * 1024);
            else
                load_to_lds4(w_src + ((uint32_t)lt * (uint32_t)R + (uint32_t)j) * (uint32_t)N,
                             st + kStA + j * 1024 + wave * 256);
        }
        if constexpr (kAff)
            load_to_lds4(s_src + (size_t)lg * N, st + kStA + kStB + wave * 256);
        else if (lane < 32) {
            if constexpr (kSBase)
                load_to_lds4_s(p.scales + (size_t)lg * N, s_off_b, st + kStA + kStB + wave * 128);
            else
                load_to_lds4(s_src + (size_t)lg * N, st + kStA + kStB + wave * 128);
        }
        if (!kSym && lane < 8) {
            if constexpr (kSBase)
                load_to_lds4_s(p.qzeros + (size_t)lg * (N / 8), z_off_b, st + kStA + kStB + kStS + wave * 32);
            else
                load_to_lds4(z_src + (size_t)lg * (N / 8), st + kStA + kStB + kStS + wave * 32);
        }
        if (lt + 1 < s0 + steps) {   // past the slice's last step the stage reloads it (uniform)
            ++lt;
            if (++lpos == spg) {
                lpos = 0;
                ++lg;
            }
        }
    };

    // ---- compute ------------------------------------------------------------------------------
    const int n0 = tn + (kDual ? wn & 1 : wn) * 64 + cl * 4;   // the lane's 4 output columns
    const Masks mk = make_masks();
    float4_t acc[4][4];
    float4_t tot[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
            tot[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
    ZeroSub zs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) zs[j] = zero_sub_sym();
    // affine codes: the activations' own sums per row block (times the group's bias), and the
    // words holding the lane's 8 codes: bit a_bit = 8 * kBits * rl of the step's column stream
    // onwards, in word row w_row0 and, for widths that cross a word, w_row1 (a row of the step
    // whose bits are not used when the codes end in w_row0)
    float4_t acc_one[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_one[i] = float4_t{0.f, 0.f, 0.f, 0.f};
    const half8_t ones = half8_t{1, 1, 1, 1, 1, 1, 1, 1};
    constexpr bool kTwoWords = kAff && !(kBits == 1 || kBits == 2 || kBits == 4);
    const int a_bit = kAff ? 8 * kBits * rl : 0;
    const int c_off = a_bit & 31, c_off4 = c_off + 4 * kBits;   // bit positions of rows k0 and k4
    const int w_row0 = kAff ? a_bit >> 5 : rl;
    const int w_row1 = min(w_row0 + 1, R - 1);
    int cpos = 0;   // position of the computed step in its group
    int a_off[4];   // the lane's A fragment of each row block within a stage
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + cl;
        a_off[i] = row * 64 + ((rl ^ ((row >> 2) & 3)) * 16);
    }
    const int b_off = kStA + w_row0 * 1024 + (wn * 64 + cl * 4) * 4;
    const int b_off1 = kStA + w_row1 * 1024 + (wn * 64 + cl * 4) * 4;
    const int s_off = kAff ? kStA + kStB + wn * 256 + cl * 8 : kStA + kStB + (wn * 64 + cl * 4) * 2;
    const int z_off = kStA + kStB + kStS + (wn * 8 + (cl >> 1)) * 4;

    constexpr bool kZeroStart = prefill_min_waves<kSym, kBits>() == 2;
    auto step = [&](int buf, auto first_tag) {
        constexpr bool kFirst = decltype(first_tag)::value;   // the group's first step
        const unsigned char *st = lds + buf * kStBytes;
        if (!kSym && cpos == 0) {   // a new group's zero points (uniform)
            const uint32_t zw = *reinterpret_cast<const uint32_t *>(st + z_off);
#pragma unroll
            for (int j = 0; j < 4; ++j) zs[j] = zero_sub(zero_of(zw, (uint32_t)(n0 + j)));
        }
        const uint4 w = *reinterpret_cast<const uint4 *>(st + b_off);
        const uint32_t words[4] = {w.x, w.y, w.z, w.w};
        uint32_t words1[4] = {0u, 0u, 0u, 0u};
        if constexpr (kTwoWords) {
            const uint4 w1 = *reinterpret_cast<const uint4 *>(st + b_off1);
            words1[0] = w1.x;
            words1[1] = w1.y;
            words1[2] = w1.z;
            words1[3] = w1.w;
        }
        half8_t b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (kAff)
                b[j] = affine_codes<kBits>(words[j], words1[j], c_off, c_off4, mk);
            else
                b[j] = dequant_word(words[j], kSym ? zero_sub_sym() : zs[j], mk);
        }
        // With registers to spare (the 2-wave instances), a group's first step starts its sums
        // from zero in the products themselves (a zero C operand), so the group's end needs no
        // clearing moves; the 3-wave instances would spill for it and clear at the group's end.
        const float4_t zero4 = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half8_t a = *reinterpret_cast<const half8_t *>(st + a_off[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], kFirst ? zero4 : acc[i][j], 0, 0, 0);
            if constexpr (kAff)
                acc_one[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, kFirst ? zero4 : acc_one[i], 0, 0, 0);
        }
        if (++cpos == spg) {   // the group's end: scale its sums once (uniform)
            cpos = 0;
            const uint2 sv = *reinterpret_cast<const uint2 *>(st + s_off);
            float sc[4], bi[4];
            if constexpr (kAff) {
                const uint2 bv = *reinterpret_cast<const uint2 *>(st + s_off + 128);
                sc[0] = bf16_bits_to_float(sv.x & 0xFFFFu);
                sc[1] = bf16_bits_to_float(sv.x >> 16);
                sc[2] = bf16_bits_to_float(sv.y & 0xFFFFu);
                sc[3] = bf16_bits_to_float(sv.y >> 16);
                bi[0] = bf16_bits_to_float(bv.x & 0xFFFFu);
                bi[1] = bf16_bits_to_float(bv.x >> 16);
                bi[2] = bf16_bits_to_float(bv.y & 0xFFFFu);
                bi[3] = bf16_bits_to_float(bv.y >> 16);
            } else {
                sc[0] = half_bits_to_float(sv.x & 0xFFFFu);
                sc[1] = half_bits_to_float(sv.x >> 16);
                sc[2] = half_bits_to_float(sv.y & 0xFFFFu);
                sc[3] = half_bits_to_float(sv.y >> 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        tot[i][j][r] = __builtin_fmaf(acc[i][j][r], sc[j], tot[i][j][r]);
                        if constexpr (kAff) tot[i][j][r] = __builtin_fmaf(acc_one[i][r], bi[j], tot[i][j][r]);
                    }
                    if constexpr (!kZeroStart) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
                }
                if constexpr (kAff && !kZeroStart) acc_one[i] = float4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    };

    // Stages 0 .. kStages-2 first; at step t, after the wait for stage t and the barrier (every
    // wave is past step t-1), stage t + kStages - 1 refills the buffer step t-1 used.
#pragma unroll
    for (int u = 0; u + 1 < kStages; ++u) issue(u);
    for (int t = 0; t < steps; ++t) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * kLoads));
        __syncthreads();
        issue((t + kStages - 1) % kStages);
        if (kZeroStart && cpos == 0)   // uniform
            step(t % kStages, std::true_type{});
        else
            step(t % kStages, std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the last stages' reloads land before the wave ends

    // Lane holds rows 4 rl + r of each row block, its 4 columns: undo the row's rescale, store
    // (or store the slice's fp32 sums for the slice reduction, 2N wide for a pair).
    if (kDual && p.splits == 1) {   // up sums to LDS (over the dead ring), then silu(gate) * up
        __syncthreads();
        float *upl = reinterpret_cast<float *>(lds);   // [64 rows][128 columns]
        if (wave >= 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = tm + 16 * i + 4 * rl + r;
                    const int sh = p.shifts[min(m, M - 1)];
                    *reinterpret_cast<float4 *>(upl + (16 * i + 4 * rl + r) * kOutCols + (wn & 1) * 64 + cl * 4) =
                        make_float4(__builtin_amdgcn_ldexpf(tot[i][0][r], sh), __builtin_amdgcn_ldexpf(tot[i][1][r], sh),
                                    __builtin_amdgcn_ldexpf(tot[i][2][r], sh), __builtin_amdgcn_ldexpf(tot[i][3][r], sh));
                }
        }
        __syncthreads();
        if (wave >= 2 || n0 >= N) return;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = tm + 16 * i + 4 * rl + r;
                if (m >= M) continue;
                const int sh = p.shifts[m];
                const float4 u = *reinterpret_cast<const float4 *>(upl + (16 * i + 4 * rl + r) * kOutCols + wn * 64 + cl * 4);
                const float x0 = silu_f32(__builtin_amdgcn_ldexpf(tot[i][0][r], sh)) * u.x;
                const float x1 = silu_f32(__builtin_amdgcn_ldexpf(tot[i][1][r], sh)) * u.y;
                const float x2 = silu_f32(__builtin_amdgcn_ldexpf(tot[i][2][r], sh)) * u.z;
                const float x3 = silu_f32(__builtin_amdgcn_ldexpf(tot[i][3][r], sh)) * u.w;
                const size_t o = (size_t)m * N + n0;
                if (p.out_bf16) {
                    uint2 q;
                    q.x = float_to_bf16_bits(x0) | (float_to_bf16_bits(x1) << 16);
                    q.y = float_to_bf16_bits(x2) | (float_to_bf16_bits(x3) << 16);
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + o) = q;
                } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o) = make_float4(x0, x1, x2, x3);
                }
            }
        return;
    }
    if (n0 >= N) return;
    if (p.splits > 1) {
        const size_t NV = kDual ? 2 * (size_t)N : (size_t)N;   // partial row: [gate | up] for a pair
        float *part = p.partials + (size_t)slice * M * NV + (kDual && wave >= 2 ? N : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = tm + 16 * i + 4 * rl + r;
                if (m >= M) continue;
                const int sh = p.shifts[m];
                *reinterpret_cast<float4 *>(part + (size_t)m * NV + n0) =
                    make_float4(__builtin_amdgcn_ldexpf(tot[i][0][r], sh), __builtin_amdgcn_ldexpf(tot[i][1][r], sh),
                                __builtin_amdgcn_ldexpf(tot[i][2][r], sh), __builtin_amdgcn_ldexpf(tot[i][3][r], sh));
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = tm + 16 * i + 4 * rl + r;
            if (m >= M) continue;
            const int sh = p.shifts[m];
            const float x0 = __builtin_amdgcn_ldexpf(tot[i][0][r], sh), x1 = __builtin_amdgcn_ldexpf(tot[i][1][r], sh);
            const float x2 = __builtin_amdgcn_ldexpf(tot[i][2][r], sh), x3 = __builtin_amdgcn_ldexpf(tot[i][3][r], sh);
            const size_t o = (size_t)m * N + n0;
            if (p.out_bf16) {
                uint2 q;
                q.x = float_to_bf16_bits(x0) | (float_to_bf16_bits(x1) << 16);
                q.y = float_to_bf16_bits(x2) | (float_to_bf16_bits(x3) << 16);
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + o) = q;
            } else {
                *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o) = make_float4(x0, x1, x2, x3);
            }
        }
}

// out = the sum of the K slices in slice order (deterministic), 4 outputs per thread; for a
// gated pair silu(gate sum) * up sum, the slices' rows being [gate | up].
template <bool kDual>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillArgs p)
{
    const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;   // float4 index of the output
    const size_t mn = (size_t)p.M * p.N;
    if (q * 4 >= mn) return;
    auto slice_sum = [&](size_t at) {   // float index at of a slice, summed over the slices
        const size_t stride = kDual ? 2 * mn : mn;
        float4 v = *reinterpret_cast<const float4 *>(p.partials + at);
        for (int s = 1; s < p.splits; ++s) {
            const float4 w = *reinterpret_cast<const float4 *>(p.partials + (size_t)s * stride + at);
            v.x += w.x;
            v.y += w.y;
            v.z += w.z;
            v.w += w.w;
        }
        return v;
    };
    float4 v;
    if constexpr (kDual) {
        const size_t m = q * 4 / p.N, n = q * 4 - m * p.N;
        const float4 gs = slice_sum(m * 2 * p.N + n), us = slice_sum(m * 2 * p.N + p.N + n);
        v = make_float4(silu_f32(gs.x) * us.x, silu_f32(gs.y) * us.y, silu_f32(gs.z) * us.z, silu_f32(gs.w) * us.w);
    } else {
        v = slice_sum(q * 4);
    }
    if (p.out_bf16) {
        uint2 o;
        o.x = float_to_bf16_bits(v.x) | (float_to_bf16_bits(v.y) << 16);
        o.y = float_to_bf16_bits(v.z) | (float_to_bf16_bits(v.w) << 16);
        reinterpret_cast<uint2 *>(p.out)[q] = o;
    } else {
        reinterpret_cast<float4 *>(p.out)[q] = v;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    const bool dual = a.qweight2 != nullptr;
    const int out_cols = dual ? kPrefillTileN / 2 : kPrefillTileN;
    const int units = ((a.M + kPrefillTileM - 1) / kPrefillTileM) * ((a.N + out_cols - 1) / out_cols) * a.splits;
    const dim3 grid((unsigned)((units + kXcds - 1) / kXcds * kXcds));   // whole rounds of the 8 dies
    const bool sym = a.qzeros == nullptr;
    void (*kern)(PrefillArgs) = dual ? (sym ? w4a16_prefill_kernel<true, true> : w4a16_prefill_kernel<false, true>)
                                     : (sym ? w4a16_prefill_kernel<true, false> : w4a16_prefill_kernel<false, false>);
    switch (a.bits) {   // affine codes (the host admits these widths only)
    case 0: break;
    case 1: kern = w4a16_prefill_kernel<true, false, 1>; break;
    case 2: kern = w4a16_prefill_kernel<true, false, 2>; break;
    case 3: kern = w4a16_prefill_kernel<true, false, 3>; break;
    case 4: kern = w4a16_prefill_kernel<true, false, 4>; break;
    case 5: kern = w4a16_prefill_kernel<true, false, 5>; break;
    case 6: kern = w4a16_prefill_kernel<true, false, 6>; break;
    case 8: kern = w4a16_prefill_kernel<true, false, 8>; break;
    default: return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    const size_t quads = (size_t)a.M * a.N / 4;   // N % 8 == 0
    void (*reduce)(PrefillArgs) = dual ? prefill_reduce_kernel<true> : prefill_reduce_kernel<false>;
    hipLaunchKernelGGL(reduce, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a16
