// Host-side interface between the C ABI (w4a16_api.hip) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// Columns of a column tile: one wave wide, 16 lanes x `cols` adjacent columns each (4 or 8). The
// waves of a workgroup share the tile and split its K range.
inline int tile_columns(int cols) { return 16 * cols; }
// Matrices at least this wide get 128-column tiles by default (64 otherwise).
constexpr int kWideTileMinN = 32768;
// K rows consumed per step (4 packed word rows = one 16x16x32 MFMA K step).
constexpr int kStepK = 32;
// Largest dynamic LDS a GEMM workgroup may ask for (gfx950: 160 KiB per workgroup).
constexpr int kMaxLds = 160 * 1024 - 256;
// Staged activations (plus scales and zero words) per wave beyond which a 64-column plan takes
// prepared activations instead: larger staging areas cost more waves per CU than they save.
constexpr int kLdsStageBudget = 8 * 1024;
// LDS of one compute unit, and the waves per CU the 128-column matrix-core kernels reach (their
// registers cap them at 4 waves per SIMD): staging that still leaves room for that many waves
// costs them nothing.
constexpr int kLdsPerCu = 160 * 1024;
constexpr int kWideTileWavesPerCu = 16;

// Bound on the split-K reducer's wait for another slice's sums (each try sleeps about 128
// cycles). Only reached if a workgroup never finished, which a correct launch rules out; those
// outputs are then NaN instead of a hang.
constexpr uint32_t kSpinLimit = 1u << 24;

// The split-K exchange: fp32 slots [slices, M, N] that hold this bit pattern (a signalling NaN)
// between calls. A workgroup publishes its slice by storing it; the reducer takes each slot
// once it no longer holds the pattern and writes the pattern back. The kernels publish only
// results of floating-point arithmetic, which never produce a signalling NaN, so a slot changes
// exactly when its slice arrives. (Were a published value a NaN of this very payload, the
// reducer would wait out kSpinLimit and output NaN: the sum it stands for is NaN anyway.)
constexpr uint32_t kSliceEmpty = 0x7FBADBADu;

// Ints of per-row data at the start of a GEMM workgroup's LDS, per wave: 16 rescale exponents
// and 16 rescale multipliers.
constexpr int kRowHeader = 32;
// Ring depth (steps of packed weights in flight per wave). Shallow rings measure best: with
// thousands of short waves in flight, HBM is kept busy by the number of waves, and a deep ring
// only lengthens each wave's start. One step deeper when activations are staged in LDS (a slot
// is one 16-byte load) than when each slot also carries an activation fragment, except for
// packed zero points on 64-column tiles: their register floor (5 waves per SIMD) leaves room for a
// third slot (89 VGPRs), which measured 0.3-0.6 us faster at 11-16 rows on the 17408 x 5120
// projection; the other unstaged instances would spill or lose a wave per SIMD with it.
constexpr int kRingStaged = 3;
constexpr int kRingConvert = 2;

// How a column's weights are formed from its codes q:
//   kZeroPacked  w = (q - z) * s, zero points z in packed words (GPTQ)
//   kZeroSym     w = (q - 8) * s (GPTQ symmetric)
//   kAffine      w = s * q + b, bf16 scales and biases (MLX affine)
enum ZeroMode : int { kZeroPacked = 0, kZeroSym = 1, kAffine = 2 };

// Ring depth of a matrix-core instance whose activations come prepared (see kRingConvert).
template <int kZM, int kC>
constexpr int ring_unstaged()
{
    return kZM == kZeroPacked && kC == 4 ? 3 : kRingConvert;
}

struct GemmArgs {
    const uint16_t *A;
    const uint32_t *qweight;
    const uint16_t *scales;
    const uint32_t *qzeros;   // nullptr: symmetric zero point 8
    const uint16_t *biases;   // affine codes: bf16 biases [K/g, N] (scales are then bf16 too)
    // gated pair: the up projection (same shape as qweight, the gate); out = silu(gate) * up.
    // qweight2 == nullptr: a single matrix.
    const uint32_t *qweight2;
    const uint16_t *scales2;
    const uint32_t *qzeros2;
    const uint16_t *biases2;  // affine pair: the second matrix's biases
    int pair_sum;             // pair: 1 -> out = (A x W) + (A x W2) (split planes); 0 -> silu(gate) * up
    void *out;
    uint16_t *A16;            // [M, K] prepared activations (matrix-core path)
    int *ashift;              // [splits * waves_k, M] their rescale per K piece and row
    float *partials;          // split-K exchange [splits, M, N] (gated pair: [splits, M, 2N]), kSliceEmpty between calls
    uint32_t *counters;       // one per column tile, zero between calls
    unsigned long long *amax_keys;   // fused pick: [tiles, 16] row keys, one slot per column tile, zero between
                                     // calls (nullptr: off)
    int32_t *amax_idx;               // fused pick: [M] output indices
    int M, N, K, g;
    int splits;               // workgroups along K per column tile
    int out_bf16;
    int wave_lds;             // LDS bytes of one wave's staging area
    int scale_off;            // offset of the scales within a wave's area
    int zero_off;             // offset of the zero words (affine: the biases) within a wave's area
};

// How one call is launched.
struct GemmPlan {
    bool mfma;     // false: the M = 1 dot-product GEMV
    bool lds_a;    // activations staged once per wave in LDS (else converted per step)
    bool prep_a;   // activations prepared once per call by act_prep_kernel (matrix-core path)
    int cols;      // adjacent columns per lane (4 or 8): tiles of 64 or 128 columns
    int wk;        // waves per workgroup, each a contiguous K range (1, 2, 4, 8 or 16)
    int splits;    // workgroups per column tile, reduced through the scratch buffer
    size_t lds;    // dynamic LDS bytes per workgroup
    int wave_lds, scale_off, zero_off;
};

// Steps (of kStepK rows) of the largest K range a single wave gets under a plan.
inline int max_wave_steps(int K, int splits, int wk)
{
    const int steps = K / kStepK;
    const int per_split = (steps + splits - 1) / splits;
    return (per_split + wk - 1) / wk;
}

inline size_t round_up_sz(size_t x, size_t a) { return (x + a - 1) / a * a; }

// LDS layout of a plan: per-wave row shifts, then one staging area per wave (activations if
// staged, the scales and the zero words -- or for affine codes the biases -- of the wave's
// groups, filled by direct loads), and, after the main loop, the cross-wave reduction buffer
// over the same bytes.
inline size_t gemm_lds_layout(int M, int K, int g, int splits, int wk, int cols, bool lds_a, ZeroMode zm,
                              bool argmax, GemmPlan *pl)
{
    const size_t tile = (size_t)tile_columns(cols);
    const int ws = max_wave_steps(K, splits, wk);
    const int spg = g / kStepK;
    const size_t groups = (size_t)(ws + spg - 1) / spg + 1;
    const size_t a_bytes = lds_a ? round_up_sz((size_t)M * ws * 4, 64) * 16 : 0;
    const size_t s_bytes = groups * (tile / 8) * 16;                         // 8 scales per item
    const size_t z_bytes = zm == kZeroSym ? 0
                           : zm == kAffine ? s_bytes                                   // one bias per scale
                                           : round_up_sz(groups * (tile / 8) * 4, 16);   // 8 zeros per word
    const size_t wave = a_bytes + s_bytes + z_bytes;
    const size_t header = (size_t)wk * kRowHeader * sizeof(int);
    const size_t red = (wk > 1 || splits > 1 || argmax) ? (size_t)wk * M * tile * sizeof(float) : 0;
    const size_t body = (size_t)wk * wave > red ? (size_t)wk * wave : red;
    if (pl) {
        pl->wave_lds = (int)wave;
        pl->scale_off = (int)a_bytes;
        pl->zero_off = (int)(a_bytes + s_bytes);
    }
    return header + body;
}

// Activation preparation (matrix-core path): one workgroup per K piece of the launch.
struct ActPrepArgs {
    const uint16_t *A;
    uint16_t *A16;
    int *shifts;
    int M, K, splits, wk;
};

hipError_t launch_gemm(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream);
// Activations to fp16 in slot order with one power-of-two rescale per (K piece, row); with
// splits = wk = 1 a single piece covers the whole K of each row.
hipError_t launch_act_prep(const ActPrepArgs &pa, hipStream_t stream);

// Many-row GEMM (prompt processing): out[M, N] = A x W for any M, on the matrix cores, from
// activations prepared by launch_act_prep with one piece per row (A16, shifts).
struct PrefillArgs {
    const uint16_t *A16;      // [M, K] fp16, slot order, rescaled per row
    const int *shifts;        // [M] the rescale of each row (out = sum * 2^shift)
    const uint32_t *qweight;
    const uint16_t *scales;
    const uint32_t *qzeros;   // nullptr: symmetric zero point 8
    // gated pair: the up projection (same shape as qweight, the gate); out = silu(gate) * up.
    // qweight2 == nullptr: a single matrix.
    const uint32_t *qweight2;
    const uint16_t *scales2;
    const uint32_t *qzeros2;
    // affine codes (bits > 0): qweight is the column bit stream [K * bits / 32, N], scales and
    // biases bf16 [K / g, N], no zero points, a single matrix
    const uint16_t *biases;
    int bits;
    void *out;
    float *partials;          // [splits, M, N] fp32 slices when splits > 1 ([splits, M, 2N] for a pair)
    int M, N, K, g;
    int out_bf16;
    int splits;               // workgroups per tile along K, each a contiguous range of groups
};
// Output tile of one prefill workgroup (4 waves of 64 x 64 side by side).
constexpr int kPrefillTileM = 64;
constexpr int kPrefillTileN = 256;
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

// Decode GEMM (w4a16_decode.hip): a workgroup is `tiles` x `kw` waves over one K slice, wave
// (w, k) on column tile w (tiles adjacent, 64 or 128 columns each) and K piece k of the slice;
// the workgroup's activation slice is converted once into LDS for all of them and the pieces
// are added in LDS. `slices` workgroups share each group of columns along K; their fp32 sums
// meet through scratch: a counter per group of columns and a flag per slice (the writers wait for
// their stores to complete and raise the slice's flag; the reducer waits for the flags).
constexpr int kDecMaxWaves = 8;
constexpr int kDecodeMinN = 65536;   // plain calls this wide take the decode kernel by default
constexpr int kDecodeMidN = 16384;   // and from this width, plain calls of more than 8 rows
constexpr int kDecodeMidWgs = 192;   // their workgroups: at least this many, in one round
constexpr int kCus = 256;            // compute units of an MI355X (the planner is host-only)
constexpr int kDecMaxSlices = 16;
constexpr int kDecMaxTopK = 8;       // largest k of the fused pick
// Activation items (8 bf16 values) each thread of a decode workgroup keeps in registers between
// the row maximum and the conversion; a longer slice reads the rest twice.
constexpr int kDecHeld = 8;
struct DecodeArgs {
    const uint16_t *A;
    const uint32_t *qweight;  // GPTQ [K/8, N]; affine codes: column bit streams [K * bits / 32, N]
    const uint16_t *scales;   // fp16 (GPTQ) or bf16 (affine) [K/g, N]
    const uint32_t *qzeros;   // nullptr: symmetric zero point 8
    const uint16_t *biases;   // affine codes: bf16 [K/g, N] (nullptr: GPTQ)
    int bits;                 // affine codes: bits per code (1, 2, 3, 4, 5, 6 or 8)
    void *out;
    float *partials;          // [slices, M, N] fp32 (slices > 1), written before they are read
    uint32_t *counters;       // [groups] zero between calls
    uint32_t *flags;          // [groups, slices] zero between calls
    int M, N, K, g;
    int tiles;                // adjacent column tiles per workgroup
    int kw;                   // K pieces per tile (waves per tile) in a workgroup
    int slices;               // workgroups along K per group of columns
    int groups;               // groups of columns (tiles adjacent tiles each)
    int out_bf16;
    int a_off, s_off, z_off, r_off;   // LDS offsets: fragments, scales, zero words, piece sums
    int mp_log2;              // matrix-core fragments hold rows padded to 2^mp_log2 (4, 8 or 16)
    uint32_t part_bytes;      // bytes of the partials region (bounds the buffer accesses)
    // fused pick of the k best columns per row (topk = 0: off)
    int topk;                       // k, 1..kDecMaxTopK
    int pick_none;                  // index written where a row has no candidate left
    unsigned long long *pick_slots; // [M, groups, topk] each column group's best keys (written before read)
    uint32_t *pick_counter;         // column groups done, zero between calls
    int32_t *pick_idx;              // [M, topk] the call's picks
};
struct DecodePlan {
    bool mfma;                // false: the one-row dot-product GEMV
    int cols;                 // adjacent columns per lane: 4 or 8 (tiles of 64 or 128 columns)
    int tiles;
    int kw;
    int slices;
    int ring;                 // ring slots of packed weights in flight per wave (template instance)
    int sub;                  // 32-row steps per ring slot: 1, or 4 / bits for 1- and 2-bit affine codes
    bool one_round;           // the default launch of 9-16 rows below kDecodeMinN columns found its slices
    size_t lds;
    int a_off, s_off, z_off, r_off;
};
// Rows (4, 8 or 16, as log2) the matrix-core fragments of M rows are padded to.
inline int decode_mp_log2(int M) { return M <= 4 ? 2 : M <= 8 ? 3 : 4; }
// LDS of a decode plan: 16 row maxima, the activation slice as fp16 fragments (MFMA: 4 x 16 bytes
// per row of the padded rows per step; GEMV: 64 bytes per step), the workgroup's scales and zero
// words of its groups, and the K pieces' sums (kw - 1 pieces of every tile).
inline size_t decode_lds_layout(int M, int K, int g, bool mfma, int cols, int tiles, int kw, int slices, bool packed,
                                bool pick, DecodePlan *pl, bool affine = false, int sub = 1)
{
    const int units = K / kStepK / sub;   // slices are whole blocks of `sub` steps
    const int smax = (units + slices - 1) / slices * sub;
    const int spg = g / kStepK;
    const size_t groups = (size_t)(smax + spg - 1) / spg + 1;
    const size_t wc = (size_t)tiles * 16 * cols;
    const size_t a_off = 128;
    // the fragments; after the main loop the fused pick reuses the region for the finished
    // outputs, [M][wc] fp32, and then for each wave's best keys, [waves][kDecMaxTopK] 64-bit
    const size_t a_frag = (size_t)smax * (mfma ? (size_t)64 << decode_mp_log2(M) : 64);
    const size_t a_out = (size_t)M * wc * sizeof(float), a_keys = (size_t)tiles * kw * kDecMaxTopK * 8;
    const size_t a_pick = pick ? (a_out > a_keys ? a_out : a_keys) : 0;
    const size_t a_bytes = a_frag > a_pick ? a_frag : a_pick;
    const size_t s_off = a_off + a_bytes;
    const size_t s_bytes = groups * wc * 2;
    const size_t z_off = s_off + round_up_sz(s_bytes, 16);
    // the zero words, or for affine codes the biases (laid out as the scales)
    const size_t z_bytes = affine ? s_bytes : packed ? groups * (wc / 8) * 4 : 0;
    const size_t r_off = round_up_sz(z_off + z_bytes, 16);
    const size_t r_bytes = (size_t)(kw - 1) * tiles * 64 * cols * (mfma ? 4 : 1) * sizeof(float);
    if (pl) {
        pl->a_off = (int)a_off;
        pl->s_off = (int)s_off;
        pl->z_off = (int)z_off;
        pl->r_off = (int)r_off;
    }
    return r_off + r_bytes;
}
hipError_t launch_decode(const DecodeArgs &a, const DecodePlan &plan, hipStream_t stream);
// Ends the small-row kernel's fused greedy pick: idx[m] from the largest of keys[s * 16 + m] over
// the slots s < slots, and those keys cleared.
hipError_t launch_argmax_finish(unsigned long long *keys, int slots, int32_t *idx, int M, hipStream_t stream);

struct ArgmaxArgs {
    const float *logits;
    int32_t *idx;
    unsigned long long *keys;   // [M], zero between calls
    uint32_t *counters;         // [M], zero between calls
    int M, N;
    int chunks;                 // workgroups per row
};

constexpr int kArgmaxChunk = 4096;   // logits per argmax workgroup

hipError_t launch_argmax(const ArgmaxArgs &a, hipStream_t stream);
// Codes of 1..4 bits in column bit streams [K*bits/32, N] rewritten as 4-bit codes [K/8, N]
// (each code keeps its value).
hipError_t launch_affine_widen(const uint32_t *packed, int bits, int K, int N, uint32_t *qweight, hipStream_t s);
// Codes of 5..8 bits split into a low and a high 4-bit plane ([2K/8, N]: low rows, then high rows),
// with the planes' scales [2K/g, N] (s, then 16 s) and biases (b, then 0).
hipError_t launch_affine_split(const uint32_t *packed, int bits, const uint16_t *scales, const uint16_t *biases,
                               int g, int K, int N, uint32_t *qweight, uint16_t *scales_out, uint16_t *biases_out,
                               hipStream_t s);
hipError_t launch_stream_read(const void *buf, long long bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_unpack_u8(const uint32_t *qweight, int K, int N, uint8_t *q, hipStream_t s);
hipError_t launch_dequant_f32(const uint32_t *qweight, const uint16_t *scales,
                              const uint32_t *qzeros, int g, int K, int N, float *w,
                              hipStream_t s);

}  // namespace w4a16
