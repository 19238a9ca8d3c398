// W4A16 GEMM for many rows (prompt processing) on gfx950's matrix cores.
//
// The GRIMOIRE v1.8 release notes ('What changed', INT4 prompt processing) route GPTQ int4
// weights through a fast prompt path. With hundreds of rows every packed weight feeds hundreds
// of multiply-adds, so the bound is the matrix cores, not HBM, and the shape is a plain tiled
// GEMM:
//   * a workgroup owns a 128 x 128 output tile; its 4 waves own 64 x 64 quarters (4 x 4 blocks of
//     one v_mfma_f32_16x16x32_f16 each per 32-row K step);
//   * the activations come prepared once per call (act_prep_kernel with one piece per row):
//     fp16 in the packed-word slot order after an exact power-of-two rescale of each row, so a
//     lane's 16-byte load is an MFMA A fragment as is;
//   * the packed weights are loaded as in the small-row kernel (lane: 4 adjacent columns of one
//     word row, 256 contiguous bytes per 16 lanes) and dequantised exactly in registers into the
//     B fragments of the wave's 4 column blocks (w4a16_device.h);
//   * sums are kept per quantisation group and scaled once at the group's end in fp32, so the
//     exact (q - z) * scale product never rounds before accumulation;
//   * each step's activation fragments, weight words, and the scales and zero word of its group
//     travel in one ring slot: every load of the loop is unconditional, one step ahead per slot.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {
namespace {

constexpr int kPrefillPf = 2;   // ring depth in steps

// One step's operands: the A fragments of the wave's 4 row blocks, 4 packed words (the lane's
// 4 columns), and the fp16 scales and zero word of the step's group for those columns.
struct PrefillSlot {
    uint4 a[4];
    uint4 w;
    uint2 s;
    uint32_t z;
};

template <bool kSym>
__global__ __launch_bounds__(256) void w4a16_prefill_kernel(PrefillArgs p)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cl = lane & 15;   // A row / B column of the lane within a 16 x 16 block
    const int rl = lane >> 4;   // word row (8 K rows) of the lane within a 32-row step
    const int M = p.M;
    const int N = p.N;
    const int K = p.K;
    const int n0 = blockIdx.x * kPrefillTileN + (wave & 1) * 64 + cl * 4;   // the lane's 4 columns
    const bool col_ok = n0 < N;
    const int nc = col_ok ? n0 : 0;
    const int mb = blockIdx.y * kPrefillTileM + (wave >> 1) * 64;   // the wave's first row
    const int steps = K / kStepK;
    const int spg = p.g / kStepK;
    const int groups = K / p.g;

    const uint32_t *wl = p.qweight + (size_t)rl * N + nc;
    const uint16_t *al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = min(mb + 16 * i + cl, M - 1);   // rows past M read the last row, never stored
        al[i] = p.A16 + (size_t)m * K + rl * 8;
    }
    const uint16_t *sl = p.scales + nc;
    const uint32_t *zl = kSym ? nullptr : p.qzeros + nc / 8;

    // Loads run one slot ahead of use, in step order; their group is tracked by counting.
    int lt = 0, lg = 0, lpos = 0;   // next step to load, its group and position in the group
    auto load = [&](PrefillSlot &s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s.a[i] = *reinterpret_cast<const uint4 *>(al[i] + (size_t)lt * kStepK);
        s.w = *reinterpret_cast<const uint4 *>(wl + (uint32_t)(lt * 4 * N));   // < 2^32 words (host)
        s.s = *reinterpret_cast<const uint2 *>(sl + (size_t)lg * N);
        if (!kSym) s.z = zl[(size_t)lg * (N / 8)];
        if (lt + 1 < steps) {   // past the last step the slot reloads it (uniform)
            ++lt;
            if (++lpos == spg) {
                lpos = 0;
                lg = min(lg + 1, groups - 1);
            }
        }
    };

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
    int cpos = 0;   // position of the computed step in its group

    auto step = [&](const PrefillSlot &s) {
        if (!kSym && cpos == 0) {   // a new group's zero points (uniform)
#pragma unroll
            for (int j = 0; j < 4; ++j) zs[j] = zero_sub(zero_of(s.z, (uint32_t)(nc + j)));
        }
        const uint32_t words[4] = {s.w.x, s.w.y, s.w.z, s.w.w};
        half8_t b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = dequant_word(words[j], kSym ? zero_sub_sym() : zs[j], mk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half8_t a = __builtin_bit_cast(half8_t, s.a[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], acc[i][j], 0, 0, 0);
        }
        if (++cpos == spg) {   // the group's end: scale its sums once (uniform)
            cpos = 0;
            float sc[4];
            sc[0] = half_bits_to_float(s.s.x & 0xFFFFu);
            sc[1] = half_bits_to_float(s.s.x >> 16);
            sc[2] = half_bits_to_float(s.s.y & 0xFFFFu);
            sc[3] = half_bits_to_float(s.s.y >> 16);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) tot[i][j][r] = __builtin_fmaf(acc[i][j][r], sc[j], tot[i][j][r]);
                    acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
                }
        }
    };

    PrefillSlot ring[kPrefillPf];
#pragma unroll
    for (int u = 0; u < kPrefillPf; ++u) load(ring[u]);
    // Whole rounds of the ring, each slot computed and then reloaded unconditionally; the last
    // steps % kPrefillPf steps are left in the first slots.
    const int full_end = steps / kPrefillPf * kPrefillPf;
    int t0 = 0;
    for (; t0 < full_end; t0 += kPrefillPf) {
#pragma unroll
        for (int u = 0; u < kPrefillPf; ++u) {
            step(ring[u]);
            load(ring[u]);
        }
    }
#pragma unroll
    for (int u = 0; u + 1 < kPrefillPf; ++u)
        if (t0 + u < steps) step(ring[u]);

    // Lane holds rows 4 rl + r of each row block, its 4 columns: undo the row's rescale, store.
    if (!col_ok) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mb + 16 * i + 4 * rl + r;
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

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.N + kPrefillTileN - 1) / kPrefillTileN),
                    (unsigned)((a.M + kPrefillTileM - 1) / kPrefillTileM));
    if (a.qzeros == nullptr)
        hipLaunchKernelGGL(w4a16_prefill_kernel<true>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(w4a16_prefill_kernel<false>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a16
