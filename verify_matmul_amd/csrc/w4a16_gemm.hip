// W4A16 GEMV (M = 1) and small-M MFMA GEMM (M = 1..16) for gfx950.
//
// Work layout
//   * A column tile is 64 columns, one wave wide. Lane l owns 4 adjacent columns (one 128-bit
//     load per packed word row) and word row l / 16 of every 4-row step, so one wave-wide load
//     fetches 4 rows x 256 contiguous bytes.
//   * The `wk` waves of a workgroup share one column tile and split its K range into contiguous
//     pieces; their sums meet in LDS at the end. With enough column tiles (N >= 16384) every
//     workgroup owns a tile outright and no reduction ever leaves the CU.
//   * Narrow matrices also split K across `splits` workgroups. Their fp32 partials are written
//     with agent-scope atomic stores and the last workgroup to arrive (atomic counter) adds them
//     in slice order, so results are bit-identical from run to run. Because the partials are
//     themselves coherent atomic stores, publishing them needs only a wait for their completion,
//     not an L2 write-back. The pages reduce split-K through per-slice partials too on GPUs
//     without thread-block clusters (TensorFold PR #859, commit messages).
//
// Per step (32 K rows x 64 columns per wave)
//   * a ring of kPf steps of loads is kept in flight: every iteration issues exactly one step of
//     loads (clamped to the wave's last step past the end) so the in-order load counter lets
//     the compiler wait for the oldest step only;
//   * each packed word becomes 8 exact fp16 values (q - z) (w4a16_device.h);
//   * GEMV: v_dot2c_f32_f16 into one fp32 sum per column; the four word rows of a step are
//     added across lanes at the end. GEMM: one v_mfma_f32_16x16x32_f16 per word column
//     (16 rows x 16 columns x 32 K), activations padded with zero rows up to 16;
//   * sums are kept per quantisation group and scaled once at the group's end.
//
// Activations: fp16 after an exact per-row power-of-two rescale chosen from the row's largest
// exponent over the wave's K range. With few rows they are converted once into the wave's own
// LDS; with many rows each lane converts its MFMA fragment as it arrives.
//
// Why this shape (GRIMOIRE v1.7 release notes, 'What changed': a GEMV for one user and a
// matrix-engine GEMM for 2-16 rows; GRIMOIRE v1.8, 'What changed': the small-row kernel got
// faster from register budgeting and from splitting work over more threads): every
// configuration is bound by streaming the packed weights from HBM, so the VALU work is only
// the exact dequantisation and the loads stay in flight from the first instruction on.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {
namespace {

struct Slot {
    uint4 w;      // packed words of 4 columns, one word row
    uint2 s;      // fp16 scales of the 4 columns for the step's group
    uint32_t z;   // packed zero word of the columns (asymmetric only)
    uint4 a;      // raw bf16 activation fragment (per-step conversion only)
};

template <bool kMfma, bool kSym, bool kLdsA, int kWK, int kPf>
__global__ __launch_bounds__(kWK * 64) void w4a16_gemm_kernel(GemmArgs p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: K-range math stays scalar
    const int cl = lane & 15;   // column quad (and MFMA A row) of this lane
    const int rl = lane >> 4;   // word row within the step
    const int M = p.M;
    const int N = p.N;
    const int K = p.K;
    const int spg = p.g / kStepK;   // steps per quantisation group
    const int tile = blockIdx.x;
    const int split = blockIdx.y;
    const int steps = K / kStepK;
    const int sb = (int)((long long)split * steps / p.splits);
    const int se = (int)((long long)(split + 1) * steps / p.splits);
    const int wb = sb + (int)((long long)wave * (se - sb) / kWK);
    const int we = sb + (int)((long long)(wave + 1) * (se - sb) / kWK);   // we > wb (host)

    int *shift_lds = reinterpret_cast<int *>(smem) + wave * 16;   // this wave's per-row shifts
    unsigned char *region = smem + kWK * 16 * sizeof(int);
    half8_t *a_lds = reinterpret_cast<half8_t *>(region) + (size_t)wave * p.a_stride;

    const int n0 = tile * kTileN + cl * 4;
    const bool col_ok = n0 < N;
    const int nc = col_ok ? n0 : 0;            // clamped column for loads of dead lanes
    const int arow = cl < M ? cl : 0;          // clamped activation row (MFMA fragments)
    const uint32_t *qw_lane = p.qweight + (size_t)rl * N + nc;
    const uint16_t *sc_lane = p.scales + nc;
    const uint32_t *qz_lane = kSym ? nullptr : p.qzeros + nc / 8;
    const uint16_t *a_lane = p.A + (size_t)arow * K + rl * 8;

    auto load_slot = [&](int t) {
        Slot s;
        s.w = *reinterpret_cast<const uint4 *>(qw_lane + (size_t)t * 4 * N);
        const int gi = t / spg;
        s.s = *reinterpret_cast<const uint2 *>(sc_lane + (size_t)gi * N);
        s.z = kSym ? 0u : qz_lane[(size_t)gi * (N / 8)];
        if (!kLdsA) s.a = *reinterpret_cast<const uint4 *>(a_lane + (size_t)t * kStepK);
        return s;
    };

    // ---- the weight stream starts first ---------------------------------------------------
    Slot ring[kPf];
#pragma unroll
    for (int u = 0; u < kPf; ++u) ring[u] = load_slot(min(wb + u, we - 1));

    // ---- per-row exponent of the activations over this wave's K range --------------------
    const int nwr = (we - wb) * 4;   // packed word rows in the wave's range
    const int items = M * nwr;       // 8-value activation items
    if (lane < 16) shift_lds[lane] = 0;
    for (int it = lane; it < items; it += 64) {
        const int m = it / nwr;
        const int wr = it - m * nwr;
        const uint4 raw = *reinterpret_cast<const uint4 *>(p.A + (size_t)m * K + (size_t)(wb * 4 + wr) * 8);
        const uint32_t e = max_exp8(raw);
        if (e) atomicMax(&shift_lds[m], (int)e);
    }
    if (lane < 16) shift_lds[lane] = act_shift((uint32_t)shift_lds[lane]);
    if (kLdsA) {
        for (int it = lane; it < items; it += 64) {
            const int m = it / nwr;
            const int wr = it - m * nwr;
            const uint4 raw = *reinterpret_cast<const uint4 *>(p.A + (size_t)m * K + (size_t)(wb * 4 + wr) * 8);
            a_lds[wr * M + m] = act8_to_slots(raw, pow2_neg(shift_lds[m]));
        }
    }
    const float a_mul = pow2_neg(shift_lds[arow]);   // per-step conversion of this lane's row

    // ---- stream ------------------------------------------------------------------------
    const Masks mk = make_masks();
    const half8_t zero8 = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    float4_t acc[4];
    float4_t tot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
        tot[j] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    ZeroSub zs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) zs[j] = zero_sub_sym();
    int zs_group = -1;

    for (int t0 = wb; t0 < we; t0 += kPf) {
#pragma unroll
        for (int u = 0; u < kPf; ++u) {
            const int t = t0 + u;
            if (t < we) {
                const Slot &cur = ring[u];
                half8_t a;
                if (kLdsA) {
                    const int wrow = (t - wb) * 4 + rl;
                    if (kMfma) {
                        a = zero8;
                        if (cl < M) a = a_lds[wrow * M + cl];
                    } else {
                        a = a_lds[wrow];
                    }
                } else {
                    a = act8_to_slots(cur.a, a_mul);
                    if (cl >= M) a = zero8;
                }
                if (!kSym) {   // zero points change once per group (uniform branch)
                    const int gi = t / spg;
                    if (gi != zs_group) {
                        zs_group = gi;
#pragma unroll
                        for (int j = 0; j < 4; ++j) zs[j] = zero_sub(zero_of(cur.z, (uint32_t)(nc + j)));
                    }
                }
                const uint32_t words[4] = {cur.w.x, cur.w.y, cur.w.z, cur.w.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half8_t b = dequant_word(words[j], kSym ? zero_sub_sym() : zs[j], mk);
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
                if (((t + 1) % spg == 0) || (t + 1 == we)) {
                    const float s4[4] = {half_bits_to_float(cur.s.x & 0xFFFFu), half_bits_to_float(cur.s.x >> 16),
                                         half_bits_to_float(cur.s.y & 0xFFFFu), half_bits_to_float(cur.s.y >> 16)};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
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
            }
            ring[u] = load_slot(min(t + kPf, we - 1));
        }
    }

    // ---- this wave's sums: add the word rows (GEMV), undo the activation rescale ---------------
    // GEMM: lane holds rows 4*rl + r of its 4 columns. GEMV: lanes with rl == 0 hold row 0.
    constexpr int kRows = kMfma ? 4 : 1;
    if (!kMfma) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
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
        for (int j = 0; j < 4; ++j) tot[j][r] = __builtin_amdgcn_ldexpf(tot[j][r], sh);
    }

    auto store_out = [&](int m, int n, float v) {
        if (p.out_bf16)
            static_cast<uint16_t *>(p.out)[(size_t)m * N + n] = (uint16_t)float_to_bf16_bits(v);
        else
            static_cast<float *>(p.out)[(size_t)m * N + n] = v;
    };

    if (kWK == 1 && p.splits == 1) {
        if (!holder || !col_ok) return;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int m = row_base + r;
            if (m >= M) break;
            const size_t o = (size_t)m * N + n0;
            if (p.out_bf16) {
                uint2 v;
                v.x = float_to_bf16_bits(tot[0][r]) | (float_to_bf16_bits(tot[1][r]) << 16);
                v.y = float_to_bf16_bits(tot[2][r]) | (float_to_bf16_bits(tot[3][r]) << 16);
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + o) = v;
            } else {
                *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o) =
                    make_float4(tot[0][r], tot[1][r], tot[2][r], tot[3][r]);
            }
        }
        return;
    }

    // ---- cross-wave reduction in LDS, in wave order ---------------------------------------
    float *red = reinterpret_cast<float *>(region);   // [kWK][M][64]; the staged activations are dead
    if (kWK > 1) {
        __syncthreads();
        if (holder) {
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const int m = row_base + r;
                if (m < M) {
                    float *dst = red + ((size_t)wave * M + m) * kTileN + cl * 4;
                    *reinterpret_cast<float4_t *>(dst) = float4_t{tot[0][r], tot[1][r], tot[2][r], tot[3][r]};
                }
            }
        }
        __syncthreads();
    } else {
        // one wave: stage its sums the same way so the split-K path below has one layout
        if (holder) {
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const int m = row_base + r;
                if (m < M) {
                    float *dst = red + (size_t)m * kTileN + cl * 4;
                    *reinterpret_cast<float4_t *>(dst) = float4_t{tot[0][r], tot[1][r], tot[2][r], tot[3][r]};
                }
            }
        }
        __syncthreads();
    }
    constexpr int kThreads = kWK * 64;
    for (int idx = tid; idx < M * kTileN; idx += kThreads) {
        const int m = idx / kTileN;
        const int c = idx - m * kTileN;
        float v = red[(size_t)m * kTileN + c];
#pragma unroll
        for (int w = 1; w < kWK; ++w) v += red[((size_t)w * M + m) * kTileN + c];
        const int n = tile * kTileN + c;
        if (n >= N) continue;
        if (p.splits == 1)
            store_out(m, n, v);
        else
            __hip_atomic_store(p.partials + ((size_t)split * M + m) * N + n, v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (p.splits == 1) return;

    // ---- split-K across workgroups: the last to arrive adds the slices in order -------------
    // The partials above are agent-scope atomic stores: once complete (waitcnt) they are
    // visible to every CU, so the counter increment after the barrier publishes them.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned)(p.splits - 1);
    }
    __syncthreads();
    if (!s_last) return;
    for (int idx = tid; idx < M * kTileN; idx += kThreads) {
        const int m = idx / kTileN;
        const int c = idx - m * kTileN;
        const int n = tile * kTileN + c;
        if (n >= N) continue;
        float v = 0.f;
        for (int sp = 0; sp < p.splits; ++sp)
            v += __hip_atomic_load(p.partials + ((size_t)sp * M + m) * N + n, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        store_out(m, n, v);
    }
    if (tid == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kPf = 4;

template <bool kMfma, bool kSym, bool kLdsA, int kWK>
hipError_t launch_one(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream)
{
    const auto kern = w4a16_gemm_kernel<kMfma, kSym, kLdsA, kWK, kPf>;
    if (plan.lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)((a.N + kTileN - 1) / kTileN), (unsigned)a.splits);
    hipLaunchKernelGGL(kern, grid, dim3(kWK * 64), plan.lds, stream, a);
    return hipGetLastError();
}

template <bool kMfma, bool kSym, bool kLdsA>
hipError_t launch_wk(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream)
{
    switch (plan.wk) {
    case 1: return launch_one<kMfma, kSym, kLdsA, 1>(a, plan, stream);
    case 2: return launch_one<kMfma, kSym, kLdsA, 2>(a, plan, stream);
    case 4: return launch_one<kMfma, kSym, kLdsA, 4>(a, plan, stream);
    case 8: return launch_one<kMfma, kSym, kLdsA, 8>(a, plan, stream);
    case 16: return launch_one<kMfma, kSym, kLdsA, 16>(a, plan, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &a, const GemmPlan &plan, hipStream_t stream)
{
    const bool sym = a.qzeros == nullptr;
    if (!plan.mfma) {   // GEMV: one row, activations always staged
        return sym ? launch_wk<false, true, true>(a, plan, stream) : launch_wk<false, false, true>(a, plan, stream);
    }
    if (plan.lds_a)
        return sym ? launch_wk<true, true, true>(a, plan, stream) : launch_wk<true, false, true>(a, plan, stream);
    return sym ? launch_wk<true, true, false>(a, plan, stream) : launch_wk<true, false, false>(a, plan, stream);
}

}  // namespace w4a16
