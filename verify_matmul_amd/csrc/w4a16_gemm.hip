// W4A16 GEMV (M = 1) and small-M MFMA GEMM (M = 2..16) for gfx950.
//
// Both kernels share one skeleton:
//   * A workgroup is 4 waves side by side along N (256 columns) and one K-slice. Lane l of a
//     wave owns 4 adjacent columns (one 128-bit load per packed word row) and word row l / 16
//     of every 4-row step, so one wave-wide load fetches 4 rows x 256 contiguous bytes.
//   * The workgroup first stages its K-slice of the activations in LDS, converted to fp16
//     after an exact per-row power-of-two rescale and permuted into the dequantiser's slot
//     order (see w4a16_device.h), so every wave reads ready operands with one ds_read_b128.
//   * The K loop streams packed words with a PF-deep register prefetch ring, dequantises each
//     word into 8 exact fp16 values of (q - z), and multiply-accumulates:
//       GEMV: v_dot2c_f32_f16 into one fp32 sum per column, then a cross-lane reduction over
//             the four word rows of a step;
//       GEMM: one v_mfma_f32_16x16x32_f16 per word column (16 rows x 16 columns x 32 K), the
//             activations padded with zero rows up to 16.
//     Sums are kept per quantisation group and scaled once at the group's end.
//   * Split-K: each K-slice writes fp32 partials; the last workgroup of a column tile to
//     arrive (atomic counter) adds the partials in slice order and writes the output, so the
//     result is bit-identical from run to run. The pages' split-K on GPUs without thread-block
//     clusters also reduces through per-slice partials (TensorFold PR #859, commit messages).
//
// Why this shape (GRIMOIRE v1.7 release notes, 'What changed': a GEMV for one user and a
// matrix-engine GEMM for 2-16 rows; GRIMOIRE v1.8, 'What changed': the small-row kernel got
// faster from register budgeting and from splitting work over more threads): every
// configuration is bound by streaming the packed weights from HBM, so the design spends
// VALU only on the exact dequantisation (about 1.1 operations per weight) and keeps enough
// loads in flight per CU to cover HBM latency.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {
namespace {

constexpr int kWaves = kTileN / 64;
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ uint4 load_words(const uint32_t *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

template <bool kMfma, bool kSym, int kPf>
__global__ __launch_bounds__(kThreads) void w4a16_gemm_kernel(GemmArgs p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    int *row_e = reinterpret_cast<int *>(smem);                    // [16]: exponent, then shift
    half8_t *a_lds = reinterpret_cast<half8_t *>(smem + kLdsHeader);  // [word row][M] slots
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cl = lane & 15;   // column quad within the wave
    const int rl = lane >> 4;   // word row within the step
    const int M = p.M;
    const int N = p.N;
    const int tile = blockIdx.x;
    const int split = blockIdx.y;
    const int steps = p.K / kStepK;
    const int sb = (int)((long long)split * steps / p.splits);
    const int se = (int)((long long)(split + 1) * steps / p.splits);
    const int wr0 = sb * 4;            // first packed word row of the slice
    const int nwr = (se - sb) * 4;     // packed word rows in the slice

    // ---- stage activations: per-row exponent, then exact rescale to fp16 slots ------------
    if (tid < 16) row_e[tid] = 0;
    __syncthreads();
    const int items = M * nwr;
    for (int it = tid; it < items; it += kThreads) {
        const int m = it / nwr;
        const int wr = it - m * nwr;
        const uint4 raw = *reinterpret_cast<const uint4 *>(p.A + (size_t)m * p.K + (size_t)(wr0 + wr) * 8);
        const uint32_t e = max_exp8(raw);
        if (e) atomicMax(&row_e[m], (int)e);
    }
    __syncthreads();
    if (tid < 16) row_e[tid] = act_shift((uint32_t)row_e[tid]);
    __syncthreads();
    for (int it = tid; it < items; it += kThreads) {
        const int m = it / nwr;
        const int wr = it - m * nwr;
        const uint4 raw = *reinterpret_cast<const uint4 *>(p.A + (size_t)m * p.K + (size_t)(wr0 + wr) * 8);
        a_lds[wr * M + m] = act8_to_slots(raw, row_e[m]);
    }
    __syncthreads();

    // ---- stream the weights ------------------------------------------------------------------
    const int n0 = tile * kTileN + wave * 64 + cl * 4;   // first of this lane's 4 columns
    const bool col_ok = n0 < N;
    const Masks mk = make_masks();
    const size_t step_stride = (size_t)4 * N;
    const uint32_t *qw = p.qweight + (size_t)(wr0 + rl) * N + n0;

    uint4 ring[kPf];
#pragma unroll
    for (int u = 0; u < kPf; ++u) {
        ring[u] = make_uint4(0, 0, 0, 0);
        if (sb + u < se && col_ok) ring[u] = load_words(qw + (size_t)u * step_stride);
    }

    float4_t acc[4];   // per-group sums (GEMM: 16x16 tile per word column; GEMV: element 0)
    float4_t tot[4];   // scaled totals
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
        tot[j] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    ZeroSub zs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) zs[j] = zero_sub_sym();
    uint2 sc = make_uint2(0, 0);
    int cur_group = -1;
    const half8_t zero8 = half8_t{0, 0, 0, 0, 0, 0, 0, 0};

    for (int t0 = sb; t0 < se; t0 += kPf) {
#pragma unroll
        for (int u = 0; u < kPf; ++u) {
            const int t = t0 + u;
            if (t >= se) break;
            const uint4 wv = ring[u];
            if (t + kPf < se && col_ok) ring[u] = load_words(qw + (size_t)(t + kPf - sb) * step_stride);

            const int gi = (t * kStepK) / p.g;
            if (gi != cur_group) {
                cur_group = gi;
                sc = make_uint2(0, 0);
                if (col_ok) sc = *reinterpret_cast<const uint2 *>(p.scales + (size_t)gi * N + n0);
                if (!kSym) {
                    const uint32_t zw = col_ok ? p.qzeros[(size_t)gi * (N / 8) + n0 / 8] : 0u;
#pragma unroll
                    for (int j = 0; j < 4; ++j) zs[j] = zero_sub(zero_of(zw, (uint32_t)(n0 + j)));
                }
            }

            const int wrow = (t - sb) * 4 + rl;
            half8_t a;
            if (kMfma) {
                a = zero8;
                if (cl < M) a = a_lds[wrow * M + cl];
            } else {
                a = a_lds[wrow];
            }
            const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
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

            const bool group_end = (((t + 1) * kStepK) % p.g == 0) || (t + 1 == se);
            if (group_end) {
                const float s4[4] = {half_bits_to_float(sc.x & 0xFFFFu), half_bits_to_float(sc.x >> 16),
                                     half_bits_to_float(sc.y & 0xFFFFu), half_bits_to_float(sc.y >> 16)};
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
    }

    // ---- finish: cross-lane reduction (GEMV), undo the activation rescale --------------------
    // GEMM: lane holds rows 4*rl + r of its 4 columns. GEMV: sum the 4 word rows of a step.
    if (!kMfma) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = tot[j][0];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            tot[j][0] = v;
        }
    }
    const int rows_here = kMfma ? 4 : 1;
    const int row_base = kMfma ? 4 * rl : 0;
    const bool writer = col_ok && (kMfma || rl == 0);
#pragma unroll
    for (int r = 0; r < rows_here; ++r) {
        const int m = row_base + r;
        const int sh = m < M ? row_e[m] : 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) tot[j][r] = __builtin_amdgcn_ldexpf(tot[j][r], sh);
    }

    if (p.splits == 1) {
        if (!writer) return;
#pragma unroll
        for (int r = 0; r < rows_here; ++r) {
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

    // ---- split-K: publish this slice's partials, last arriver reduces in slice order --------
    if (writer) {
#pragma unroll
        for (int r = 0; r < rows_here; ++r) {
            const int m = row_base + r;
            if (m >= M) break;
            float *dst = p.partials + ((size_t)split * M + m) * N + n0;
            *reinterpret_cast<float4 *>(dst) = make_float4(tot[0][r], tot[1][r], tot[2][r], tot[3][r]);
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (unsigned)(p.splits - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    constexpr int kQuads = kTileN / 4;
    for (int it = tid; it < M * kQuads; it += kThreads) {
        const int m = it / kQuads;
        const int n = tile * kTileN + (it - m * kQuads) * 4;
        if (n >= N) continue;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp = 0; sp < p.splits; ++sp) {
            const float4_t v = *reinterpret_cast<const float4_t *>(p.partials + ((size_t)sp * M + m) * N + n);
            s.x += v[0]; s.y += v[1]; s.z += v[2]; s.w += v[3];
        }
        const size_t o = (size_t)m * N + n;
        if (p.out_bf16) {
            uint2 v;
            v.x = float_to_bf16_bits(s.x) | (float_to_bf16_bits(s.y) << 16);
            v.y = float_to_bf16_bits(s.z) | (float_to_bf16_bits(s.w) << 16);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + o) = v;
        } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o) = s;
        }
    }
    if (tid == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool kMfma, bool kSym>
hipError_t launch_variant(const GemmArgs &a, hipStream_t stream)
{
    constexpr int kPf = 8;
    const dim3 grid((unsigned)((a.N + kTileN - 1) / kTileN), (unsigned)a.splits);
    const size_t lds = gemm_lds_bytes(a.M, a.K, a.splits);
    hipLaunchKernelGGL((w4a16_gemm_kernel<kMfma, kSym, kPf>), grid, dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream)
{
    const bool sym = a.qzeros == nullptr;
    if (a.M == 1) return sym ? launch_variant<false, true>(a, stream) : launch_variant<false, false>(a, stream);
    return sym ? launch_variant<true, true>(a, stream) : launch_variant<true, false>(a, stream);
}

}  // namespace w4a16
