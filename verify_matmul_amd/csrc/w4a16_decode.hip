// W4A16 decode GEMM for gfx950: one row (dot-product GEMV) or 2..16 rows (matrix cores), with
// the activation slice of a workgroup converted once and shared by all of its column tiles.
//
// Work layout
//   * A workgroup is `tiles` x `kw` waves over one K slice. Wave (w, k) owns column tile w of
//     the workgroup (64 columns, 4 adjacent per lane, or 128, 8 per lane) and K piece k of the
//     slice. The tiles are adjacent, so at every step the workgroup reads `tiles` x 256 (or 512)
//     contiguous bytes of each word row it touches: measured on MI355X, reading the FFN matrix's
//     codes with four adjacent tiles per workgroup takes 8.2-8.7 us against 9.4 us when the
//     waves of a workgroup all split one tile's K range.
//   * The slice's activations (all M rows) are loaded once by the whole workgroup, rescaled per
//     row by one exact power of two, and stored in LDS as fp16 fragments in the order the dot
//     products or the matrix cores read them. Had every wave loaded its own fragments from L2,
//     the same read would take 14-21 us.
//   * The `kw` pieces of a tile are added in LDS in piece order; `slices` workgroups cover each
//     group of columns along K, their fp32 sums meeting in scratch, where the last workgroup to
//     start adds them in slice order. Splitting K inside the workgroup moves no partial sums
//     through memory; slices across workgroups write and read `slices - 1` copies of the output.
//
// Per step (32 K rows): each packed word becomes 8 exact fp16 values (q - z) (w4a16_device.h);
// the GEMV multiplies them with v_dot2c_f32_f16, the matrix-core path with one
// v_mfma_f32_16x16x32_f16 per word column (rows past M are not stored). Sums are kept per
// quantisation group and scaled once in fp32 at the group's end, so (q - z) * scale never rounds
// before accumulation (GRIMOIRE v1.7 release notes, 'What changed': an exact (q - z) * scale
// dequantisation, a GEMV for one user and a matrix-engine kernel for 2-16 rows).
//
// The weights are loaded with non-temporal 16-byte buffer loads (each byte is read once per call)
// into a ring of `kU` steps per wave, issued before the activation slice is converted so that
// they are in flight from the first instructions on.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Buffer resource over `bytes` bytes at `base`: accesses past the end read zero and write
// nothing, without a memory request.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kCoherent = 16;     // cache-policy operand of the buffer builtins: sc1 (agent scope)
constexpr int kNonTemporal = 2;   // and: nt

constexpr int kHeld = kDecHeld;

// LDS position (in 16-byte fragments) of the matrix-core fragment of row m, word row wr of the
// slice, with the rows stored padded to mp = 4, 8 or 16 (the smallest that holds M; mp_log2 is
// its log2): step t = wr / 4 holds 4 mp fragments, fragment q * mp + m is row m, K quarter q. The
// row index is XOR-swizzled with the step (and K quarter) so that 16 lanes writing 16
// consecutive word rows of one row hit 16 different LDS bank groups; the 16 lanes of a K
// quarter reading a step read mp consecutive fragments.
__device__ __forceinline__ int frag_swz(int t, int q, int mp_log2)
{
    // mp = 16: ((t & 3) << 2) | q; mp = 8: ((t & 3) << 1) | (q >> 1); mp = 4: t & 3 (q < 4), in one
    // form without branches (mp_log2 is uniform)
    return ((t & 3) << (mp_log2 - 2)) | (q >> (4 - mp_log2));
}
__device__ __forceinline__ int frag_pos(int m, int wr, int mp_log2)
{
    const int t = wr >> 2, q = wr & 3;
    return ((t * 4 + q) << mp_log2) + (m ^ frag_swz(t, q, mp_log2));
}

// kLd: 16-byte weight loads per lane and step. GPTQ codes: kLd = kV (one word row of 4 * kV
// columns). Affine codes (kZM == kAffine, 4 columns per lane): each column is a bit stream of
// kBits bits per row, so a step's 32 rows are kBits word rows, and a lane's 8 rows are 8 * kBits
// bits that start at bit 8 * kBits * (lane's K quarter) of the step: in one word row for 1, 2 and
// 4 bits (kLd = 1), in two consecutive ones otherwise (kLd = 2; 3, 5, 6 and 8 bits).
// kSub: 32-row steps per ring slot. 1, or for 1- and 2-bit affine codes 4 / kBits: then lane q
// loads word q of a block of kSub steps (each lane a word of its own, where at kSub = 1 two or
// four lanes would load the same word for 8 rows each) and holds rows 32 q / kBits onwards, i.e.
// 8-row chunks kSub * q .. kSub * q + kSub - 1 of the block; the block takes kSub matrix-core
// products (or dot-product rounds) per column, product h pairing each lane's chunk kSub * q + h
// of the codes with the same chunk of the activations. Slices and pieces are whole blocks.
template <bool kMfma, int kZM, int kU, int kV, int kLd = kV, int kBits = 4, int kSub = 1>
__global__ __launch_bounds__(kDecMaxWaves * 64) void decode_kernel(DecodeArgs p)
{
    constexpr bool kAff = kZM == kAffine;
    static_assert(!kAff || kLd == ((kBits == 1 || kBits == 2 || kBits == 4) ? 1 : 2), "word rows per lane and step");
    static_assert(!kAff || kV == 1, "affine codes run on 64-column tiles");
    static_assert(kSub == 1 || (kAff && kSub * kBits == 4), "blocks of steps: 1- and 2-bit affine codes");
    constexpr int kC = 4 * kV;      // adjacent columns per lane
    constexpr int kTile = 16 * kC;  // columns per wave
    constexpr int kRows = kMfma ? 4 : 1;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_last, s_failed, s_pick_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NW = p.tiles * p.kw;              // waves of the workgroup
    const int T = NW * 64;
    const int w_tile = wave % p.tiles;          // the wave's column tile
    const int w_k = wave / p.tiles;             // and K piece
    const int cl = lane & 15;   // column block of the lane (and its MFMA A row)
    const int rl = lane >> 4;   // word row of the lane within a step
    const int M = p.M, N = p.N, K = p.K;
    const int spg = p.g / kStepK;
    const int P = p.slices;
    const int cg = blockIdx.x / P;              // group of columns
    const int sl = blockIdx.x - cg * P;         // K slice
    const int steps = K / kStepK;
    const int units = steps / kSub;   // blocks of kSub steps (host: K % (32 kSub) == 0)
    const int sb = kSub * (int)((long long)sl * units / P);
    const int se = kSub * (int)((long long)(sl + 1) * units / P);   // se > sb (host: slices <= units)
    const int su = (se - sb) / kSub;
    const int wb = sb + kSub * (int)((long long)w_k * su / p.kw);          // the wave's piece [wb, we)
    const int we = sb + kSub * (int)((long long)(w_k + 1) * su / p.kw);    // (host: slices * kw <= units)
    const int g0 = sb / spg;
    const int ng = (se - 1) / spg - g0 + 1;
    const int WC = p.tiles * kTile;             // columns of the workgroup
    const int c0 = cg * WC;
    const int lcol = w_tile * kTile + cl * kC;  // the lane's first column within the workgroup
    const int n0 = c0 + lcol;
    const bool col_ok = n0 < N;                 // N % 8 == 0, so a lane's columns are all in or all out
    const int nc = col_ok ? n0 : 0;

    uint32_t arrival = 0;
    if (P > 1 && tid == 0)
        arrival = __hip_atomic_fetch_add(&p.counters[cg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    uint32_t *rowmax = reinterpret_cast<uint32_t *>(smem);                   // [16] largest |a| bits per row
    uint4 *a_lds = reinterpret_cast<uint4 *>(smem + p.a_off);                // fp16 fragments
    uint16_t *sc_lds = reinterpret_cast<uint16_t *>(smem + p.s_off);         // [group][WC] scales
    uint32_t *z_lds = reinterpret_cast<uint32_t *>(smem + p.z_off);          // [group][WC/8] zero words
    float *red = reinterpret_cast<float *>(smem + p.r_off);                  // [kw-1][tiles][kC*kRows][64]

    // ---- 1. scales and zero words of the workgroup's columns and groups, straight into LDS ----
    {
        const int per = WC / 8;   // 16-byte scale items (and zero words) per group
        const int sitems = ng * per;
        for (int b = wave * 64; b < sitems; b += T) {
            const int it = b + lane;
            const int gi = g0 + it / per;
            int c = c0 + (it - (it / per) * per) * 8;
            if (c >= N) c = 0;
            if (it < sitems) load_to_lds16(p.scales + (size_t)gi * N + c, sc_lds + (size_t)b * 8);
        }
        if constexpr (kZM == kZeroPacked) {
            for (int b = wave * 64; b < sitems; b += T) {
                const int it = b + lane;
                const int gi = g0 + it / per;
                int c = c0 + (it - (it / per) * per) * 8;
                if (c >= N) c = 0;
                if (it < sitems) load_to_lds4(p.qzeros + (size_t)gi * (N / 8) + c / 8, z_lds + b);
            }
        }
        if constexpr (kAff) {   // the biases, laid out as the scales, over the zero words' region
            uint16_t *bi_lds = reinterpret_cast<uint16_t *>(z_lds);
            for (int b = wave * 64; b < sitems; b += T) {
                const int it = b + lane;
                const int gi = g0 + it / per;
                int c = c0 + (it - (it / per) * per) * 8;
                if (c >= N) c = 0;
                if (it < sitems) load_to_lds16(p.biases + (size_t)gi * N + c, bi_lds + (size_t)b * 8);
            }
        }
    }
    asm volatile("" ::: "memory");

    // ---- 2. the activation slice into registers ---------------------------------------------
    // Item = (row m, word row wr) of 8 bf16 values. With at least as many rows as waves, wave v
    // takes whole rows v, v + NW, ...; otherwise each row is shared by `wr_w` = NW / M waves, each
    // taking every wr_w-th block of 64 word rows. A lane takes word rows lane, lane + 64 * wr_w, ...
    // of each of its rows: item j of a lane is chunk j % chunks of the wave's row j / chunks. The
    // first kHeld items stay in registers from the row-maximum pass to the conversion; a longer
    // slice reads the rest twice (L2 hits).
    const int NWR = (se - sb) * 4;                        // word rows of the slice
    const bool by_row = M >= NW;
    const int wr_w = by_row ? 1 : NW / M;                 // waves per row
    const int m_first = by_row ? wave : wave / wr_w;      // >= M: the wave holds no activations
    const int part = by_row ? 0 : wave - (wave / wr_w) * wr_w;
    const int rstep = by_row ? NW : M;                    // to the wave's next row
    const int chunks = (NWR + 64 * wr_w - 1) / (64 * wr_w);
    const int rows_w = m_first >= M ? 0 : (M - 1 - m_first) / rstep + 1;   // rows of the wave
    const int n_items = rows_w * chunks;                  // items per lane (uniform)
    const uint16_t *a_slice = p.A + (size_t)sb * 32;
    auto item_src = [&](int i_m, int c) {
        const int wr = (part + c * wr_w) * 64 + lane;
        return wr < NWR ? a_slice + (size_t)i_m * K + (size_t)wr * 8 : nullptr;
    };
    uint4 held[kHeld];
    {
        int i_m = m_first, c = 0;
#pragma unroll
        for (int j = 0; j < kHeld; ++j) {
            held[j] = uint4{0u, 0u, 0u, 0u};
            if (j < n_items) {
                const uint16_t *src = item_src(i_m, c);
                if (src) held[j] = *reinterpret_cast<const uint4 *>(src);
            }
            if (++c == chunks) {
                c = 0;
                i_m += rstep;
            }
        }
    }
    asm volatile("" ::: "memory");

    // ---- 3. the weight ring ----------------------------------------------------------------
    // A buffer resource over exactly the word rows of the wave's piece: the ring reloads steps
    // past the piece unconditionally (no branch in the loop), and those reads return zero without
    // a memory request (over the whole slice they would fetch the next piece's first steps
    // again). Non-temporal: every byte is read once per call.
    constexpr int R = kAff ? kBits : 4;   // word rows per step
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(p.qweight + (size_t)wb * R * N, (uint32_t)((we - wb) * R * 4 * N));
    // affine codes: the lane's 8 rows start at bit `a_bit` of the step, in word row a_bit / 32
    // (blocks of kSub > 1 steps: word row rl of the block)
    const int a_bit = kAff && kSub == 1 ? 8 * kBits * rl : 0;
    const uint32_t w_lane = ((uint32_t)(kAff && kSub == 1 ? a_bit >> 5 : rl) * (uint32_t)N + (uint32_t)nc) * 4u;   // bytes (< 2 GiB)
    uint4 ring[kU][kLd];
    auto load_w = [&](uint4 *dst, int t) {
#pragma unroll
        for (int v = 0; v < kLd; ++v) {   // GPTQ: the next 4 columns; affine: the next word row
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
                wrs, (int)(w_lane + (uint32_t)(t - wb) * (uint32_t)R * 4u * (uint32_t)N + (kAff ? 4u * (uint32_t)N : 16u) * v),
                0, kNonTemporal);
            dst[v] = uint4{x.x, x.y, x.z, x.w};
        }
    };
    // (issued in slot order, each behind a compiler barrier: the loop waits for slot u with
    // exactly kU - 1 later loads outstanding, which holds on its first round only if the
    // prologue issued the slots in the same order)
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        load_w(ring[u], wb + u * kSub);
        asm volatile("" ::: "memory");
    }

    // ---- 4. row maxima, then the fp16 fragments ---------------------------------------------
    if (tid < 16) rowmax[tid] = 0u;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kU * kLd));   // all but the ring: scales, zeros or biases, activations
    __syncthreads();                                  // every wave's direct loads have landed
    {   // each wave: the largest magnitude of each of its rows, one LDS atomic per row
        int i_m = m_first, c = 0;
        uint32_t run = 0;
        auto fold = [&](uint4 x) {   // one item of row i_m; the row's last folds the row maximum in
            run = max(run, max_mag8(x));
            if (++c == chunks) {
                run = wave_max_u32(run);
                if (lane == 0 && run) atomicMax(&rowmax[i_m], run);
                run = 0;
                c = 0;
                i_m += rstep;
            }
        };
#pragma unroll
        for (int j = 0; j < kHeld; ++j)
            if (j < n_items) fold(held[j]);
        for (int j = kHeld; j < n_items; ++j) {   // a long slice: items past the held ones
            const uint16_t *src = item_src(i_m, c);
            fold(src ? *reinterpret_cast<const uint4 *>(src) : uint4{0u, 0u, 0u, 0u});
        }
    }
    __syncthreads();
    const int mp_log2 = p.mp_log2;
    {
        int i_m = m_first, c = 0;
        float mul = i_m < M ? pow2_neg(act_shift(rowmax[i_m] >> 7)) : 0.f;
        auto put = [&](uint4 x, bool ok) {   // one item of row i_m, as an fp16 fragment
            if (ok) {
                const int wr = (part + c * wr_w) * 64 + lane;
                a_lds[kMfma ? frag_pos(i_m, wr, mp_log2) : wr] = __builtin_bit_cast(uint4, act8_to_slots(x, mul));
            }
            if (++c == chunks) {
                c = 0;
                i_m += rstep;
                mul = i_m < M ? pow2_neg(act_shift(rowmax[i_m] >> 7)) : 0.f;
            }
        };
#pragma unroll
        for (int j = 0; j < kHeld; ++j)
            if (j < n_items) put(held[j], item_src(i_m, c) != nullptr);
        for (int j = kHeld; j < n_items; ++j) {
            const uint16_t *src = item_src(i_m, c);
            put(src ? *reinterpret_cast<const uint4 *>(src) : uint4{0u, 0u, 0u, 0u}, src != nullptr);
        }
    }
    __syncthreads();

    // ---- 5. stream the wave's piece ------------------------------------------------------------
    const Masks mk = make_masks();
    float4_t acc[kC], tot[kC];
#pragma unroll
    for (int j = 0; j < kC; ++j) {
        acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
        tot[j] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    ZeroSub zs[kC];
#pragma unroll
    for (int j = 0; j < kC; ++j) zs[j] = zero_sub_sym();
    // affine codes: the sums of the activations themselves (times the group's bias), from one
    // more product per step against ones; and the bit positions of the lane's 8 codes (rows k0..k3
    // from bit a_off of its first word, rows k4..k7 from a_off + 4 * bits)
    float4_t acc_one = float4_t{0.f, 0.f, 0.f, 0.f};
    const int a_off = a_bit & 31, a_off4 = a_off + 4 * kBits;
    const half8_t ones = half8_t{1, 1, 1, 1, 1, 1, 1, 1};
    int gi = wb / spg, gpos = wb - (wb / spg) * spg;
    bool first = true;
    // the lane's matrix-core fragment within a step: lane q * 16 + m reads row m, K quarter q.
    // Lanes of rows past the stored ones read row m mod mp: an MFMA row only feeds its own output
    // row, and output rows past M are never stored.
    const int mp = 1 << mp_log2;
    const int q_l = lane >> 4;
    const int lx = (q_l << mp_log2) + ((cl & (mp - 1)) ^ (q_l >> (4 - mp_log2)));
    const int sx = mp_log2 - 2;   // the step's swizzle: (t mod 4) << sx

    auto step = [&](int t, const uint4 *wv) {
        const bool last = gpos + kSub == spg || t + kSub == we;   // (host: spg % kSub == 0)
        const int tt = t - sb;
        const half8_t a = __builtin_bit_cast(half8_t, kMfma ? a_lds[((tt * 4) << mp_log2) + (lx ^ ((tt & 3) << sx))]
                                                            : a_lds[tt * 4 + rl]);
        if (kZM == kZeroPacked && first) {   // zero points change once per group (uniform)
            const uint32_t zw = z_lds[(gi - g0) * (WC / 8) + lcol / 8];
#pragma unroll
            for (int j = 0; j < kC; ++j) zs[j] = zero_sub(zero_of(zw, (uint32_t)(lcol + j)));
        }
        uint32_t words[kC], words1[kC];
#pragma unroll
        for (int v = 0; v < kV; ++v) {
            words[4 * v] = wv[v].x;
            words[4 * v + 1] = wv[v].y;
            words[4 * v + 2] = wv[v].z;
            words[4 * v + 3] = wv[v].w;
        }
        if constexpr (kAff && kLd == 2) {
            words1[0] = wv[1].x;
            words1[1] = wv[1].y;
            words1[2] = wv[1].z;
            words1[3] = wv[1].w;
        }
        auto mac = [&](const half8_t &x, const half8_t &b, float4_t &c) {
            if constexpr (kMfma) {
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, b, c, 0, 0, 0);
            } else {
                float s = c[0];
                s = __builtin_amdgcn_fdot2(b.lo.lo, x.lo.lo, s, false);
                s = __builtin_amdgcn_fdot2(b.lo.hi, x.lo.hi, s, false);
                s = __builtin_amdgcn_fdot2(b.hi.lo, x.hi.lo, s, false);
                s = __builtin_amdgcn_fdot2(b.hi.hi, x.hi.hi, s, false);
                c[0] = s;
            }
        };
        if constexpr (kSub > 1) {   // a block of kSub steps: one product per 8-row chunk of the lane's word
#pragma unroll
            for (int h = 0; h < kSub; ++h) {
                const int wr = tt * 4 + kSub * rl + h;   // the chunk's word row of the slice
                const half8_t x = __builtin_bit_cast(half8_t, kMfma ? a_lds[frag_pos(cl & (mp - 1), wr, mp_log2)] : a_lds[wr]);
                mac(x, ones, acc_one);   // the activations' own sums, for the bias
#pragma unroll
                for (int j = 0; j < kC; ++j)
                    mac(x, affine_codes<kBits>(words[j], 0u, 8 * kBits * h, 8 * kBits * h + 4 * kBits, mk), acc[j]);
            }
        } else {
            if constexpr (kAff) mac(a, ones, acc_one);   // the activations' own sums, for the bias
#pragma unroll
            for (int j = 0; j < kC; ++j) {
                half8_t b;
                if constexpr (kAff) {
                    b = affine_codes<kBits>(words[j], kLd == 2 ? words1[j] : 0u, a_off, a_off4, mk);
                } else {
                    b = dequant_word(words[j], kZM == kZeroSym ? zero_sub_sym() : zs[j], mk);
                }
                mac(a, b, acc[j]);
            }
        }
        if (last) {   // the group's scale, once, on fp32 sums
            const uint16_t *sp = sc_lds + (gi - g0) * WC + lcol;
            uint32_t sw[kC / 2];
            if constexpr (kC == 4) {
                const uint2 v = *reinterpret_cast<const uint2 *>(sp);
                sw[0] = v.x;
                sw[1] = v.y;
            } else {
                const uint4 q = *reinterpret_cast<const uint4 *>(sp);
                sw[0] = q.x;
                sw[1] = q.y;
                sw[2] = q.z;
                sw[3] = q.w;
            }
            uint32_t bw[kC / 2];   // affine: the group's biases, laid out as the scales
            if constexpr (kAff) {
                const uint2 v = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(z_lds) +
                                                                 (gi - g0) * WC + lcol);
                bw[0] = v.x;
                bw[1] = v.y;
            }
#pragma unroll
            for (int j = 0; j < kC; ++j) {
                const uint32_t sbits = (sw[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
                const float s = kAff ? bf16_bits_to_float(sbits) : half_bits_to_float(sbits);
                const float bias = kAff ? bf16_bits_to_float((bw[j / 2] >> (16 * (j & 1))) & 0xFFFFu) : 0.f;
                if constexpr (kMfma) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        tot[j][r] = __builtin_fmaf(acc[j][r], s, tot[j][r]);
                        if constexpr (kAff) tot[j][r] = __builtin_fmaf(acc_one[r], bias, tot[j][r]);
                    }
                    acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
                } else {
                    tot[j][0] = __builtin_fmaf(acc[j][0], s, tot[j][0]);
                    if constexpr (kAff) tot[j][0] = __builtin_fmaf(acc_one[0], bias, tot[j][0]);
                    acc[j][0] = 0.f;
                }
            }
            if constexpr (kAff) acc_one = float4_t{0.f, 0.f, 0.f, 0.f};
        }
        first = last;
        gpos += kSub;
        if (gpos == spg) {
            gpos = 0;
            ++gi;
        }
    };

    // Whole rounds of the ring: every step computes and reissues its slot unconditionally, so the
    // wait before a step covers only that slot.
    const int full_end = wb + (we - wb) / (kU * kSub) * (kU * kSub);
    int t0 = wb;
    for (; t0 < full_end; t0 += kU * kSub) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            step(t0 + u * kSub, ring[u]);
            load_w(ring[u], t0 + (u + kU) * kSub);   // past the slice: no memory request
        }
    }
#pragma unroll
    for (int u = 0; u + 1 < kU; ++u)
        if (t0 + u * kSub < we) step(t0 + u * kSub, ring[u]);

    // ---- 6. the K pieces of each tile, added in LDS in piece order ------------------------------
    if (p.kw > 1) {
        constexpr int kVals = kC * kRows;   // floats per lane
        if (w_k > 0) {
            float *dst = red + ((size_t)(w_k - 1) * p.tiles + w_tile) * kVals * 64 + lane;
#pragma unroll
            for (int j = 0; j < kC; ++j)
#pragma unroll
                for (int r = 0; r < kRows; ++r) dst[(j * kRows + r) * 64] = tot[j][r];
        }
        __syncthreads();
        if (w_k == 0) {
            for (int k = 1; k < p.kw; ++k) {
                const float *src = red + ((size_t)(k - 1) * p.tiles + w_tile) * kVals * 64 + lane;
#pragma unroll
                for (int j = 0; j < kC; ++j)
#pragma unroll
                    for (int r = 0; r < kRows; ++r) tot[j][r] += src[(j * kRows + r) * 64];
            }
        }
    }

    // ---- 7. the tile's sums: add the word rows (GEMV), undo the activation rescale -------------
    if constexpr (!kMfma) {
#pragma unroll
        for (int j = 0; j < kC; ++j) {
            float v = tot[j][0];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            tot[j][0] = v;
        }
    }
    const int row_base = kMfma ? 4 * rl : 0;
    const bool holder = (kMfma || rl == 0) && col_ok && w_k == 0;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int m = row_base + r;
        const int sh = m < M ? act_shift(rowmax[m] >> 7) : 0;
#pragma unroll
        for (int j = 0; j < kC; ++j) tot[j][r] = __builtin_amdgcn_ldexpf(tot[j][r], sh);
    }

    auto store_out = [&](int m, int v, float x0, float x1, float x2, float x3) {
        const size_t o = (size_t)m * N + n0 + 4 * v;
        if (p.out_bf16) {
            uint2 q;
            q.x = float_to_bf16_bits(x0) | (float_to_bf16_bits(x1) << 16);
            q.y = float_to_bf16_bits(x2) | (float_to_bf16_bits(x3) << 16);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + o) = q;
        } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o) = make_float4(x0, x1, x2, x3);
        }
    };

    // Fused pick of the k best columns per row (the output layer's greedy pick is k = 1), in this
    // launch: the column group's finished fp32 outputs go to LDS (over the fragments, no longer
    // read); one wave per row takes the group's k best keys (the keys of argmax_rows_kernel: larger
    // value first, then lower column; NaN never) and stores them to the group's slot with the
    // agent-scope coherence bit; the workgroup waits until its stores have completed and counts
    // itself in. The last group to count in merges every group's keys per row into the call's k
    // picks and lowers the counter again (zero between calls). Called by every thread of the
    // workgroup that finished the column group.
    const int KP = p.topk;
    float *vals = reinterpret_cast<float *>(smem + p.a_off);   // [M][WC] finished outputs
    auto stage = [&](int r, int j, float v) {                   // a holder's finished output
        vals[(size_t)(row_base + r) * WC + lcol + j] = v;
    };
    auto pick = [&]() {
        __syncthreads();   // every output of the group is in LDS
        constexpr int kPer = 2 * kC;   // keys per lane: WC / 64, at most 8 tiles of 16 * kC columns
        for (int m = wave; m < M; m += NW) {
            unsigned long long kk[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int c = lane + 64 * i;
                const float v = c < WC ? vals[(size_t)m * WC + c] : 0.f;
                kk[i] = c < WC && c0 + c < N && v == v ? argmax_key(v, (uint32_t)(c0 + c)) : 0ull;
            }
            for (int r = 0; r < KP; ++r) {
                unsigned long long best = 0ull;
#pragma unroll
                for (int i = 0; i < kPer; ++i) best = kk[i] > best ? kk[i] : best;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) {
                    const unsigned long long other = shfl_xor_u64(best, o);
                    best = other > best ? other : best;
                }
#pragma unroll
                for (int i = 0; i < kPer; ++i)   // keys are distinct (they hold the column): one lane drops it
                    if (kk[i] == best) kk[i] = 0ull;
                if (lane == 0)
                    __hip_atomic_store(&p.pick_slots[((size_t)m * p.groups + cg) * KP + r], best, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        wait_vm_all();     // this thread's slot stores have completed ...
        __syncthreads();   // ... and so have every other thread's
        if (tid == 0)
            s_pick_last = __hip_atomic_fetch_add(p.pick_counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                          (uint32_t)(p.groups - 1);
        __syncthreads();
        if (!s_pick_last) return;
        // the last group merges the rows, min(M, waves) at a time, each row on waves / that many
        // waves: each lane keeps the KP best of its share of the row's groups x KP keys (contiguous
        // in the slots), sorted; each wave takes its KP best in KP rounds of the wave's largest
        // head, and the row's first wave the KP best of its waves'
        const int cand = p.groups * KP;
        unsigned long long *wbest = reinterpret_cast<unsigned long long *>(vals);   // [NW][KP], over the outputs
        const int rows_at_once = M < NW ? M : NW;
        const int wpr = NW / rows_at_once;    // waves per row
        const int part = wave % wpr;          // the wave's share of its row
        unsigned long long top[kDecMaxTopK];
        auto insert = [&](unsigned long long x) {   // x sinks to its place; the smallest falls off
#pragma unroll
            for (int j = 0; j < kDecMaxTopK; ++j) {
                if (j < KP && x > top[j]) {
                    const unsigned long long t = top[j];
                    top[j] = x;
                    x = t;
                }
            }
        };
        auto wave_take = [&](auto &&emit) {   // KP rounds of the wave's largest head
            for (int r = 0; r < KP; ++r) {
                unsigned long long best = top[0];
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) {
                    const unsigned long long other = shfl_xor_u64(best, o);
                    best = other > best ? other : best;
                }
                if (best != 0ull && top[0] == best) {   // the lane holding it moves to its next
#pragma unroll
                    for (int j = 0; j + 1 < kDecMaxTopK; ++j) top[j] = top[j + 1];
                    top[kDecMaxTopK - 1] = 0ull;
                }
                emit(r, best);
            }
        };
        for (int m0 = 0; m0 < M; m0 += rows_at_once) {
            const int m = m0 + wave / wpr;
            const bool mine = wave / wpr < rows_at_once && m < M;   // wave-uniform
#pragma unroll
            for (int j = 0; j < kDecMaxTopK; ++j) top[j] = 0ull;
            if (mine) {
                const unsigned long long *row = p.pick_slots + (size_t)m * cand;
                constexpr int kB = 8;   // loads in flight per lane
                const int stride = wpr * 64;
                for (int i0 = part * 64 + lane; i0 < cand; i0 += stride * kB) {
                    unsigned long long x[kB];
#pragma unroll
                    for (int b = 0; b < kB; ++b) {
                        const int i = i0 + stride * b;
                        x[b] = i < cand ? __hip_atomic_load(row + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
                    }
#pragma unroll
                    for (int b = 0; b < kB; ++b) insert(x[b]);
                }
                wave_take([&](int r, unsigned long long best) {
                    if (lane == 0) wbest[wave * KP + r] = best;
                });
            }
            __syncthreads();
            if (mine && part == 0) {
#pragma unroll
                for (int j = 0; j < kDecMaxTopK; ++j) top[j] = 0ull;
                for (int i = lane; i < wpr * KP; i += 64) insert(wbest[wave * KP + i]);
                wave_take([&](int r, unsigned long long best) {
                    if (lane == 0)
                        p.pick_idx[(size_t)m * KP + r] = best ? (int32_t)(0xFFFFFFFFu - (uint32_t)best) : p.pick_none;
                });
            }
            __syncthreads();   // wbest is read before the next rows reuse it
        }
        if (tid == 0) __hip_atomic_store(p.pick_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    if (P == 1) {
        if (holder) {
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const int m = row_base + r;
                if (m < M) {
#pragma unroll
                    for (int v = 0; v < kV; ++v)
                        store_out(m, v, tot[4 * v][r], tot[4 * v + 1][r], tot[4 * v + 2][r], tot[4 * v + 3][r]);
                }
            }
        }
        if (KP > 0) {
            __syncthreads();   // every wave is past the main loop: the fragments are no longer read
            if (holder) {
#pragma unroll
                for (int r = 0; r < kRows; ++r)
                    if (row_base + r < M) {
#pragma unroll
                        for (int j = 0; j < kC; ++j) stage(r, j, tot[j][r]);
                    }
            }
            pick();
        }
        return;
    }

    // ---- 8. slices across workgroups ----------------------------------------------------------
    // Every workgroup of the column group counted itself in when it started; the last one to
    // start adds the slices. The others store their slice (16-byte stores with the agent-scope
    // coherence bit), wait until every store of the workgroup has completed, and raise their
    // slice's flag. The reducer waits for each other slice's flag, reads the slices, adds them in
    // slice order (bit-identical results from run to run), and lowers the flags and the counter
    // again: counters and flags are zero between calls, so no state carries from one call to
    // the next and a replayed graph runs as it ran when it was captured.
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(p.partials, p.part_bytes);
    uint32_t *const flags = p.flags + (size_t)cg * P;
    if (tid == 0) {
        s_last = arrival == (uint32_t)(P - 1);
        s_failed = 0;
    }
    __syncthreads();
    if (!s_last) {
        if (holder) {
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const int m = row_base + r;
                if (m < M) {
#pragma unroll
                    for (int v = 0; v < kV; ++v) {
                        const f32x4 x = f32x4{tot[4 * v][r], tot[4 * v + 1][r], tot[4 * v + 2][r], tot[4 * v + 3][r]};
                        const uint32_t off = (uint32_t)((((size_t)sl * M + m) * N + n0 + 4 * v) * sizeof(float));
                        __builtin_amdgcn_raw_buffer_store_b128(x, prs, (int)off, 0, kCoherent);
                    }
                }
            }
        }
        wait_vm_all();     // this thread's stores have completed ...
        __syncthreads();   // ... and so have every other thread's
        if (tid == 0) __hip_atomic_store(&flags[sl], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    for (int sp = tid; sp < P; sp += T) {
        if (sp == sl) continue;
        uint32_t spins = 0;
        while (__hip_atomic_load(&flags[sp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins == kSpinLimit) {   // cannot happen while every workgroup runs to its end
                s_failed = 1;
                break;
            }
        }
    }
    __syncthreads();   // every flag seen raised: the other slices' stores have completed
    const bool failed = s_failed != 0;
    // Each output adds the slices in slice order. The loads of a batch of slices for all of the
    // lane's rows are in flight together (one round trip per batch, not one per row: a slice
    // read from another die's stores takes about half a microsecond to arrive).
    constexpr int kOut = kRows * kV;                      // float4 outputs per lane
    constexpr int kBatch = kOut >= 8 ? 1 : 8 / kOut;      // slices per batch: at most 8 loads in flight
    if (holder) {
        f32x4 sum[kOut];
#pragma unroll
        for (int o = 0; o < kOut; ++o) sum[o] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int b = 0; b < P; b += kBatch) {   // slices in order
            f32x4 x[kBatch][kOut];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
#pragma unroll
                for (int o = 0; o < kOut; ++o) {
                    const int r = o / kV, v = o - (o / kV) * kV;
                    const int sp = b + i, m = row_base + r;
                    x[i][o] = f32x4{tot[4 * v][r], tot[4 * v + 1][r], tot[4 * v + 2][r], tot[4 * v + 3][r]};
                    if (sp < P && sp != sl && m < M) {
                        const uint32_t off = (uint32_t)((((size_t)sp * M + m) * N + n0 + 4 * v) * sizeof(float));
                        x[i][o] = __builtin_amdgcn_raw_buffer_load_b128(prs, (int)off, 0, kCoherent);
                    }
                }
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
#pragma unroll
                for (int o = 0; o < kOut; ++o)
                    if (b + i < P) sum[o] += x[i][o];
        }
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int m = row_base + r;
            if (m >= M) continue;
#pragma unroll
            for (int v = 0; v < kV; ++v) {
                f32x4 sm = sum[r * kV + v];
                if (failed) sm = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
                const f32x4 sum = sm;
                store_out(m, v, sum.x, sum.y, sum.z, sum.w);
                if (KP > 0) {   // every wave is past the main loop (the flag wait ended in a barrier)
                    stage(r, 4 * v, sum.x);
                    stage(r, 4 * v + 1, sum.y);
                    stage(r, 4 * v + 2, sum.z);
                    stage(r, 4 * v + 3, sum.w);
                }
            }
        }
    }
    if (KP > 0) pick();
    for (int sp = tid; sp < P; sp += T)
        if (sp != sl) __hip_atomic_store(&flags[sp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) __hip_atomic_store(&p.counters[cg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool kMfma, int kZM, int kU, int kV, int kLd = kV, int kBits = 4, int kSub = 1>
hipError_t launch_one(const DecodeArgs &a, const DecodePlan &plan, hipStream_t stream)
{
    const auto kern = decode_kernel<kMfma, kZM, kU, kV, kLd, kBits, kSub>;
    if (plan.lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.groups * a.slices)), dim3(a.tiles * a.kw * 64), plan.lds, stream, a);
    return hipGetLastError();
}

template <bool kMfma, int kZM>
hipError_t launch_ring(const DecodeArgs &a, const DecodePlan &plan, hipStream_t stream)
{
    if (plan.cols == 8) {
        switch (plan.ring) {
        case 2: return launch_one<kMfma, kZM, 2, 2>(a, plan, stream);
        case 4: return launch_one<kMfma, kZM, 4, 2>(a, plan, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (plan.ring) {
    case 2: return launch_one<kMfma, kZM, 2, 1>(a, plan, stream);
    case 3: return launch_one<kMfma, kZM, 3, 1>(a, plan, stream);
    case 4: return launch_one<kMfma, kZM, 4, 1>(a, plan, stream);
    case 6: return launch_one<kMfma, kZM, 6, 1>(a, plan, stream);
    case 8: return launch_one<kMfma, kZM, 8, 1>(a, plan, stream);
    default: return hipErrorInvalidValue;
    }
}

// affine codes: 64-column tiles, a ring of 4 steps, one instance per code width
template <bool kMfma>
hipError_t launch_affine(const DecodeArgs &a, const DecodePlan &plan, hipStream_t stream)
{
    if (plan.ring != 4) return hipErrorInvalidValue;
    switch (a.bits) {
    case 1: return plan.sub == 4 ? launch_one<kMfma, kAffine, 4, 1, 1, 1, 4>(a, plan, stream)
                                 : launch_one<kMfma, kAffine, 4, 1, 1, 1>(a, plan, stream);
    case 2: return plan.sub == 2 ? launch_one<kMfma, kAffine, 4, 1, 1, 2, 2>(a, plan, stream)
                                 : launch_one<kMfma, kAffine, 4, 1, 1, 2>(a, plan, stream);
    case 3: return launch_one<kMfma, kAffine, 4, 1, 2, 3>(a, plan, stream);
    case 4: return launch_one<kMfma, kAffine, 4, 1, 1, 4>(a, plan, stream);
    case 5: return launch_one<kMfma, kAffine, 4, 1, 2, 5>(a, plan, stream);
    case 6: return launch_one<kMfma, kAffine, 4, 1, 2, 6>(a, plan, stream);
    case 8: return launch_one<kMfma, kAffine, 4, 1, 2, 8>(a, plan, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, const DecodePlan &plan, hipStream_t stream)
{
    if (a.biases) return plan.mfma ? launch_affine<true>(a, plan, stream) : launch_affine<false>(a, plan, stream);
    if (a.qzeros)
        return plan.mfma ? launch_ring<true, kZeroPacked>(a, plan, stream) : launch_ring<false, kZeroPacked>(a, plan, stream);
    return plan.mfma ? launch_ring<true, kZeroSym>(a, plan, stream) : launch_ring<false, kZeroSym>(a, plan, stream);
}

}  // namespace w4a16
