// Device-side code readers shared by every W4A16 kernel (gfx950).
//
// One header holds the unpack and dequantisation so the GEMV, the MFMA GEMM and the test hooks
// cannot drift apart (TensorFold PR #859 keeps its code readers in one header shared by its
// GEMV and GEMM for the same reason).
//
// Exact dequantisation in fp16. The pages keep the dequantisation exact, (q - z) * scale
// (GRIMOIRE v1.7 release notes, 'What changed'). d = q - z is an integer in [-15, 15], exact in
// fp16, so the kernels build d directly as packed fp16 pairs with two VALU operations per pair:
//   (word & 0x000F000F) | 0x64006400  ->  fp16 pair (1024 + q_j, 1024 + q_{j+4})
//   (word & 0x00F000F0) | 0x54005400  ->  fp16 pair (  64 + q_j,   64 + q_{j+4})
// (0x6400 is 1024 with a unit of 1 in the low fraction bits, 0x5400 is 64 with a unit of 1/16,
// so a nibble sitting at bit 4 still reads as q), and one v_pk_add_f16 with the packed
// constant -(1024 + z) or -(64 + z) leaves q - z exactly in both halves. The scale is applied
// once per group to fp32 sums, so the product d * scale never rounds before accumulation.
//
// A word of column n holds rows 8i..8i+7; the dequantised pairs come out in the slot order
//   slot:  0   1   2   3   4   5   6   7
//   row :  k0  k4  k1  k5  k2  k6  k3  k7      (relative to 8i)
// Activations are staged in the same slot order so that slot t of A meets slot t of B in the
// dot products and in the MFMA K dimension.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t as_half2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ __forceinline__ uint32_t as_u32(half2_t x) { return __builtin_bit_cast(uint32_t, x); }

// Packed fp16 constants that subtract the zero point from the two magic encodings.
struct ZeroSub {
    uint32_t even;  // -(1024 + z) in both halves, for nibbles read at bit 0 of a half
    uint32_t odd;   // -(64 + z) in both halves, for nibbles read at bit 4 of a half
};

__device__ __forceinline__ ZeroSub zero_sub(uint32_t z)
{
    const uint32_t e = 0xE400u | z;          // fp16 -(1024 + z)
    const uint32_t o = 0xD400u | (z << 4);   // fp16 -(64 + z)
    return ZeroSub{e | (e << 16), o | (o << 16)};
}

// The symmetric zero point 8.
__device__ __forceinline__ ZeroSub zero_sub_sym() { return ZeroSub{0xE408E408u, 0xD480D480u}; }

// Nibble masks kept in VGPRs so the and/or pair fuses into one v_and_or_b32 (gfx950's VOP3 has
// no literal operand, and two SGPR sources would break the constant-bus limit).
struct Masks {
    uint32_t lo, hi;
};

__device__ __forceinline__ Masks make_masks()
{
    Masks m{0x000F000Fu, 0x00F000F0u};
    asm volatile("" : "+v"(m.lo), "+v"(m.hi));
    return m;
}

// One packed word -> 8 exact fp16 values (q - z) in slot order.
__device__ __forceinline__ half8_t dequant_word(uint32_t w, ZeroSub zs, Masks mk)
{
    const uint32_t h = w >> 8;
    const half2_t p0 = as_half2((w & mk.lo) | 0x64006400u) + as_half2(zs.even);   // k0, k4
    const half2_t p1 = as_half2((w & mk.hi) | 0x54005400u) + as_half2(zs.odd);    // k1, k5
    const half2_t p2 = as_half2((h & mk.lo) | 0x64006400u) + as_half2(zs.even);   // k2, k6
    const half2_t p3 = as_half2((h & mk.hi) | 0x54005400u) + as_half2(zs.odd);    // k3, k7
    half8_t r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// Zero point of column n from its packed word (nibble n % 8).
__device__ __forceinline__ uint32_t zero_of(uint32_t zword, uint32_t n)
{
    return (zword >> (4u * (n & 7u))) & 0xFu;
}

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// bf16 bits -> fp32 (exact: bf16 is the upper half of a binary32).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits)
{
    return __builtin_bit_cast(float, bits << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Per-row rescale of activations into fp16. With e_max the largest bf16 exponent field of the
// row's slice, the slice is multiplied by 2^-shift with shift = e_max - 141 so that every
// magnitude lands below 2^15 (fp16 tops out at 65504). A bf16 value keeps all 8 significant
// bits in fp16 as long as it stays above 2^-17 after the rescale, i.e. within 2^31 of the
// slice's largest magnitude; the rescale itself is exact. The shift is kept >= -126 so that
// 2^-shift stays a finite fp32 (that only affects rows whose largest magnitude is below 2^-112).
__device__ __forceinline__ int act_shift(uint32_t e_max)
{
    const int s = (int)e_max - 141;
    return s < -126 ? -126 : s;
}

// 8 bf16 activations of one word's rows (k order: raw.x = k0,k1 ... raw.w = k6,k7) -> fp16 in
// slot order, times `mul` (= 2^-shift, so the product is exact). The fp32 -> fp16 step rounds
// toward zero; it is exact for every value inside fp16's range, which the rescale guarantees
// for all but the smallest magnitudes of a row.
__device__ __forceinline__ half8_t act8_to_slots(uint4 raw, float mul)
{
    const float k0 = bf16_bits_to_float(raw.x & 0xFFFFu) * mul, k1 = __builtin_bit_cast(float, raw.x & 0xFFFF0000u) * mul;
    const float k2 = bf16_bits_to_float(raw.y & 0xFFFFu) * mul, k3 = __builtin_bit_cast(float, raw.y & 0xFFFF0000u) * mul;
    const float k4 = bf16_bits_to_float(raw.z & 0xFFFFu) * mul, k5 = __builtin_bit_cast(float, raw.z & 0xFFFF0000u) * mul;
    const float k6 = bf16_bits_to_float(raw.w & 0xFFFFu) * mul, k7 = __builtin_bit_cast(float, raw.w & 0xFFFF0000u) * mul;
    const half2_t p0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(k0, k4));
    const half2_t p1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(k1, k5));
    const half2_t p2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(k2, k6));
    const half2_t p3 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(k3, k7));
    half8_t r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// ---- memory helpers shared by the kernels --------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt encoding (gfx9): wait until at most `n` vector memory operations are outstanding.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Direct global->LDS loads: lane i's 16 (or 4) bytes land at lds_base + 16 i (4 i). They are
// written as inline assembly on purpose. Had the compiler seen these LDS writes, it would guard
// every LDS read that follows any later global load with a full vmcnt(0) wait -- one per
// iteration of the main loop, draining the weight ring. The kernel instead waits for them
// itself, once, with an explicit vmcnt before the staged data is first read. (Vector-memory
// operations the compiler cannot see only make its own wait counts stricter, never looser.)
__device__ __forceinline__ uint32_t lds_offset(void *lds_base)
{
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)(lds_base));
}

__device__ __forceinline__ void load_to_lds16(const void *src, void *lds_base)
{
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_offset(lds_base)) : "memory");
}

__device__ __forceinline__ void load_to_lds4(const void *src, void *lds_base)
{
    asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_offset(lds_base)) : "memory");
}

// The same loads from a base address held in scalar registers plus a 32-bit byte offset per lane
// (the instruction's scalar-base form). A loop that moves the base by the same amount in every
// lane then keeps that arithmetic off the vector unit. `base` must be equal in all lanes of the
// wave (it is computed from kernel arguments and wave-uniform values only). The optimiser's
// uniformity analysis is what places such a base in scalar registers; an unoptimised build (the
// host-sanitizer build compiles the device code at -O0) takes the full-address form instead.
__device__ __forceinline__ void load_to_lds16_s(const void *base, uint32_t off, void *lds_base)
{
#if defined(__OPTIMIZE__)
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_offset(lds_base)) : "memory");
#else
    load_to_lds16(static_cast<const unsigned char *>(base) + off, lds_base);
#endif
}

__device__ __forceinline__ void load_to_lds4_s(const void *base, uint32_t off, void *lds_base)
{
#if defined(__OPTIMIZE__)
    asm volatile("global_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_offset(lds_base)) : "memory");
#else
    load_to_lds4(static_cast<const unsigned char *>(base) + off, lds_base);
#endif
}

// SiLU, the gate of a gated feed-forward pair: x * logistic(x) = x / (1 + e^-x). Large
// negative x give e^-x = inf and a signed zero.
__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// 2^-shift as a float (shift within [-126, 114]).
__device__ __forceinline__ float pow2_neg(int shift) { return __builtin_amdgcn_ldexpf(1.0f, -shift); }

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

// Largest magnitude bits (sign cleared) of 8 bf16 values, in packed 16-bit halves. The largest
// magnitude has the largest exponent field: result >> 7 is the largest exponent field of the 8.
__device__ __forceinline__ uint32_t max_mag8(uint4 raw)
{
    const ushort2_t a = __builtin_bit_cast(ushort2_t, raw.x & 0x7FFF7FFFu);
    const ushort2_t b = __builtin_bit_cast(ushort2_t, raw.y & 0x7FFF7FFFu);
    const ushort2_t c = __builtin_bit_cast(ushort2_t, raw.z & 0x7FFF7FFFu);
    const ushort2_t d = __builtin_bit_cast(ushort2_t, raw.w & 0x7FFF7FFFu);
    const ushort2_t r = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    return max((uint32_t)r.x, (uint32_t)r.y);
}

// The same maximum kept packed (two 16-bit halves), folded into a running packed maximum.
__device__ __forceinline__ uint32_t max_mag8_packed(uint4 raw, uint32_t run)
{
    const ushort2_t a = __builtin_bit_cast(ushort2_t, raw.x & 0x7FFF7FFFu);
    const ushort2_t b = __builtin_bit_cast(ushort2_t, raw.y & 0x7FFF7FFFu);
    const ushort2_t c = __builtin_bit_cast(ushort2_t, raw.z & 0x7FFF7FFFu);
    const ushort2_t d = __builtin_bit_cast(ushort2_t, raw.w & 0x7FFF7FFFu);
    const ushort2_t r = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(r, __builtin_bit_cast(ushort2_t, run)));
}

// Greedy selection on the device, as lucebox PR #823 (PR description) does to avoid reading a
// whole vocabulary row back to the host. A (value, index) pair is packed into one 64-bit key
// whose unsigned order is "larger value first, then smaller index": the high word is the fp32
// bit pattern mapped to an unsigned total order (-0 folded onto +0), the low word is
// 0xFFFFFFFF - index. The maximum key over a row is therefore unique and independent of the
// order in which workgroups combine it, so the result is deterministic.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t n)
{
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;                       // -0 == +0
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - n);
}

// The largest of v over the wave's 64 lanes, in every lane: rotations within each row of 16
// lanes (DPP row_ror 8, 4, 2, 1; VALU operands, no LDS round trip as a lane shuffle takes), then
// the four rows' results read as scalars. Every lane must be active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m)
{
    const uint32_t lo = __shfl_xor((uint32_t)v, m);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((unsigned long long)hi << 32) | lo;
}

// Affine codes stored as column bit streams of kBits bits per row (MLX affine checkpoints,
// TensorFold PR #859, commit messages): a step of 32 rows is kBits word rows of a column, and
// the 8 rows of K quarter q start at bit 8 * kBits * q of the step, so they sit in one word for
// 1, 2 and 4 bits and in two consecutive words otherwise.
// The 8 codes of one column that a lane reads from an affine bit stream, as exact fp16 values q
// in the slot order of dequant_word (pairs (k0, k4), (k1, k5), (k2, k6), (k3, k7)). The lane's
// rows k0..k3 start at bit a_off of (w1:w0), rows k4..k7 at bit a_off4. Each pair is built in one
// word, a code in the low bits of each half, read as fp16 1024 + q and less 1024 (exact: q < 256).
template <int kBits>
__device__ __forceinline__ half8_t affine_codes(uint32_t w0, uint32_t w1, int a_off, int a_off4, Masks mk)
{
    if constexpr (kBits == 4) {   // the 4-bit stream is the GPTQ word layout: zero point 0
        return dequant_word(w0, zero_sub(0u), mk);
    }
    half2_t pr[4];
    const half2_t sub = as_half2(0xE400E400u);   // -1024 in both halves
    if constexpr (kBits == 8) {   // k0..k3: the bytes of w0, k4..k7: the bytes of w1
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + r) << 16) | (uint32_t)r;   // (w0 byte r, 0, w1 byte r, 0)
            pr[r] = as_half2(__builtin_amdgcn_perm(w1, w0, sel) | 0x64006400u) + sub;
        }
    } else if constexpr (kBits == 2) {
        // The 16 bits from a_off (0 or 16) are bytes (k0..k3) and (k4..k7): one byte permute puts
        // them in the two halves. Code r of each byte sits at bit 2r; read in place as the mantissa
        // of an fp16 whose unit is that bit (exponent 2^(10 - 2r)), it is 2^(10 - 2r) + q, so each
        // pair takes one and-or and one packed subtract, with no shift.
        const uint32_t y = __builtin_amdgcn_perm(0u, w0, 0x0C010C00u + 0x00020002u * ((uint32_t)a_off >> 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t magic = (uint32_t)(25 - 2 * r) << 10;   // fp16 2^(10 - 2r)
            pr[r] = as_half2((y & (0x00030003u << (2 * r))) | (magic * 0x10001u)) - as_half2(magic * 0x10001u);
        }
    } else if constexpr (kBits == 1) {
        // The byte at a_off (a multiple of 8) holds k0..k7 at bits 0..7; permuted into both halves,
        // pair r takes bit r of the low half and bit r + 4 of the high one, each read in place as
        // the mantissa of an fp16 whose unit is that bit.
        const uint32_t bsel = (uint32_t)a_off >> 3;
        const uint32_t y = __builtin_amdgcn_perm(0u, w0, 0x0C000C00u | (bsel << 16) | bsel);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t magic = ((uint32_t)(25 - r) << 10) | ((uint32_t)(21 - r) << 26);   // 2^(10 - r), 2^(6 - r)
            pr[r] = as_half2((y & ((1u << r) | (1u << (20 + r)))) | magic) - as_half2(magic);
        }
    } else {   // 3, 5 and 6 bits: two 32-bit windows of (w1:w0)
        const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, (uint32_t)a_off);
        const uint32_t hi = a_off4 >= 32 ? w1 >> (uint32_t)(a_off4 - 32) : __builtin_amdgcn_alignbit(w1, w0, (uint32_t)a_off4);
        constexpr uint32_t kMask2 = ((1u << kBits) - 1u) * 0x10001u;   // a code in both halves
        if constexpr (kBits <= 4) {   // k0..k3 in the low half of y, k4..k7 in the high half
            constexpr uint32_t kHalf = (1u << (4 * kBits)) - 1u;
            const uint32_t y = (lo & kHalf) | ((hi & kHalf) << 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) pr[r] = as_half2(((y >> (kBits * r)) & kMask2) | 0x64006400u) + sub;
        } else {                      // (k0, k1 | k4, k5) and (k2, k3 | k6, k7)
            constexpr uint32_t kHalf = (1u << (2 * kBits)) - 1u;
            const uint32_t y0 = (lo & kHalf) | ((hi & kHalf) << 16);
            const uint32_t y1 = ((lo >> (2 * kBits)) & kHalf) | (((hi >> (2 * kBits)) & kHalf) << 16);
            pr[0] = as_half2((y0 & kMask2) | 0x64006400u) + sub;
            pr[1] = as_half2(((y0 >> kBits) & kMask2) | 0x64006400u) + sub;
            pr[2] = as_half2((y1 & kMask2) | 0x64006400u) + sub;
            pr[3] = as_half2(((y1 >> kBits) & kMask2) | 0x64006400u) + sub;
        }
    }
    half8_t b;
    b[0] = pr[0][0]; b[1] = pr[0][1]; b[2] = pr[1][0]; b[3] = pr[1][1];
    b[4] = pr[2][0]; b[5] = pr[2][1]; b[6] = pr[3][0]; b[7] = pr[3][1];
    return b;
}

}  // namespace w4a16
