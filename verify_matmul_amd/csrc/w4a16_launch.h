// Host-side interface between the C ABI (w4a16_api.hip) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// Columns covered by one GEMM/GEMV workgroup (4 waves x 64 columns).
constexpr int kTileN = 256;
// K rows consumed per step (4 packed word rows = one 16x16x32 MFMA K step).
constexpr int kStepK = 32;
// Largest dynamic LDS a GEMM workgroup may ask for.
constexpr int kMaxLds = 64 * 1024 - 256;   // leaves room for the static LDS
// LDS bytes before the staged activations (per-row shifts).
constexpr int kLdsHeader = 64;

struct GemmArgs {
    const uint16_t *A;
    const uint32_t *qweight;
    const uint16_t *scales;
    const uint32_t *qzeros;   // nullptr: symmetric zero point 8
    void *out;
    float *partials;          // [splits, M, N] when splits > 1
    uint32_t *counters;       // one per column tile, zero between calls
    int M, N, K, g;
    int splits;
    int out_bf16;
};

// LDS bytes a GEMM workgroup needs for the given rows and split.
inline size_t gemm_lds_bytes(int M, int K, int splits)
{
    const int steps = K / kStepK;
    const int max_steps = (steps + splits - 1) / splits;
    return (size_t)kLdsHeader + (size_t)max_steps * 4 * (size_t)M * 16;
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream);

struct ArgmaxArgs {
    const float *logits;
    int32_t *idx;
    unsigned long long *keys;   // [M], zero between calls
    uint32_t *counters;         // [M], zero between calls
    int M, N;
    int chunks;                 // workgroups per row
};

constexpr int kArgmaxChunk = 16384;   // logits per argmax workgroup

hipError_t launch_argmax(const ArgmaxArgs &a, hipStream_t stream);
hipError_t launch_unpack_u8(const uint32_t *qweight, int K, int N, uint8_t *q, hipStream_t s);
hipError_t launch_dequant_f32(const uint32_t *qweight, const uint16_t *scales,
                              const uint32_t *qzeros, int g, int K, int N, float *w,
                              hipStream_t s);

}  // namespace w4a16
