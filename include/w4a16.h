/*
 * w4a16.h -- C ABI of libw4a16.so: group-quantised int4-weight x bf16-activation matmul for
 * LLM decode on AMD Instinct MI355X (gfx950).
 *
 *   out[M, N] = A[M, K] x W[K, N],   W[k][n] = (q[k][n] - z[k/g][n]) * scale[k/g][n]
 *
 * The operation is the int4 path of the GRIMOIRE v1.7 release notes ('What changed'): int4
 * weights and bf16 activations, an exact (q - z) * scale dequantisation, one kernel for a
 * single decoding row (M = 1) and a matrix-core kernel for the 2-16 rows that several users
 * or a speculative verify pass produce. GRIMOIRE v1.8 ('What changed') checks its 1 + 4
 * drafted MTP rows through that small-M path and scores the output layer in one pass; the
 * 248k-row output layer of strix-llama.cpp PR #105 is such a call. lucebox PR #823 moves the
 * greedy pick over a vocabulary row onto the GPU (w4a16_argmax_rows).
 *
 * Storage (the GPTQ convention):
 *   qweight  uint32 [K/8, N]    nibble j (bits 4j..4j+3) of word [i][n] is the code of row 8i+j
 *   scales   fp16   [K/g, N]    IEEE binary16 bit patterns
 *   qzeros   uint32 [K/g, N/8]  nibble j of word [gi][c] is the zero point of column 8c+j, used
 *                               as stored (no +1 offset); NULL means every zero point is 8
 *   A        bf16   [M, K]      row-major
 *   out      fp32 or bf16 [M, N] row-major, fully overwritten
 * All tensors are dense with the row strides implied by their shapes.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers (memory the caller owns; the library never frees or keeps
 *     them). Calls are asynchronous on `stream` (0 = the null stream); results are valid once
 *     the stream has reached the call. Inputs and outputs must not overlap.
 *   - Arguments are checked on the host before any device work; a non-OK status means no
 *     device work was enqueued. The library never aborts and never prints: w4a16_last_error()
 *     returns a description of the last non-OK status of the calling thread.
 *   - The library owns one scratch buffer per (device, stream) for tile counters and slice
 *     flags, split-K partial sums, prepared activations and the fused pick's row keys. It is
 *     allocated (with hipMalloc, then set up by small kernels on the stream) on the first call
 *     that needs it on that stream; a later call that needs more gets a new, larger buffer and
 *     the old one is kept until w4a16_release_scratch (a graph captured earlier may still use
 *     it). Every call leaves the counters, flags and keys zero and the small-row kernel's
 *     split-K exchange empty, and writes its other data before it reads it, so no state carries
 *     from one call to the next: calls may be captured into a HIP graph and
 *     replayed any number of times. A call that would have to allocate while its stream is
 *     being captured returns W4A16_ERR_UNSUPPORTED instead, so run the same calls on the stream
 *     once before capturing it (that also keeps allocation out of timed regions). Calls on
 *     different streams never share scratch; calls on one stream are ordered, and calls that
 *     run concurrently on one stream's scratch (e.g. two graphs captured from one stream and
 *     replayed at once on different streams) are not supported.
 *   - Results are deterministic: the same inputs and launch give bit-identical outputs (the
 *     split-K partials are summed in a fixed order, never with float atomics).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = -1,   /* null pointer, size or divisibility violation, bad dtype */
    W4A16_ERR_UNSUPPORTED = -2,   /* pointer not 16-byte aligned, qweight of 2^32 words or more, or
                                     scratch needed while the stream is being captured */
    W4A16_ERR_HIP = -3,           /* a HIP runtime call failed; see w4a16_last_error() */
    W4A16_ERR_NO_MEMORY = -4      /* the scratch buffer could not be allocated */
} w4a16_status;

typedef enum { W4A16_OUT_F32 = 0, W4A16_OUT_BF16 = 1 } w4a16_out_dtype;

/*
 * out = A x dequant(qweight, scales, qzeros).
 *   A         bf16 [M, K], 16-byte aligned
 *   qweight   uint32 [K/8, N], 16-byte aligned, fewer than 2^32 words (16 GiB)
 *   scales    fp16 bits [K/g, N], 16-byte aligned
 *   qzeros    uint32 [K/g, N/8], 16-byte aligned, or NULL for the symmetric zero point 8
 *   group_size g: a positive multiple of 32 that divides K
 *   M in 1..16; N > 0 and a multiple of 8; K > 0 and a multiple of g
 *   out       [M, N] fp32 (out_dtype W4A16_OUT_F32) or bf16 (W4A16_OUT_BF16, round to
 *             nearest even), 16-byte aligned
 * On matrices of fewer than 65536 columns, M = 1 on 64-column tiles runs the single-row GEMV and
 * everything else (M = 2..16, and M = 1 on the 128-column tiles of matrices with N >= 32768) the
 * matrix-core GEMM; wider matrices run the decode kernel of w4a16_gemm_decode_ex (its GEMV at one
 * row, its matrix-core GEMM beyond), with its default launch. Accuracy: every output
 * is within 4e-3 * sum_k |a_k * w_kn| + 1e-6 of the exact value for finite inputs whose
 * nonzero activations within one row span less than 2^30 in magnitude (activations enter the
 * fp16 matrix cores through an exact power-of-two rescale per row and K-slice).
 */
int w4a16_gemm(const void *A, const uint32_t *qweight, const uint16_t *scales,
               const uint32_t *qzeros, int group_size, int M, int N, int K,
               void *out, int out_dtype, hipStream_t stream);

/*
 * w4a16_gemm for callers that cannot allocate device memory: code being captured into a HIP graph
 * on a stream that has not been warmed up, tight serving loops, and harnesses that forbid
 * hipMalloc. Same operation, arguments, accuracy contract and determinism as w4a16_gemm; it calls
 * no hipMalloc, hipFree or allocating routine. Its scratch is one fixed 16 MiB array in device
 * memory per GPU (1 MiB of counters and flags, 6 MiB of split-K exchange, 9 MiB of partial sums
 * and prepared activations), held until the process ends; its first call on a device takes the
 * array's address and sets up the counters and the exchange with small kernels on `stream`. A
 * launch whose scratch would not fit takes fewer split-K workgroups per column tile (or, on
 * matrices of 65536 columns or more, fewer K slices) so its rounding may differ from
 * w4a16_gemm's, within the same contract; if even one does not fit (or the K slice then no
 * longer fits in LDS), W4A16_ERR_UNSUPPORTED. Every call on a GPU uses the same array and leaves
 * its counters and flags zero and its exchange empty: calls that overlap on one GPU (on
 * different streams, or graphs replayed concurrently) race and must not be made.
 */
int w4a16_gemm_noalloc(const void *A, const uint32_t *qweight, const uint16_t *scales,
                       const uint32_t *qzeros, int group_size, int M, int N, int K,
                       void *out, int out_dtype, hipStream_t stream);

/*
 * w4a16_gemm with an explicit launch: `splits` workgroups share each column tile along K
 * (their fp32 partials are added in slice order through the library's scratch buffer),
 * `waves_k` waves of each workgroup split that workgroup's K range (1, 2, 4, 8 or 16), and
 * `tile_cols` is the tile width (64 or 128 columns: 4 or 8 adjacent columns per lane). 0 picks
 * what w4a16_gemm picks for that knob. splits * waves_k must not exceed K/32. Every launch meets
 * the same accuracy contract and is deterministic; different launches round differently. Meant
 * for tests and tuning sweeps.
 */
int w4a16_gemm_ex(const void *A, const uint32_t *qweight, const uint16_t *scales,
                  const uint32_t *qzeros, int group_size, int M, int N, int K,
                  void *out, int out_dtype, int splits, int waves_k, int tile_cols,
                  hipStream_t stream);

/*
 * w4a16_gemm on the decode kernel with an explicit launch: a workgroup is `tiles` x `kw` waves
 * (at most 8), `tiles` adjacent column tiles of `tile_cols` columns (64 or 128) over one K slice,
 * each tile's slice split into `kw` pieces whose sums are added in LDS; `slices` workgroups (1..16)
 * split each group of columns along K (their fp32 sums are added in slice order through the
 * library's scratch buffer); slices * kw must not exceed K/32. `ring` is the number of 32-row steps
 * of packed weights each wave keeps in flight (2, 3, 4, 6 or 8 on 64-column tiles, 2 or 4 on
 * 128-column tiles). 0 picks the kernel's default for that knob. A launch whose activation slice
 * or scales would not fit in a workgroup's LDS is refused with W4A16_ERR_INVALID_ARG. Same
 * operation, arguments, accuracy contract (with the activations rescaled per row and K slice) and
 * determinism as w4a16_gemm.
 * topk, idx: 0 and NULL, or the fused pick of w4a16_gemm_topk (k = topk, idx int32 [M, topk]
 * device). Meant for tests and tuning sweeps.
 */
int w4a16_gemm_decode_ex(const void *A, const uint32_t *qweight, const uint16_t *scales,
                         const uint32_t *qzeros, int group_size, int M, int N, int K,
                         void *out, int out_dtype, int slices, int tiles, int kw, int tile_cols,
                         int ring, int topk, int32_t *idx, hipStream_t stream);

/* The decode kernel's launch for a shape and explicit knobs (0 = default), checked exactly as
 * w4a16_gemm_decode_ex checks it, without any device work: W4A16_OK and, if plan_out is not NULL,
 * plan_out[0..6] = slices, tiles, kw, tile_cols, ring, LDS bytes per workgroup, and the 32-row
 * K-steps per ring slot (1; or 2 and 4 for 2- and 1-bit affine codes whose groups hold whole
 * blocks of 64 and 128 rows, read a word per lane; slices and K pieces are then whole blocks);
 * or the status and w4a16_last_error() that w4a16_gemm_decode_ex would return. packed_zeros: nonzero for packed zero
 * points (qzeros given); topk: 0, or the k of a fused pick; affine_bits: 0 for GPTQ codes, or the
 * width of the affine codes of w4a16_gemm_affine_bits_ex. Host only. */
int w4a16_decode_plan(int M, int N, int K, int group_size, int packed_zeros, int slices, int tiles,
                      int kw, int tile_cols, int ring, int topk, int affine_bits, int *plan_out);

/* The launch w4a16_gemm picks for a shape (symmetric zero points): *kernel = 0 for the small-row
 * kernel's one-row GEMV, 1 for its MFMA GEMM, with *splits, *waves_k and *tile_cols as in
 * w4a16_gemm_ex; or 2 (one row) / 3 (matrix cores) for the decode kernel of w4a16_gemm_decode_ex,
 * which w4a16_gemm takes for matrices of 65536 columns or more (an output layer), with *splits =
 * its slices, *waves_k = its kw and *tile_cols. Any output pointer may be NULL. Host only. */
int w4a16_plan(int M, int N, int K, int group_size, int *kernel, int *splits, int *waves_k,
               int *tile_cols);

/*
 * w4a16_gemm and the greedy pick (the output layer): out as in w4a16_gemm, and idx[m] = smallest
 * n with out[m][n] (in fp32, before any bf16 rounding) equal to the row maximum, with the
 * conventions of w4a16_argmax_rows. The pick is made in the GEMM's epilogue from the values it
 * writes, so the logits are not read back. On matrices of 65536 columns or more the whole pick
 * runs inside the GEMM's launch (w4a16_gemm_topk with k = 1); on narrower ones each column tile
 * leaves its keys in the stream's scratch and a small kernel next on the stream reduces them.
 * idx: int32 [M] device.
 */
int w4a16_gemm_argmax(const void *A, const uint32_t *qweight, const uint16_t *scales,
                      const uint32_t *qzeros, int group_size, int M, int N, int K,
                      void *out, int out_dtype, int32_t *idx, hipStream_t stream);

/*
 * w4a16_gemm and the k best columns of each row in one launch (the output layer of a verify
 * pass): out as in w4a16_gemm, and idx[m][r] (int32 [M, k] device) = the column of row m's r-th
 * largest output, decided in fp32 before any bf16 rounding, largest first, equal values by lowest
 * column, -0 equal to +0, NaN never chosen, -1 once the row has no column left (k > N or NaN
 * outputs). idx[m][0] is the greedy pick of w4a16_gemm_argmax (which gives 0, not -1, for a row
 * with no number). The lucebox PR #823 description
 * moves the greedy choice over the vocabulary row onto the device; the k best extend that choice
 * to the next candidates in the same order. k in 1..8. Each group of columns keeps its k best per
 * row and the last group to finish merges them, inside the GEMM's launch: no logits read back, no
 * second launch. Runs on the decode kernel (w4a16_gemm_decode_ex's default launch for the shape),
 * whatever N. Uses the stream's scratch (a counter, and groups x M x k 64-bit keys). Deterministic.
 */
int w4a16_gemm_topk(const void *A, const uint32_t *qweight, const uint16_t *scales,
                    const uint32_t *qzeros, int group_size, int M, int N, int K,
                    void *out, int out_dtype, int k, int32_t *idx, hipStream_t stream);

/*
 * out[M,N] = A x W for many rows (prompt processing), on the matrix cores: the same operation,
 * storage layout and argument rules as w4a16_gemm, with M in 1..W4A16_PREFILL_MAX_M. The GRIMOIRE
 * v1.8 release notes ('What changed', INT4 prompt processing) run GPTQ int4 weights through a
 * fast prompt path; with hundreds of rows each weight feeds hundreds of multiply-adds and the
 * matrix cores, not HBM, set the pace. Each row of A is rescaled by one power of two over its
 * whole K before the fp16 matrix cores (exact; a bf16 value keeps all its bits when it lies
 * within 2^31 of its row's largest magnitude), so results match w4a16_gemm's accuracy
 * contract. Uses M * K * 2 + M * 4 bytes of the stream's scratch for the prepared activations,
 * and when the output has fewer 64 x 256 tiles than the device runs at once, up to
 * 16 * M * N * 4 more for fp32 sums of whole-group K slices, added in slice order (scratch is
 * allocated on the first call of a size on a stream). Deterministic. Meant for M well above 16;
 * any M works.
 */
#define W4A16_PREFILL_MAX_M 65536
int w4a16_gemm_prefill(const void *A, const uint32_t *qweight, const uint16_t *scales,
                       const uint32_t *qzeros, int group_size, int M, int N, int K,
                       void *out, int out_dtype, hipStream_t stream);

/*
 * Gated feed-forward input in one launch: two matrices of the same shape read against the same
 * activations, combined as
 *   out[m][n] = silu(g[m][n]) * u[m][n],   silu(x) = x / (1 + e^-x),
 *   g = A x dequant(qweight_gate, scales_gate, qzeros_gate), u = A x dequant(qweight_up, ...)
 * with g and u summed in fp32 exactly as w4a16_gemm sums them; silu and the product are
 * evaluated in fp32, a bf16 out is that fp32 value rounded to nearest even. The GRIMOIRE v1.8
 * release notes ('What changed', INT4 prompt processing) fuse the feed-forward gate into the
 * int4 path; the pages do not name the gate's nonlinearity, and SiLU is the gate of the
 * Qwen-family feed-forward they run. The activations are staged once for both matrices and
 * only [M, N] is written.
 * Every argument is as in w4a16_gemm, for each matrix; both matrices have the same N, K and
 * group size, and qzeros_gate and qzeros_up are both NULL (symmetric) or both given
 * (INVALID_ARG otherwise). out must not overlap any input.
 * The _ex form fixes the launch as w4a16_gemm_ex does (0 = default), on 128-column tiles of the
 * pair (64 output columns of each matrix): splits * waves_k must not exceed K/32.
 */
int w4a16_gemm_gate_up(const void *A, const uint32_t *qweight_gate, const uint16_t *scales_gate,
                       const uint32_t *qzeros_gate, const uint32_t *qweight_up,
                       const uint16_t *scales_up, const uint32_t *qzeros_up, int group_size,
                       int M, int N, int K, void *out, int out_dtype, hipStream_t stream);
int w4a16_gemm_gate_up_ex(const void *A, const uint32_t *qweight_gate, const uint16_t *scales_gate,
                          const uint32_t *qzeros_gate, const uint32_t *qweight_up,
                          const uint16_t *scales_up, const uint32_t *qzeros_up, int group_size,
                          int M, int N, int K, void *out, int out_dtype, int splits, int waves_k,
                          hipStream_t stream);

/*
 * The gated feed-forward input for many rows (prompt processing), on the matrix cores: the
 * operation and argument rules of w4a16_gemm_gate_up with M in 1..W4A16_PREFILL_MAX_M, computed
 * as w4a16_gemm_prefill computes a product (so g and u follow its accuracy contract), with
 * silu(g) * u formed before the single [M, N] store. This is where the GRIMOIRE v1.8 release
 * notes ('What changed', INT4 prompt processing) fuse the feed-forward gate. Scratch as
 * w4a16_gemm_prefill, the K-slice sums being 2N wide.
 */
int w4a16_gemm_gate_up_prefill(const void *A, const uint32_t *qweight_gate,
                               const uint16_t *scales_gate, const uint32_t *qzeros_gate,
                               const uint32_t *qweight_up, const uint16_t *scales_up,
                               const uint32_t *qzeros_up, int group_size, int M, int N, int K,
                               void *out, int out_dtype, hipStream_t stream);

/*
 * Affine codes (the MLX affine format of the checkpoints in TensorFold PR #859, commit messages):
 *
 *   out[M, N] = A[M, K] x W[K, N],   W[k][n] = scale[k/g][n] * q[k][n] + bias[k/g][n]
 *
 *   qweight  uint32 [K/8, N]    4-bit codes 0..15 in the qweight layout above (nibble j of word
 *                               [i][n] is row 8i+j); narrower codes are widened onto it first
 *                               (w4a16_affine_widen)
 *   scales   bf16   [K/g, N]    bit patterns
 *   biases   bf16   [K/g, N]    bit patterns
 * A, out, M (1..16), group_size, K, N, alignment, scratch and determinism as w4a16_gemm; there is
 * no zero point. The sum of a group is formed as scale * sum(a * q) + bias * sum(a), so the
 * accuracy contract is
 *   |out - exact| <= 4e-3 * sum_k |A[m][k]| * (|scale * q| + |bias|) + 1e-6.
 * w4a16_gemm_affine_ex takes the launch overrides of w4a16_gemm_ex (0 = the library's choice).
 */
int w4a16_gemm_affine(const void *A, const uint32_t *qweight, const uint16_t *scales,
                      const uint16_t *biases, int group_size, int M, int N, int K, void *out,
                      int out_dtype, hipStream_t stream);
int w4a16_gemm_affine_ex(const void *A, const uint32_t *qweight, const uint16_t *scales,
                         const uint16_t *biases, int group_size, int M, int N, int K, void *out,
                         int out_dtype, int splits, int waves_k, int tile_cols, hipStream_t stream);

/*
 * Affine codes read at their own width (TensorFold PR #859, commit messages: 2, 3, 5 and 6-bit
 * codes get tiles of their own width, 8-bit codes their own GEMV, so that a mostly 2-bit
 * checkpoint does not stream as many bytes as a 4-bit one):
 *
 *   out[M, N] = A[M, K] x W[K, N],   W[k][n] = scale[k/g][n] * q[k][n] + bias[k/g][n]
 *
 *   packed   uint32 [K*bits/32, N]  the codes as column bit streams, the input layout of
 *                                   w4a16_affine_widen (row k of column n at stream bits
 *                                   [k*bits, (k+1)*bits)); bits = 1, 2, 3, 4, 5, 6 or 8 (7-bit
 *                                   codes: w4a16_affine_split)
 *   scales, biases  bf16 [K/g, N]   bit patterns
 * Each call streams K*N*bits/8 bytes of codes: nothing is widened or split. A, out, M (1..16),
 * group_size, K, N, alignment, scratch, determinism and the accuracy contract as
 * w4a16_gemm_affine. Runs on the decode kernel (w4a16_gemm_decode_ex), whose code reader pulls
 * each lane's 8 codes out of one or two words of the stream. w4a16_gemm_affine_bits_ex takes
 * that kernel's launch knobs (0 = its default; 64-column tiles; ring 4).
 */
int w4a16_gemm_affine_bits(const void *A, const uint32_t *packed, int bits, const uint16_t *scales,
                           const uint16_t *biases, int group_size, int M, int N, int K, void *out,
                           int out_dtype, hipStream_t stream);
int w4a16_gemm_affine_bits_ex(const void *A, const uint32_t *packed, int bits,
                              const uint16_t *scales, const uint16_t *biases, int group_size,
                              int M, int N, int K, void *out, int out_dtype, int slices, int tiles,
                              int kw, int ring, hipStream_t stream);

/*
 * The same product for many rows (prompt processing), on the prompt GEMM of w4a16_gemm_prefill
 * (TensorFold PR #859, PR description: a prompt GEMM for the affine codes beside their GEMV):
 * packed, bits, scales and biases as w4a16_gemm_affine_bits, each code read at its own width;
 * A, out, M (1..W4A16_PREFILL_MAX_M), the per-row rescale of A, scratch and determinism as
 * w4a16_gemm_prefill; the accuracy contract of w4a16_gemm_affine. Every group adds
 * scale * sum(a q) + bias * sum(a) in fp32, sum(a) taken on the matrix cores from the same fp16
 * activations. Errors as w4a16_gemm_affine_bits (bits outside 1..6 and 8, a missing bias
 * pointer, codes beyond 2^32 words), then as w4a16_gemm_prefill.
 */
int w4a16_gemm_affine_bits_prefill(const void *A, const uint32_t *packed, int bits,
                                   const uint16_t *scales, const uint16_t *biases, int group_size,
                                   int M, int N, int K, void *out, int out_dtype,
                                   hipStream_t stream);

/*
 * The gated feed-forward input of two affine matrices, out = silu(A x W_gate) * (A x W_up), each W
 * = scale * q + bias as in w4a16_gemm_affine (4-bit codes, bf16 scales and biases, same shape):
 * the operation, launch and scratch of w4a16_gemm_gate_up, each product under w4a16_gemm_affine's
 * accuracy contract (carried through silu and the product as for w4a16_gemm_gate_up).
 */
int w4a16_gemm_affine_gate_up(const void *A, const uint32_t *qweight_gate,
                              const uint16_t *scales_gate, const uint16_t *biases_gate,
                              const uint32_t *qweight_up, const uint16_t *scales_up,
                              const uint16_t *biases_up, int group_size, int M, int N, int K,
                              void *out, int out_dtype, hipStream_t stream);

/*
 * Codes of `bits` = 1..4 bits rewritten as the 4-bit codes w4a16_gemm_affine reads, each keeping
 * its value (scales and biases are unchanged), as TensorFold PR #859 first ran 2 and 3-bit
 * checkpoints on its 4-bit tiles. Input layout: for column n the codes of rows 0, 1, 2, ... form
 * one little-endian bit stream, row k at stream bits [k*bits, (k+1)*bits), and stream bit i is bit
 * i % 32 of word [i/32][n] of packed (uint32 [K*bits/32, N]); at bits = 4 this is the qweight
 * layout itself. Output qweight uint32 [K/8, N]. K % 32 == 0, N % 8 == 0, both 16-byte aligned,
 * not overlapping. Bit-exact integer work; no scratch.
 */
int w4a16_affine_widen(const uint32_t *packed, int bits, int K, int N, uint32_t *qweight,
                       hipStream_t stream);

/*
 * Codes of 5..8 bits (TensorFold PR #859, commit messages: MLX checkpoints of 5 to 8 bits, each
 * code keeping its value, scale and bias). Every code splits exactly into two 4-bit codes,
 * q = 16 * hi + lo, so w = s * q + b = (s * lo + b) + (16 s) * hi.
 *
 * w4a16_affine_split (once, at load): from the column bit streams `packed` (uint32
 * [K*bits/32, N], the layout of w4a16_affine_widen) and the bf16 scales and biases [K/g, N] it
 * writes the two planes as one 4-bit matrix over 2K rows:
 *   qweight_out uint32 [2K/8, N]   rows 0..K-1 the low nibbles, rows K..2K-1 the high nibbles
 *   scales_out  bf16   [2K/g, N]   s, then 16 s (exact; a scale of magnitude 2^124 or more
 *                                  overflows to infinity)
 *   biases_out  bf16   [2K/g, N]   b, then 0
 * bits in 5..8; K % 32 == 0, K % group_size == 0, group_size % 32 == 0, N % 8 == 0; 16-byte
 * aligned, no overlap. Bit-exact; no scratch.
 *
 * w4a16_gemm_affine_split: out[M, N] = A[M, K] x W with W = s * q + b from those planes (qweight,
 * scales, biases as written above, for the original K). The two planes run as a pair of
 * matrices over the same activations in one launch, as w4a16_gemm_gate_up does, their two sums
 * of a column added in the epilogue; the accuracy contract is w4a16_gemm_affine's, with the bound
 * sum |a| (|s q| + |b|) of the original codes. M in 1..16; A, out, scratch and the other rules as
 * w4a16_gemm_affine.
 */
int w4a16_affine_split(const uint32_t *packed, int bits, const uint16_t *scales,
                       const uint16_t *biases, int group_size, int K, int N,
                       uint32_t *qweight_out, uint16_t *scales_out, uint16_t *biases_out,
                       hipStream_t stream);
int w4a16_gemm_affine_split(const void *A, const uint32_t *qweight, const uint16_t *scales,
                            const uint16_t *biases, int group_size, int M, int N, int K, void *out,
                            int out_dtype, hipStream_t stream);

/*
 * Greedy pick per row: idx[m] = smallest n with logits[m][n] equal to the row maximum (fp32
 * comparison, -0 == +0, NaN entries ignored; an all-NaN row gives 0).
 *   logits fp32 [M, N] device, 16-byte aligned; M in 1..65535; N in 1..2^31-1
 *   idx    int32 [M] device
 */
int w4a16_argmax_rows(const float *logits, int M, int N, int32_t *idx, hipStream_t stream);

/*
 * Test hooks running the kernels' own unpack/dequant device code.
 * w4a16_unpack_u8: q_out[k][n] (uint8 [K, N]) = code of row k, column n. K % 8 == 0, N % 4 == 0.
 * w4a16_dequant_f32: w_out[k][n] (fp32 [K, N]) = (q - z) * scale, exact. Same size rules as
 * w4a16_gemm for group_size, K and N. All pointers 16-byte aligned.
 */
int w4a16_unpack_u8(const uint32_t *qweight, int K, int N, uint8_t *q_out, hipStream_t stream);
int w4a16_dequant_f32(const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                      int group_size, int K, int N, float *w_out, hipStream_t stream);

/*
 * Measurement hook: a plain streaming read of `bytes` bytes at `buf` (16-byte non-temporal loads,
 * each workgroup one contiguous 16 KiB chunk), the ceiling that the weight-streaming kernels'
 * HBM rate is compared with. Reads the buffer once; stores one word to `sink` (device, 4 bytes)
 * only if the XOR of what a thread read equals a fixed constant. bytes: a positive multiple of
 * 16; buf 16-byte aligned.
 */
int w4a16_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Release every scratch buffer the library holds (all devices, all streams). The caller
 * must ensure no library work is still running. Returns W4A16_OK or W4A16_ERR_HIP. */
int w4a16_release_scratch(void);

const char *w4a16_status_string(int status);
const char *w4a16_last_error(void);
int w4a16_version(void);   /* 100 * major + minor */
/* Hash of the sources and compiler flags the library was built from (16 hex digits); the
 * Python binding refuses a library whose hash differs from its sources'. */
const char *w4a16_source_hash(void);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_H */
