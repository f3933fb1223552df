/*
 * kvq.h -- C ABI of the MI355X (gfx950) VAR-Q packed KV-cache library.
 *
 * VAR-Q ("VAR-Q: Tuning-Free KV Cache Quantization for Visual Autoregressive
 * Image and Video Generation", abstract and key contributions) observes that
 * block-by-block visual AR decoding produces KV caches whose massive-value
 * channels are persistent inside a (block, channel) cell and shift across
 * cells, and quantizes in groups along exactly those two axes, taking the
 * block boundaries from the generation loop; bit-packing kernels make the
 * memory saving real at run time.  This library is that hot path on one GPU:
 *
 *   kvq_quantize_block  quantize one freshly decoded block of K and V with an
 *                       asymmetric min/max grid per (sequence, block, head,
 *                       channel) group and bit-pack the codes into the cache;
 *   kvq_pack            the bit-packing step alone (codes given one per byte);
 *   kvq_attend_packed   block-causal attention of the block's queries over the
 *                       packed cache of blocks 0..k, dequantizing on the fly;
 *   kvq_quantize_attend one decode step of one layer: kvq_quantize_block then
 *                       kvq_attend_packed for the same block, in one launch
 *                       where a fused kernel covers the shape;
 *   kvq_attend_packed_split  kvq_attend_packed for long prefixes (next-frame
 *                       video): key ranges in a caller-provided workspace,
 *                       merged by log-sum-exp;
 *   kvq_bytes           the cache's byte accounting (host only).
 *
 * Conventions shared by every call
 *   - All buffers are owned by the caller; the library allocates nothing and
 *     keeps no state, so calls are reentrant.  Device pointers must be
 *     16-byte aligned device memory (else KVQ_E_INVAL).
 *   - Calls are asynchronous on `stream` (NULL = the null stream); argument
 *     errors are returned synchronously before anything is launched; a launch
 *     failure is returned as KVQ_E_DEVICE.
 *   - Tensor layouts (row-major, innermost last):
 *       block input  x[B][n_k][H][D]      K, V or Q of block k (n_k tokens)
 *       codes        [B][H][T][R]         T = sum of all block_tokens,
 *                                         R = ceil(bits * D / 8) bytes per row
 *       zero, scale  [B][H][NB][D]        IEEE binary16 bit patterns
 *       attention out[B][n_k][H][D]       fp32
 *     Block k's rows are tokens [off_k, off_k + n_k) with off_k the sum of
 *     block_tokens[0..k-1].
 *   - Quantizer of one group with values x_i (binary32) and L = 2^bits - 1:
 *       z = largest binary16 <= min_i x_i,
 *       s = smallest binary16 >= fp32(fp32(max_i x_i - z) / L),
 *       code_i = clamp(round_half_even(fp32(fp32(x_i - z) * fp32(1/s))), 0, L)
 *       (all codes 0 when s = 0), dequantized value fma(code, s, z).
 *     A zero extreme is taken as +0.  Every value lies on or inside
 *     [z, z + L*s], so |x - x_hat| <= s/2 up to binary32 rounding.
 *   - Packing: each (sequence, head, token) row of D codes is an LSB-first bit
 *     stream; code d occupies stream bits [bits*d, bits*d + bits) and stream
 *     bit j is bit (j mod 8) of byte floor(j/8), so 3-bit codes 2 and 5 of
 *     every eight straddle byte boundaries.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_MAX_BLOCKS 64

/*
 * Debug mode: with KVQ_DEBUG=1 (any value but empty or "0") in the environment,
 * every call that launches work synchronizes its stream after the launch
 * (unless the stream is being captured into a graph) and checks
 * hipGetLastError; a failure is printed on stderr with the call's name and
 * returned as KVQ_E_DEVICE.  Off by default: calls are asynchronous.
 */

/* return codes */
#define KVQ_OK 0
#define KVQ_E_INVAL (-1)       /* bad argument, layout, pointer or alignment */
#define KVQ_E_UNSUPPORTED (-2) /* valid, but not built for this GPU path */
#define KVQ_E_DEVICE (-3)      /* HIP launch / runtime failure */

/* device status bits OR-ed into *status_dev by kvq_quantize_block */
#define KVQ_S_NONFINITE 1 /* a NaN or +-inf input value */
#define KVQ_S_RANGE 2     /* a group extreme outside +-65504 (binary16 range) */

/* source dtypes */
#define KVQ_F32 0
#define KVQ_BF16 1

/*
 * Cache geometry, a plain value owned by the caller.
 *   batch       sequences B (>= 1)
 *   heads       H (>= 1)
 *   head_dim    D (multiple of 8; the GPU kernels are built for 64 and 128)
 *   bits        code width: 2, 3, 4 or 8 on the GPU (the byte accounting takes 1..8)
 *   n_blocks    NB, number of decode blocks (1..KVQ_MAX_BLOCKS)
 *   pack_mode   0 = dense rows: each (b, h, token) row of D codes LSB-first in
 *               ceil(bits*D/8) bytes;
 *               1 = word-aligned: each (b, h) cache is one stream of T*D codes
 *               in 32-bit words of floor(32/bits) codes, low bits first (3-bit
 *               codes: 10 per word, 3.2 stored bits, the storage the VAR-Q
 *               results table's INT3 rows correspond to).  Mode 1 is taken by
 *               kvq_bytes, kvq_pack and kvq_unpack; the decode calls return
 *               KVQ_E_UNSUPPORTED for it (one stream cannot take a block at a
 *               time);
 *               2 = block-aligned words: each (b, h, block) stream of n_k*D
 *               codes, row after row, in 32-bit words of floor(32/bits) codes
 *               as in mode 1, every block from a fresh word.  The decode calls
 *               take it: INT3 stores ten codes per word (VAR-d20, 2x128
 *               sequences, 20 layers: 3.81 GiB, a 77.04% saving beside the
 *               table's 77.06%, 4356 words per (b, h) against mode 1's 4352).
 *               With 2-, 4- or 8-bit codes and head_dim 64 or 128 its bytes
 *               are those of mode 0.
 *   block_tokens[k]  tokens of block k (>= 1), e.g. s*s for next-scale
 *                    prediction at scale s, or a frame's tokens for video
 * The decode calls (kvq_quantize_block, kvq_attend_packed, kvq_quantize_attend)
 * take batch * heads < 2^25 (else KVQ_E_UNSUPPORTED), so that each of their
 * launches stays under 2^32 work-items.
 */
typedef struct {
  int32_t batch, heads, head_dim, bits, n_blocks, pack_mode;
  int32_t block_tokens[KVQ_MAX_BLOCKS];
} kvq_layout;

/* one packed cache (K or V of one layer); device pointers */
typedef struct {
  uint8_t* codes;  /* [B][H][T][R]; pack_mode 2: [B][H][W] 32-bit words, W the
                      words of all NB blocks (code_bytes of kvq_bytes / (B*H*4)) */
  uint16_t* zero;  /* [B][H][NB][D] binary16 */
  uint16_t* scale; /* [B][H][NB][D] binary16 */
} kvq_cache;

typedef struct {
  const uint8_t* codes;
  const uint16_t* zero;
  const uint16_t* scale;
} kvq_cache_const;

/*
 * kvq_bytes -- bytes held by one (layer, K or V) cache once blocks
 * 0..n_filled-1 are stored: code_bytes = B*H*T*R with T = sum of their
 * block_tokens (pack_mode 1: B*H*4*ceil(T*D/floor(32/bits)); pack_mode 2:
 * B*H*4*sum_k ceil(n_k*D/floor(32/bits)) over those blocks), stat_bytes =
 * B*H*n_filled*D*4 (one binary16 zero + one binary16 step per (block, channel)
 * group).  With n_filled = n_blocks these are the allocation sizes of codes and
 * of zero+scale together.  Host only, pure.  Follows the KV-memory accounting
 * of the VAR-Q results table (VAR-d20 at 2x128 sequences: 16.60 -> 4.64 GiB at
 * INT4, 72.06% saving; INT3 in pack_mode 1: 3.81 GiB, 77.06%).
 * Returns KVQ_OK or KVQ_E_INVAL (bad layout, n_filled out of [0, NB], NULL out).
 */
int kvq_bytes(const kvq_layout* layout, int32_t n_filled, uint64_t* code_bytes,
              uint64_t* stat_bytes);

/*
 * kvq_quantize_block -- quantize block `block` of K and V of one layer and
 * store it packed (VAR-Q: groups keyed on (block, channel), block boundary
 * handed over by the generation loop; then bit-packing).
 *   k_src, v_src  [B][n_k][H][D], dtype src_dtype (KVQ_F32 or KVQ_BF16)
 *   k_cache, v_cache  caches of the layer; only rows [off_k, off_k + n_k) of
 *                 every (b, h) (pack_mode 2: block k's words) and stats slot k
 *                 are written, no other byte
 *   status_dev    NULL, or a device int32 into which KVQ_S_* bits are OR-ed
 *                 (read it after synchronizing the stream).  With NULL the
 *                 inputs are not screened and a non-finite or out-of-range
 *                 input leaves that group's outputs undefined.
 * Errors: KVQ_E_INVAL (layout, block, dtype, NULL or misaligned pointer),
 * KVQ_E_UNSUPPORTED (bits or head_dim not built, pack_mode 1, batch * heads >=
 * 2^25), KVQ_E_DEVICE.
 */
int kvq_quantize_block(const kvq_layout* layout, int32_t block, int32_t src_dtype,
                       const void* k_src, const void* v_src, kvq_cache k_cache,
                       kvq_cache v_cache, int32_t* status_dev, hipStream_t stream);

/*
 * kvq_pack -- the bit-packing step on its own: rows of `row_len` codes, one
 * code per byte (only the low `bits` bits of each byte are used), packed into
 * rows of ceil(bits*row_len/8) bytes at dst + r*dst_row_stride, bytes between
 * rows untouched.  Same bit layout as the cache rows written by
 * kvq_quantize_block ("bit-packing kernels", VAR-Q abstract).
 *   pack_mode 1: the n_rows*row_len codes, row after row, form one stream
 *   written as ceil(n/floor(32/bits)) 32-bit words at dst; dst_row_stride
 *   must be 0.
 *   bits 1..8, pack_mode 0 or 1, n_rows >= 0, row_len >= 1,
 *   dst_row_stride >= ceil(bits*row_len/8).
 * codes/dst: device pointers (16-byte aligned).
 */
int kvq_pack(int32_t bits, int32_t pack_mode, const uint8_t* codes, int64_t n_rows,
             int32_t row_len, uint8_t* dst, int64_t dst_row_stride, hipStream_t stream);

/*
 * kvq_attend_packed -- block-causal attention for block k's queries:
 *   out[b][i][h][:] = softmax_t(scale * q[b][i][h] . k_hat[b][h][t]) v_hat[b][h][t]
 * over every token t of blocks 0..k (the whole prefix, no mask inside block
 * k), where k_hat / v_hat are the dequantized cache values fma(code, s, z)
 * formed in registers from the packed rows (block-by-block decoding, VAR-Q
 * abstract; "quantize, then attend": block k's own keys are read packed).
 *   q_bf16   [B][n_k][H][D] bfloat16 bit patterns
 *   scale    softmax scale; <= 0 selects 1/sqrt(D)
 *   out      [B][n_k][H][D] fp32
 * Accuracy: max|out - exact| <= 2e-3 * max|exact|, per call and within every
 * (sequence, head), where exact is the binary64 attention over the same
 * dequantized values.  Arithmetic: QK^T as two bf16 MFMA products of a hi/lo
 * split of k_hat (k_hat to about 2^-17 relative), P and v_hat in fp16 (v_hat
 * formed at half scale when a V group's grid top z + L*s lies above 65504, so
 * it never overflows), fp32 accumulation and softmax.  The bound covers every
 * value the quantizer accepts (|x| <= 65504) as long as each score's absolute
 * sum scale * sum_d |q_d * k_hat_d| stays below about 100 (about 30 on
 * VAR-shaped data): a score carries an absolute error of order 2^-17 of that
 * sum, which the softmax turns into a relative error of the weights.
 * Errors as kvq_quantize_block.
 */
int kvq_attend_packed(const kvq_layout* layout, int32_t block, const uint16_t* q_bf16,
                      kvq_cache_const k_cache, kvq_cache_const v_cache, float scale,
                      float* out, hipStream_t stream);

/*
 * kvq_attend_packed_split -- kvq_attend_packed for long prefixes and few query
 * tiles (VAR-Q abstract: next-frame prediction decodes whole frames block by
 * block over a growing prefix; here 40 heads x 1560 queries over up to 16
 * frames of 1560 keys), where one workgroup per (sequence, head, 256 queries) leaves
 * most of the GPU idle in the grid's last round.  The key prefix of every
 * query tile is cut into up to max_splits ranges of whole 32-key tiles; each
 * range is attended by its own workgroup into a partial result (unnormalized
 * output, running maximum, softmax denominator) in `workspace`, and a second
 * launch merges the partials by log-sum-exp.  Same arithmetic per key as
 * kvq_attend_packed, summed in another order: results agree with it and the
 * exact attention within the same 2e-3 bound.
 *   max_splits  1..64, an upper bound: blocks of at most 128 queries, short
 *               prefixes (fewer than 16 key tiles per range) and grids that
 *               already hold about four workgroups per CU use fewer ranges,
 *               down to one (then this is exactly kvq_attend_packed)
 *   workspace   caller-owned device memory of at least workspace_bytes >=
 *               kvq_attend_split_workspace(layout, block, max_splits) bytes,
 *               16-byte aligned, not overlapping any other argument; its
 *               contents on entry are ignored and on return unspecified
 * Errors as kvq_attend_packed; KVQ_E_INVAL also for max_splits out of range
 * or a missing, misaligned or too small workspace.
 */
int kvq_attend_packed_split(const kvq_layout* layout, int32_t block, const uint16_t* q_bf16,
                            kvq_cache_const k_cache, kvq_cache_const v_cache, float scale,
                            float* out, int32_t max_splits, void* workspace,
                            uint64_t workspace_bytes, hipStream_t stream);

/* workspace bytes kvq_attend_packed_split needs for block `block` and
 * max_splits ranges: max_splits * B * n_k * H * (D + 2) * 4.  Host only. */
int kvq_attend_split_workspace(const kvq_layout* layout, int32_t block, int32_t max_splits,
                               uint64_t* bytes);

/* size of the static device scratch array of kvq_attend_packed_split_noalloc:
 * one copy per GPU the library runs on, held until the process ends (128 MiB:
 * a next-frame video frame of 40 heads x 1560 queries at head_dim 128 in 4 key
 * ranges needs 124 MiB) */
#define KVQ_STATIC_SCRATCH_BYTES (128ull << 20)

/*
 * kvq_attend_packed_split_noalloc -- kvq_attend_packed_split for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the key ranges' partials live in
 * the library's static device array of KVQ_STATIC_SCRATCH_BYTES on the current
 * GPU instead of a caller workspace.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); on its first use on a GPU it looks up that
 * GPU's copy of the array once.  Outputs equal kvq_attend_packed_split's with
 * the same layout, block, inputs, scale and max_splits.
 *   Errors as kvq_attend_packed_split; KVQ_E_INVAL also when
 *   kvq_attend_split_workspace(layout, block, max_splits) exceeds
 *   KVQ_STATIC_SCRATCH_BYTES (lower max_splits, or use the workspace call).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call writes every partial before it reads it, so nothing is
 * cleared): calls ordered on one stream are safe, calls that overlap in time
 * on one GPU (several streams, or host threads without ordering) race.
 */
int kvq_attend_packed_split_noalloc(const kvq_layout* layout, int32_t block,
                                    const uint16_t* q_bf16, kvq_cache_const k_cache,
                                    kvq_cache_const v_cache, float scale, float* out,
                                    int32_t max_splits, hipStream_t stream);

/*
 * kvq_quantize_attend -- the decode step of one layer for block k (VAR-Q
 * abstract: the block is quantized when the generation loop hands it over,
 * then the block's queries attend to the packed cache of blocks 0..k).
 * Results are those of kvq_quantize_block(layout, block, src_dtype, k_src,
 * v_src, k_cache, v_cache, status_dev) followed by kvq_attend_packed(layout,
 * block, q_bf16, k_cache, v_cache, scale, out) on the same stream: the same
 * cache bytes and statistics, and the same output values.  Where a fused
 * kernel covers the shape it is one launch in which each (sequence, head)
 * quantizes its own block and then attends: head_dim 64 with blocks of at
 * most 32 tokens (bf16 or fp32 input) or of 33..256 tokens (bf16 input).
 * Otherwise the two launches are issued in order.
 *   Arguments as in the two calls; out must not overlap the caches or inputs.
 * Errors: the union of both calls' errors, checked before any launch.
 */
int kvq_quantize_attend(const kvq_layout* layout, int32_t block, int32_t src_dtype,
                        const void* k_src, const void* v_src, const uint16_t* q_bf16,
                        kvq_cache k_cache, kvq_cache v_cache, float scale, float* out,
                        int32_t* status_dev, hipStream_t stream);

/* ---- test and measurement helpers (not on the decode path) -------------- */

/* inverse of kvq_pack: codes[r][j] = code j of packed row r (one per byte) */
int kvq_unpack(int32_t bits, int32_t pack_mode, const uint8_t* src, int64_t src_row_stride,
               int64_t n_rows, int32_t row_len, uint8_t* codes, hipStream_t stream);

/* dequantized cache of blocks 0..n_filled-1: out[B][H][T][D] fp32 with
 * T = off_{n_filled}; each value fma(code, s, z) as in the attention */
int kvq_dequantize(const kvq_layout* layout, int32_t n_filled, kvq_cache_const cache,
                   float* out, hipStream_t stream);

/* plain streaming copy of n_bytes (multiple of 16): measures the achievable
 * HBM bandwidth and calibrates the memory counters */
int kvq_stream_copy(const void* src, void* dst, uint64_t n_bytes, hipStream_t stream);

/* plain streaming read of n_bytes (multiple of 16) into nothing: measures the
 * achievable HBM read bandwidth (the decode passes mostly read); `sink` is a
 * device word that is written only if the data's xor fold equals a fixed
 * pattern, so the loads cannot be optimized away */
int kvq_stream_read(const void* src, uint64_t n_bytes, uint32_t* sink, hipStream_t stream);

/* version string of the library */
const char* kvq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
