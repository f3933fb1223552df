/*
 * kvq_oracle.h -- plain CPU oracle for the VAR-Q packed KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously correct
 * reference that the GPU library is checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header, table or constant with
 * the GPU library (visual_autoregressive_kv_amd/csrc, include/kvq.h).
 *
 * Method source: "VAR-Q: Tuning-Free KV Cache Quantization for Visual
 * Autoregressive Image and Video Generation" (abstract and key contributions):
 * KV caches of block-by-block visual AR decoding are quantized in groups along
 * two axes, block and feature channel, with block boundaries taken from the
 * generation loop, and the codes are bit-packed so the saving holds at run
 * time.  The pages print no formula; the readings used here (asymmetric
 * min/max affine quantizer, fp16 zero rounded down and fp16 step rounded up,
 * round-half-even codes, LSB-first row packing) are the plainest ones that
 * reproduce the VAR rows of the "VAR-Q Tables 2-4" results page (KV memory
 * 16.60 -> 4.64 at INT4, 72.06% saving).
 *
 * Precision: statistics and codes are decided in IEEE binary32 exactly as the
 * GPU must (integers decided by floating point are decided in the kernel's
 * precision); attention is computed in binary64.
 *
 * Parity pins: every function here is pinned by tests under tests/ against
 * properties that do not come from this file (exhaustive defining properties,
 * closed forms, brute force, the pages' table).  See the header of
 * kvq_oracle.c for the pin of each function.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQR_MAX_BLOCKS 64

/* status / error codes (values match the product ABI by convention only) */
#define KVQR_OK 0
#define KVQR_E_INVAL (-1)
#define KVQR_S_NONFINITE 1
#define KVQR_S_RANGE 2

#define KVQR_F32 0
#define KVQR_BF16 1

typedef struct {
  int32_t batch, heads, head_dim, bits, n_blocks, pack_mode;
  int32_t block_tokens[KVQR_MAX_BLOCKS];
} kvqr_layout;

typedef struct {
  uint8_t* codes;   /* [B][H][T][R] packed rows, T = sum of block_tokens (pack_mode 0);
                       [B][H][W] 32-bit words, W = words of all blocks (pack_mode 2) */
  uint16_t* zero;   /* [B][H][NB][D] binary16 bit patterns */
  uint16_t* scale;  /* [B][H][NB][D] binary16 bit patterns */
} kvqr_cache;

/* binary16 helpers (bit patterns) */
float kvqr_h2f(uint16_t h);
uint16_t kvqr_rd16(float x); /* largest binary16 <= x  */
uint16_t kvqr_ru16(float x); /* smallest binary16 >= x */
void kvqr_rd16_n(const float* x, int64_t n, uint16_t* out);
void kvqr_ru16_n(const float* x, int64_t n, uint16_t* out);

/* layout */
int kvqr_validate(const kvqr_layout* L);
int64_t kvqr_total_tokens(const kvqr_layout* L, int32_t n_filled);
int64_t kvqr_block_offset(const kvqr_layout* L, int32_t block);
int32_t kvqr_row_bytes(int32_t bits, int32_t head_dim);
/* word-aligned layout (pack_mode 1): codes per 32-bit word, words of a stream */
int32_t kvqr_codes_per_word(int32_t bits);
int64_t kvqr_stream_words(int32_t bits, int64_t n_codes);
/* block-aligned word layout (pack_mode 2): words before block `block` of one
 * (b, h) cache; each block's n_k x D codes start on a fresh word */
int64_t kvqr_block_word_offset(const kvqr_layout* L, int32_t block);

/* one (block, channel) group: n values at x[i*stride] */
int kvqr_quantize_group(const float* x, int64_t n, int64_t stride, int32_t bits,
                        uint16_t* zero, uint16_t* scale, uint8_t* codes);

/* quantize + pack block `block` of K and V for every sequence/head */
int kvqr_quantize_block(const kvqr_layout* L, int32_t block, int32_t src_dtype,
                        const void* k_src, const void* v_src, kvqr_cache k_cache,
                        kvqr_cache v_cache);

/* bit packing of rows of one-code-per-byte.  pack_mode 0: each row LSB-first
 * into ceil(bits*row_len/8) bytes at dst + r*stride.  pack_mode 1: all rows as
 * one stream into 32-bit words of floor(32/bits) codes (stride must be 0). */
void kvqr_pack_row(int32_t bits, const uint8_t* codes, int32_t n, uint8_t* out);
void kvqr_unpack_row(int32_t bits, const uint8_t* in, int32_t n, uint8_t* codes);
int kvqr_pack(int32_t bits, int32_t pack_mode, const uint8_t* codes, int64_t n_rows,
              int32_t row_len, uint8_t* dst, int64_t dst_row_stride);
int kvqr_unpack(int32_t bits, int32_t pack_mode, const uint8_t* src, int64_t src_row_stride,
                int64_t n_rows, int32_t row_len, uint8_t* codes);

/* dequantized cache [B][H][T][D] fp32 for the first n_filled blocks */
int kvqr_dequantize(const kvqr_layout* L, int32_t n_filled, kvqr_cache c, float* out);

/* block-causal attention of block `block`'s queries over blocks 0..block.
 * q: [B][n_k][H][D] bf16 bits; out: [B][n_k][H][D] fp32, written for b in [b0,b1).
 * scale <= 0 selects 1/sqrt(D). */
int kvqr_attend(const kvqr_layout* L, int32_t block, const uint16_t* q, kvqr_cache k,
                kvqr_cache v, double scale, float* out, int32_t b0, int32_t b1);
/* one output row (b, query i of the block, head h) in binary64 */
int kvqr_attend_row(const kvqr_layout* L, int32_t block, const uint16_t* q, kvqr_cache k,
                    kvqr_cache v, double scale, int32_t b, int32_t i, int32_t h,
                    double* out_row);

/* byte accounting per (layer, K or V) */
int kvqr_bytes(const kvqr_layout* L, int32_t n_filled, uint64_t* code_bytes,
               uint64_t* stat_bytes);

#ifdef __cplusplus
}
#endif
#endif
