/*
 * kvq_oracle.c -- plain, slow, obviously correct CPU oracle of the VAR-Q
 * packed KV-cache hot path.  TEST INFRASTRUCTURE ONLY: loaded by tests/, the
 * smoke check and the benchmark's CPU-baseline leg, never by the product path.
 * No threads, no SIMD, no blocking: one loop per definition.
 *
 * What it follows ("VAR-Q: Tuning-Free KV Cache Quantization for Visual
 * Autoregressive Image and Video Generation", abstract + key contributions):
 *   - decoding is block by block; block k's tokens attend to every block <= k;
 *   - quantization groups run along two axes, block and feature channel, and
 *     the block boundaries come from the generation loop (no calibration);
 *   - codes are bit-packed so the memory saving is real at run time.
 * Readings of what the pages leave open (each pinned by a test):
 *   - quantizer: asymmetric min/max affine grid with 2^b levels per
 *     (sequence, block, head, channel) group; zero z = fp16 rounded DOWN from
 *     the group minimum, step s = fp16 rounded UP from fp32 (max - z)/(2^b-1),
 *     code = round-half-even(fp32((x - z) * fp32(1/s))) clamped to [0, 2^b-1];
 *     two 16-bit statistics per group reproduce the VAR rows of the
 *     "VAR-Q Tables 2-4" results page (BF16 16.60 -> INT4 4.64, 72.06%);
 *   - packing: each (sequence, head, token) row of D codes is an LSB-first bit
 *     stream, code d occupying stream bits [b*d, b*d+b); 3-bit codes therefore
 *     straddle byte boundaries (pack_mode 0);
 *   - block-aligned words (pack_mode 2): each (sequence, head, block) stream of
 *     n_k x D codes, row after row, in 32-bit words of floor(32/b) codes, every
 *     block from a fresh word, so INT3 stores ten codes per word and a block is
 *     written once, when decoding reaches it;
 *   - attention: softmax(scale * q . k_hat) v_hat over the whole prefix of
 *     blocks 0..k, no mask inside block k, in binary64.
 *
 * Pins (tests/test_oracle_*.py):
 *   kvqr_rd16/ru16  exhaustive over all 2^32 fp32 patterns vs a merge walk over
 *                   numpy's own binary16 value table (defining property);
 *   kvqr_h2f        all 65536 patterns vs numpy float16 -> float64;
 *   quantize_group  closed forms ({0..15} -> identity grid, constant group,
 *                   {-1, 1}), brute-force argmin over the grid, half-step bound;
 *   pack/unpack     hand-computed worked bytes (tests/golden/pack_examples.txt),
 *                   exhaustive round trips; block-aligned words by a
 *                   hand-worked two-block example (block_words_example.txt);
 *   attend          independent float64 numpy softmax attention, closed forms
 *                   (single key, identical keys), block causality, permutation;
 *   bytes           the page's KV memory column (tests/golden/kv_table.txt),
 *                   every layout.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* binary16 by definition: value = (-1)^s * 2^(e-15) * (1 + m/1024) for      */
/* 0 < e < 31, (-1)^s * 2^-14 * (m/1024) for e = 0.                          */
/* ------------------------------------------------------------------------ */

float kvqr_h2f(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 31) {
    if (m != 0) return NAN;
    return sign ? -INFINITY : INFINITY;
  }
  if (e == 0)
    v = ldexp((double)m, -24);
  else
    v = ldexp((double)(1024 + m), e - 25);
  return (float)(sign ? -v : v);
}

/* bit pattern of a non-negative magnitude that is exactly a binary16 value */
static uint16_t encode_mag16(double a) {
  if (a == 0.0) return 0;
  if (a < ldexp(1.0, -14)) return (uint16_t)(a / ldexp(1.0, -24));
  int e2;
  frexp(a, &e2); /* a in [2^(e2-1), 2^e2) */
  double ulp = ldexp(1.0, e2 - 1 - 10);
  int64_t M = (int64_t)(a / ulp); /* 1024 .. 2047 */
  return (uint16_t)(((e2 - 1 + 15) << 10) | (int)(M - 1024));
}

/* grid spacing of binary16 around a non-negative magnitude a */
static double ulp16(double a) {
  if (a < ldexp(1.0, -14)) return ldexp(1.0, -24);
  int e2;
  frexp(a, &e2);
  return ldexp(1.0, e2 - 11);
}

/* largest binary16 magnitude <= a (a >= 0 finite); saturates at 65504 */
static double floor_mag16(double a) {
  if (a >= 65504.0) return 65504.0;
  double u = ulp16(a);
  return floor(a / u) * u;
}

/* smallest binary16 magnitude >= a (a >= 0 finite); +inf above 65504 */
static double ceil_mag16(double a) {
  if (a > 65504.0) return INFINITY;
  double u = ulp16(a);
  return ceil(a / u) * u;
}

static uint16_t signed16(int neg, double mag) {
  uint16_t s = neg ? 0x8000 : 0;
  if (isinf(mag)) return (uint16_t)(s | 0x7C00);
  return (uint16_t)(s | encode_mag16(mag));
}

uint16_t kvqr_rd16(float x) {
  if (isnan(x)) return 0x7E00;
  if (isinf(x)) return x > 0 ? 0x7C00 : 0xFC00;
  if (!signbit(x)) return signed16(0, floor_mag16((double)x));
  return signed16(1, ceil_mag16(-(double)x)); /* -inf below -65504 */
}

uint16_t kvqr_ru16(float x) {
  if (isnan(x)) return 0x7E00;
  if (isinf(x)) return x > 0 ? 0x7C00 : 0xFC00;
  if (!signbit(x)) return signed16(0, ceil_mag16((double)x)); /* +inf above 65504 */
  return signed16(1, floor_mag16(-(double)x));
}

void kvqr_rd16_n(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = kvqr_rd16(x[i]);
}

void kvqr_ru16_n(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = kvqr_ru16(x[i]);
}

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------------ */
/* layout                                                                   */
/* ------------------------------------------------------------------------ */

int32_t kvqr_row_bytes(int32_t bits, int32_t head_dim) { return (bits * head_dim + 7) / 8; }

/* Word-aligned layout (pack_mode 1): the codes of a whole stream go into 32-bit
 * words holding floor(32 / bits) codes each, low bits first; the word's top
 * 32 mod bits bits stay zero (3-bit codes: 10 per word, 2 spare bits, i.e. 3.2
 * stored bits per code as in the VAR-Q results table's INT3 rows). */
int32_t kvqr_codes_per_word(int32_t bits) { return 32 / bits; }
int64_t kvqr_stream_words(int32_t bits, int64_t n_codes) {
  const int64_t cpw = kvqr_codes_per_word(bits);
  return (n_codes + cpw - 1) / cpw;
}

int kvqr_validate(const kvqr_layout* L) {
  if (!L) return KVQR_E_INVAL;
  if (L->batch < 1 || L->heads < 1) return KVQR_E_INVAL;
  if (L->head_dim < 8 || L->head_dim % 8 != 0) return KVQR_E_INVAL;
  if (L->bits < 1 || L->bits > 8) return KVQR_E_INVAL;
  if (L->n_blocks < 1 || L->n_blocks > KVQR_MAX_BLOCKS) return KVQR_E_INVAL;
  if (L->pack_mode < 0 || L->pack_mode > 2) return KVQR_E_INVAL;
  for (int i = 0; i < L->n_blocks; i++)
    if (L->block_tokens[i] < 1) return KVQR_E_INVAL;
  return KVQR_OK;
}

int64_t kvqr_block_offset(const kvqr_layout* L, int32_t block) {
  int64_t off = 0;
  for (int i = 0; i < block; i++) off += L->block_tokens[i];
  return off;
}

int64_t kvqr_total_tokens(const kvqr_layout* L, int32_t n_filled) {
  return kvqr_block_offset(L, n_filled);
}

/* Block-aligned word layout (pack_mode 2): each (b, h) cache is the sequence of
 * its blocks' streams; block k's stream is its n_k x D codes, row after row,
 * in 32-bit words of floor(32 / bits) codes (as in pack_mode 1), and starts on
 * a fresh word, so every block is written once, when the generation loop hands
 * it over.  Words of blocks 0..block-1 come before block `block`. */
int64_t kvqr_block_word_offset(const kvqr_layout* L, int32_t block) {
  int64_t w = 0;
  for (int32_t k = 0; k < block; k++)
    w += kvqr_stream_words(L->bits, (int64_t)L->block_tokens[k] * L->head_dim);
  return w;
}

/* ------------------------------------------------------------------------ */
/* quantizer of one (block, channel) group                                  */
/* ------------------------------------------------------------------------ */

int kvqr_quantize_group(const float* x, int64_t n, int64_t stride, int32_t bits,
                        uint16_t* zero, uint16_t* scale, uint8_t* codes) {
  const float levels = (float)((1 << bits) - 1);
  *zero = 0;
  *scale = 0;
  for (int64_t i = 0; i < n; i++) codes[i] = 0;
  if (n < 1) return KVQR_OK;

  /* 1. finite inputs only */
  for (int64_t i = 0; i < n; i++)
    if (!isfinite(x[i * stride])) return KVQR_S_NONFINITE;

  /* 2. exact group extremes; a zero extreme is taken as +0 */
  float mn = x[0], mx = x[0];
  for (int64_t i = 1; i < n; i++) {
    float v = x[i * stride];
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  if (mn == 0.0f) mn = 0.0f;
  if (mx == 0.0f) mx = 0.0f;
  if (mn < -65504.0f || mx > 65504.0f) return KVQR_S_RANGE;

  /* 3. zero point: largest binary16 <= min, so the grid starts at or below it */
  uint16_t zb = kvqr_rd16(mn);
  float z = kvqr_h2f(zb);

  /* 4-5. step: binary32 width over the level count, rounded UP to binary16 so
   * that z + levels * s >= max (every value lies on or inside the grid) */
  float r = mx - z;
  float q = r / levels;
  uint16_t sb = kvqr_ru16(q);
  float s = kvqr_h2f(sb);
  if (isinf(s)) return KVQR_S_RANGE;

  /* 6. one reciprocal per group */
  float inv = (s > 0.0f) ? 1.0f / s : 0.0f;

  /* 7. codes: nearest grid point, ties to even, clamped to the grid */
  for (int64_t i = 0; i < n; i++) {
    float t = x[i * stride] - z;
    float u = t * inv;
    float c = rintf(u);
    if (c < 0.0f) c = 0.0f;
    if (c > levels) c = levels;
    codes[i] = (uint8_t)c;
  }
  *zero = zb;
  *scale = sb;
  return KVQR_OK;
}

/* ------------------------------------------------------------------------ */
/* packing                                                                  */
/* ------------------------------------------------------------------------ */

void kvqr_pack_row(int32_t bits, const uint8_t* codes, int32_t n, uint8_t* out) {
  int32_t nbytes = kvqr_row_bytes(bits, n);
  memset(out, 0, (size_t)nbytes);
  for (int32_t d = 0; d < n; d++) {
    for (int32_t j = 0; j < bits; j++) {
      int32_t pos = bits * d + j; /* stream bit */
      int bit = (codes[d] >> j) & 1;
      out[pos / 8] = (uint8_t)(out[pos / 8] | (bit << (pos % 8)));
    }
  }
}

void kvqr_unpack_row(int32_t bits, const uint8_t* in, int32_t n, uint8_t* codes) {
  for (int32_t d = 0; d < n; d++) {
    int c = 0;
    for (int32_t j = 0; j < bits; j++) {
      int32_t pos = bits * d + j;
      c |= ((in[pos / 8] >> (pos % 8)) & 1) << j;
    }
    codes[d] = (uint8_t)c;
  }
}

/* pack_mode 1: the n_rows x row_len codes, row after row, are one stream */
static void pack_words(int32_t bits, const uint8_t* codes, int64_t n, uint8_t* dst) {
  const int64_t cpw = kvqr_codes_per_word(bits);
  const int64_t words = kvqr_stream_words(bits, n);
  for (int64_t w = 0; w < words; w++) {
    uint32_t word = 0;
    for (int64_t k = 0; k < cpw; k++) {
      const int64_t i = w * cpw + k;
      if (i < n) word |= (uint32_t)(codes[i] & ((1u << bits) - 1u)) << (bits * k);
    }
    for (int byte = 0; byte < 4; byte++) dst[4 * w + byte] = (uint8_t)(word >> (8 * byte));
  }
}
static void unpack_words(int32_t bits, const uint8_t* src, int64_t n, uint8_t* codes) {
  const int64_t cpw = kvqr_codes_per_word(bits);
  for (int64_t i = 0; i < n; i++) {
    const int64_t w = i / cpw, k = i % cpw;
    uint32_t word = 0;
    for (int byte = 0; byte < 4; byte++) word |= (uint32_t)src[4 * w + byte] << (8 * byte);
    codes[i] = (uint8_t)((word >> (bits * k)) & ((1u << bits) - 1u));
  }
}
/* codes i0 .. i0 + n - 1 of a word stream */
static void unpack_words_at(int32_t bits, const uint8_t* src, int64_t i0, int64_t n,
                            uint8_t* codes) {
  const int64_t cpw = kvqr_codes_per_word(bits);
  for (int64_t i = 0; i < n; i++) {
    const int64_t w = (i0 + i) / cpw, k = (i0 + i) % cpw;
    uint32_t word = 0;
    for (int byte = 0; byte < 4; byte++) word |= (uint32_t)src[4 * w + byte] << (8 * byte);
    codes[i] = (uint8_t)((word >> (bits * k)) & ((1u << bits) - 1u));
  }
}

int kvqr_pack(int32_t bits, int32_t pack_mode, const uint8_t* codes, int64_t n_rows,
              int32_t row_len, uint8_t* dst, int64_t dst_row_stride) {
  if (bits < 1 || bits > 8 || n_rows < 0 || row_len < 1) return KVQR_E_INVAL;
  if (pack_mode == 1) {  /* one stream; no row stride */
    if (dst_row_stride != 0) return KVQR_E_INVAL;
    pack_words(bits, codes, n_rows * row_len, dst);
    return KVQR_OK;
  }
  if (pack_mode != 0) return KVQR_E_INVAL;
  if (dst_row_stride < kvqr_row_bytes(bits, row_len)) return KVQR_E_INVAL;
  for (int64_t r = 0; r < n_rows; r++)
    kvqr_pack_row(bits, codes + r * row_len, row_len, dst + r * dst_row_stride);
  return KVQR_OK;
}

int kvqr_unpack(int32_t bits, int32_t pack_mode, const uint8_t* src, int64_t src_row_stride,
                int64_t n_rows, int32_t row_len, uint8_t* codes) {
  if (bits < 1 || bits > 8 || n_rows < 0 || row_len < 1) return KVQR_E_INVAL;
  if (pack_mode == 1) {
    if (src_row_stride != 0) return KVQR_E_INVAL;
    unpack_words(bits, src, n_rows * row_len, codes);
    return KVQR_OK;
  }
  if (pack_mode != 0) return KVQR_E_INVAL;
  if (src_row_stride < kvqr_row_bytes(bits, row_len)) return KVQR_E_INVAL;
  for (int64_t r = 0; r < n_rows; r++)
    kvqr_unpack_row(bits, src + r * src_row_stride, row_len, codes + r * row_len);
  return KVQR_OK;
}

/* ------------------------------------------------------------------------ */
/* quantize one block of K and V                                            */
/* ------------------------------------------------------------------------ */

static int quantize_one(const kvqr_layout* L, int32_t block, int32_t src_dtype, const void* src,
                        kvqr_cache c) {
  const int32_t B = L->batch, H = L->heads, D = L->head_dim, NB = L->n_blocks;
  const int32_t n = L->block_tokens[block];
  const int64_t off = kvqr_block_offset(L, block);
  const int64_t T = kvqr_total_tokens(L, NB);
  const int32_t R = kvqr_row_bytes(L->bits, D);
  float* col = (float*)malloc(sizeof(float) * (size_t)n);
  uint8_t* gcodes = (uint8_t*)malloc((size_t)n);
  uint8_t* tile = (uint8_t*)malloc((size_t)n * (size_t)D); /* [t][d] codes */
  int status = 0;
  if (!col || !gcodes || !tile) {
    free(col);
    free(gcodes);
    free(tile);
    return KVQR_E_INVAL;
  }
  for (int32_t b = 0; b < B; b++) {
    for (int32_t h = 0; h < H; h++) {
      for (int32_t d = 0; d < D; d++) {
        for (int32_t t = 0; t < n; t++) {
          int64_t idx = (((int64_t)b * n + t) * H + h) * D + d; /* x[b][t][h][d] */
          col[t] = (src_dtype == KVQR_F32) ? ((const float*)src)[idx]
                                           : bf16_to_f32(((const uint16_t*)src)[idx]);
        }
        uint16_t zb, sb;
        status |= kvqr_quantize_group(col, n, 1, L->bits, &zb, &sb, gcodes);
        int64_t sidx = (((int64_t)b * H + h) * NB + block) * D + d;
        c.zero[sidx] = zb;
        c.scale[sidx] = sb;
        for (int32_t t = 0; t < n; t++) tile[(int64_t)t * D + d] = gcodes[t];
      }
      if (L->pack_mode == 2) { /* the block's stream of n x D codes, from a fresh word */
        const int64_t W = kvqr_block_word_offset(L, NB);
        uint8_t* words = c.codes + (((int64_t)b * H + h) * W + kvqr_block_word_offset(L, block)) * 4;
        pack_words(L->bits, tile, (int64_t)n * D, words);
      } else {
        for (int32_t t = 0; t < n; t++) {
          uint8_t* row = c.codes + (((int64_t)b * H + h) * T + off + t) * R;
          kvqr_pack_row(L->bits, tile + (int64_t)t * D, D, row);
        }
      }
    }
  }
  free(col);
  free(gcodes);
  free(tile);
  return status;
}

int kvqr_quantize_block(const kvqr_layout* L, int32_t block, int32_t src_dtype,
                        const void* k_src, const void* v_src, kvqr_cache k_cache,
                        kvqr_cache v_cache) {
  if (kvqr_validate(L) != KVQR_OK) return KVQR_E_INVAL;
  if (L->pack_mode == 1) return KVQR_E_INVAL; /* one stream per (b, h): not block-writable */
  if (block < 0 || block >= L->n_blocks) return KVQR_E_INVAL;
  if (src_dtype != KVQR_F32 && src_dtype != KVQR_BF16) return KVQR_E_INVAL;
  if (!k_src || !v_src || !k_cache.codes || !k_cache.zero || !k_cache.scale || !v_cache.codes ||
      !v_cache.zero || !v_cache.scale)
    return KVQR_E_INVAL;
  int sk = quantize_one(L, block, src_dtype, k_src, k_cache);
  if (sk < 0) return sk;
  int sv = quantize_one(L, block, src_dtype, v_src, v_cache);
  if (sv < 0) return sv;
  return sk | sv;
}

/* ------------------------------------------------------------------------ */
/* dequantization: x_hat = code * s + z with one rounding                   */
/* ------------------------------------------------------------------------ */

static int32_t block_of_token(const kvqr_layout* L, int64_t t) {
  int64_t end = 0;
  for (int32_t k = 0; k < L->n_blocks; k++) {
    end += L->block_tokens[k];
    if (t < end) return k;
  }
  return -1;
}

/* dequantized rows [0, T) of one (b, h) into out[T][D] */
static void dequant_bh(const kvqr_layout* L, kvqr_cache c, int32_t b, int32_t h, int64_t T,
                       float* out) {
  const int32_t H = L->heads, D = L->head_dim, NB = L->n_blocks;
  const int64_t Tmax = kvqr_total_tokens(L, NB);
  const int32_t R = kvqr_row_bytes(L->bits, D);
  uint8_t* codes = (uint8_t*)malloc((size_t)D);
  for (int64_t t = 0; t < T; t++) {
    int32_t k = block_of_token(L, t);
    if (L->pack_mode == 2) { /* row t - off_k of block k's word stream */
      const int64_t W = kvqr_block_word_offset(L, NB);
      const uint8_t* words =
          c.codes + (((int64_t)b * H + h) * W + kvqr_block_word_offset(L, k)) * 4;
      unpack_words_at(L->bits, words, (t - kvqr_block_offset(L, k)) * D, D, codes);
    } else {
      const uint8_t* row = c.codes + (((int64_t)b * H + h) * Tmax + t) * R;
      kvqr_unpack_row(L->bits, row, D, codes);
    }
    for (int32_t d = 0; d < D; d++) {
      int64_t sidx = (((int64_t)b * H + h) * NB + k) * D + d;
      float z = kvqr_h2f(c.zero[sidx]);
      float s = kvqr_h2f(c.scale[sidx]);
      out[t * D + d] = fmaf((float)codes[d], s, z);
    }
  }
  free(codes);
}

int kvqr_dequantize(const kvqr_layout* L, int32_t n_filled, kvqr_cache c, float* out) {
  if (kvqr_validate(L) != KVQR_OK || L->pack_mode == 1) return KVQR_E_INVAL;
  if (n_filled < 0 || n_filled > L->n_blocks || !out) return KVQR_E_INVAL;
  const int32_t B = L->batch, H = L->heads, D = L->head_dim;
  const int64_t T = kvqr_total_tokens(L, n_filled);
  for (int32_t b = 0; b < B; b++)
    for (int32_t h = 0; h < H; h++)
      dequant_bh(L, c, b, h, T, out + (((int64_t)b * H + h) * T) * D);
  return KVQR_OK;
}

/* ------------------------------------------------------------------------ */
/* block-causal attention over the packed cache, binary64                   */
/* ------------------------------------------------------------------------ */

static void attend_one(int32_t D, int64_t T, const double* q, const float* kh, const float* vh,
                       double scale, double* o, double* sc) {
  double m = -INFINITY;
  for (int64_t t = 0; t < T; t++) {
    double acc = 0.0;
    for (int32_t d = 0; d < D; d++) acc += q[d] * (double)kh[t * D + d];
    sc[t] = scale * acc;
    if (sc[t] > m) m = sc[t];
  }
  double l = 0.0;
  for (int32_t d = 0; d < D; d++) o[d] = 0.0;
  for (int64_t t = 0; t < T; t++) {
    double p = exp(sc[t] - m);
    l += p;
    for (int32_t d = 0; d < D; d++) o[d] += p * (double)vh[t * D + d];
  }
  for (int32_t d = 0; d < D; d++) o[d] /= l;
}

static int attend_args_ok(const kvqr_layout* L, int32_t block, const uint16_t* q, kvqr_cache k,
                          kvqr_cache v) {
  if (kvqr_validate(L) != KVQR_OK || L->pack_mode == 1) return 0;
  if (block < 0 || block >= L->n_blocks || !q) return 0;
  if (!k.codes || !k.zero || !k.scale || !v.codes || !v.zero || !v.scale) return 0;
  return 1;
}

int kvqr_attend(const kvqr_layout* L, int32_t block, const uint16_t* q, kvqr_cache k,
                kvqr_cache v, double scale, float* out, int32_t b0, int32_t b1) {
  if (!attend_args_ok(L, block, q, k, v) || !out) return KVQR_E_INVAL;
  if (b0 < 0 || b1 > L->batch || b0 > b1) return KVQR_E_INVAL;
  const int32_t H = L->heads, D = L->head_dim;
  const int32_t n = L->block_tokens[block];
  const int64_t T = kvqr_total_tokens(L, block + 1); /* prefix of blocks 0..block */
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  float* kh = (float*)malloc(sizeof(float) * (size_t)(T * D));
  float* vh = (float*)malloc(sizeof(float) * (size_t)(T * D));
  double* sc = (double*)malloc(sizeof(double) * (size_t)T);
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  double* od = (double*)malloc(sizeof(double) * (size_t)D);
  for (int32_t b = b0; b < b1; b++) {
    for (int32_t h = 0; h < H; h++) {
      dequant_bh(L, k, b, h, T, kh);
      dequant_bh(L, v, b, h, T, vh);
      for (int32_t i = 0; i < n; i++) {
        int64_t base = (((int64_t)b * n + i) * H + h) * D; /* [b][i][h][d] */
        for (int32_t d = 0; d < D; d++) qd[d] = (double)bf16_to_f32(q[base + d]);
        attend_one(D, T, qd, kh, vh, scale, od, sc);
        for (int32_t d = 0; d < D; d++) out[base + d] = (float)od[d];
      }
    }
  }
  free(kh);
  free(vh);
  free(sc);
  free(qd);
  free(od);
  return KVQR_OK;
}

int kvqr_attend_row(const kvqr_layout* L, int32_t block, const uint16_t* q, kvqr_cache k,
                    kvqr_cache v, double scale, int32_t b, int32_t i, int32_t h,
                    double* out_row) {
  if (!attend_args_ok(L, block, q, k, v) || !out_row) return KVQR_E_INVAL;
  const int32_t H = L->heads, D = L->head_dim;
  const int32_t n = L->block_tokens[block];
  if (b < 0 || b >= L->batch || h < 0 || h >= H || i < 0 || i >= n) return KVQR_E_INVAL;
  const int64_t T = kvqr_total_tokens(L, block + 1);
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  float* kh = (float*)malloc(sizeof(float) * (size_t)(T * D));
  float* vh = (float*)malloc(sizeof(float) * (size_t)(T * D));
  double* sc = (double*)malloc(sizeof(double) * (size_t)T);
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  dequant_bh(L, k, b, h, T, kh);
  dequant_bh(L, v, b, h, T, vh);
  int64_t base = (((int64_t)b * n + i) * H + h) * D;
  for (int32_t d = 0; d < D; d++) qd[d] = (double)bf16_to_f32(q[base + d]);
  attend_one(D, T, qd, kh, vh, scale, out_row, sc);
  free(kh);
  free(vh);
  free(sc);
  free(qd);
  return KVQR_OK;
}

/* ------------------------------------------------------------------------ */
/* bytes held per (layer, K or V) once n_filled blocks are cached           */
/* ------------------------------------------------------------------------ */

int kvqr_bytes(const kvqr_layout* L, int32_t n_filled, uint64_t* code_bytes,
               uint64_t* stat_bytes) {
  if (kvqr_validate(L) != KVQR_OK) return KVQR_E_INVAL;
  if (n_filled < 0 || n_filled > L->n_blocks || !code_bytes || !stat_bytes) return KVQR_E_INVAL;
  uint64_t BH = (uint64_t)L->batch * (uint64_t)L->heads;
  uint64_t T = (uint64_t)kvqr_total_tokens(L, n_filled);
  if (L->pack_mode == 1) /* each (b, h) cache is one word-aligned stream of T*D codes */
    *code_bytes = BH * 4u * (uint64_t)kvqr_stream_words(L->bits, (int64_t)T * L->head_dim);
  else if (L->pack_mode == 2) /* one word-aligned stream per (b, h, block) */
    *code_bytes = BH * 4u * (uint64_t)kvqr_block_word_offset(L, n_filled);
  else
    *code_bytes = BH * T * (uint64_t)kvqr_row_bytes(L->bits, L->head_dim);
  /* one binary16 zero + one binary16 step per (block, channel) */
  *stat_bytes = BH * (uint64_t)n_filled * (uint64_t)L->head_dim * 4u;
  return KVQR_OK;
}
