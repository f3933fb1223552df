// kvq_internal.h -- shared device helpers and launch descriptors of the gfx950
// kernels behind include/kvq.h.  Internal to libkvq.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// binary16 helpers.  Directed rounding is built from the hardware's
// round-to-nearest-even conversion (v_cvt_f16_f32) followed by a one-ulp step
// when the nearest value lies on the wrong side of x.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ __forceinline__ uint16_t f2h_rne(float x) {
  return __half_as_ushort(__float2half_rn(x));
}

// next binary16 toward -inf / +inf of a non-NaN pattern
__device__ __forceinline__ uint16_t h_step_down(uint16_t h) {
  if (h == 0x0000) return 0x8001;
  return (h & 0x8000) ? (uint16_t)(h + 1) : (uint16_t)(h - 1);
}
__device__ __forceinline__ uint16_t h_step_up(uint16_t h) {
  if (h == 0x8000) return 0x0001;
  return (h & 0x8000) ? (uint16_t)(h - 1) : (uint16_t)(h + 1);
}

// largest binary16 <= x (x not NaN)
__device__ __forceinline__ uint16_t rd16(float x) {
  uint16_t h = f2h_rne(x);
  return (h2f(h) > x) ? h_step_down(h) : h;
}
// smallest binary16 >= x (x not NaN)
__device__ __forceinline__ uint16_t ru16(float x) {
  uint16_t h = f2h_rne(x);
  return (h2f(h) < x) ? h_step_up(h) : h;
}

// 3-input min / max on raw registers.  Written as instructions so the compiler
// adds no NaN-quieting canonicalization around them (inputs here are plain
// finite values or the caller has opted out of screening).
__device__ __forceinline__ float min3f(float a, float b, float c) {
  float d;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// ---------------------------------------------------------------------------
// launch descriptors
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Group statistics and code packing shared by the quantize kernel and the
// fused quantize-and-attend kernel (one definition, so both write identical
// bytes).
// ---------------------------------------------------------------------------

// zero = binary16 rounded down from the group minimum, step = binary16 rounded
// up from fp32(max - zero) / (2^b - 1), and the fp32 reciprocal of the step
// (0 for a constant group).  lo, hi: exact extremes with a zero extreme as +0.
struct GroupStats {
  uint16_t zb, sb;  // binary16 bit patterns
  float zf, inv;
};
template <bool CHECK>
__device__ __forceinline__ GroupStats group_stats(float lo, float hi, float levels, int& flags) {
  GroupStats g;
  lo = (lo == 0.0f) ? 0.0f : lo;
  hi = (hi == 0.0f) ? 0.0f : hi;
  if constexpr (CHECK) {
    if (!(lo >= -65504.0f) || !(hi <= 65504.0f)) flags |= KVQ_S_RANGE;
  }
  g.zb = rd16(lo);
  g.zf = h2f(g.zb);
  const float r = hi - g.zf;
  const float q = r / levels;
  g.sb = ru16(q);
  const float sf = h2f(g.sb);
  if constexpr (CHECK) {
    if (!(sf <= 65504.0f)) flags |= KVQ_S_RANGE;
  }
  g.inv = (sf > 0.0f) ? 1.0f / sf : 0.0f;
  return g;
}

template <int BITS>
struct PackMagic {
  // sum over the 8 codes of the exponent bits 0x4B000000 of (2^23 + code),
  // shifted to the code's position, modulo 2^32
  static constexpr uint32_t value() {
    uint32_t s = 0;
    for (int j = 0; j < 8; ++j) s += (0x4B000000u << (BITS * j));
    return s;
  }
};

// codes of 8 channel values, LSB-first in the low 8*BITS bits: clamp(rne((x -
// z) * inv), 0, 2^b - 1).  Adding 2^23 rounds half-to-even and leaves the
// integer in the low mantissa bits, which the shift-add collects directly.
template <int BITS>
__device__ __forceinline__ uint32_t pack_codes8(const float x[8], const float zf[8],
                                                const float inv[8]) {
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float t = x[j] - zf[j];
    const float u = t * inv[j];
    const float c = __builtin_amdgcn_fmed3f(u, 0.0f, LEVELS);
    const float f = c + 8388608.0f;  // 2^23
    acc += __float_as_uint(f) << (BITS * j);
  }
  return acc - PackMagic<BITS>::value();
}

// Code widths the GPU kernels are built for.  Rows of D codes take 8 * BITS
// bytes per 8-code chunk (BITS bytes); chunks of 2-, 4- and 8-bit codes sit on
// BITS-byte boundaries, 3-bit chunks straddle them.
template <int BITS>
constexpr bool kWidthBuilt = BITS == 2 || BITS == 3 || BITS == 4 || BITS == 8;

// Packed bits of one chunk of 8 codes, LSB-first: all of them in lo for up to 4
// bits per code; codes 0-3 in lo and 4-7 in hi for 8 bits.
struct Packed8 {
  uint32_t lo, hi;
};

template <int BITS>
__device__ __forceinline__ Packed8 pack_chunk(const float x[8], const float zf[8],
                                              const float inv[8]) {
  static_assert(kWidthBuilt<BITS>, "code width not built");
  if constexpr (BITS <= 4) {
    return Packed8{pack_codes8<BITS>(x, zf, inv), 0u};
  } else {
    constexpr float LEVELS = (float)((1 << BITS) - 1);
    uint32_t acc[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = (x[j] - zf[j]) * inv[j];
      const float f = __builtin_amdgcn_fmed3f(u, 0.0f, LEVELS) + 8388608.0f;  // 2^23: rne
      acc[j >> 2] += __float_as_uint(f) << (8 * (j & 3));
    }
    // of the four 0x4B000000 exponent words per half only the unshifted one
    // survives modulo 2^32
    return Packed8{acc[0] - 0x4B000000u, acc[1] - 0x4B000000u};
  }
}

// store one packed chunk: BITS bytes at dst (aligned to BITS bytes for 2, 4
// and 8 bits; byte stores for 3)
template <int BITS>
__device__ __forceinline__ void store_chunk(uint8_t* dst, const Packed8& v) {
  if constexpr (BITS == 2) {
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)v.lo;
  } else if constexpr (BITS == 4) {
    *reinterpret_cast<uint32_t*>(dst) = v.lo;
  } else if constexpr (BITS == 8) {
    *reinterpret_cast<uint2*>(dst) = uint2{v.lo, v.hi};
  } else {
    dst[0] = (uint8_t)v.lo;
    dst[1] = (uint8_t)(v.lo >> 8);
    dst[2] = (uint8_t)(v.lo >> 16);
  }
}

// Block-aligned 3-bit words: each (sequence, head, block) stream of n_k x D
// codes, row after row, in 32-bit words of ten codes (code k of a word at bits
// [3k, 3k + 3), the top two bits zero), every block from a fresh word.  Word w
// of a stream is bits [30 w, 30 w + 30) of the same codes packed densely (code
// i at bit 3 i), which is how the quantizers form it from their LDS staging.
// dense: 4-byte aligned, readable 8 bytes past the n_codes codes; codes past
// n_codes come out zero.
__device__ __forceinline__ uint32_t word_from_dense3(const uint8_t* dense, int w, int n_codes) {
  const int bit = 30 * w;
  const uint32_t* d32 = reinterpret_cast<const uint32_t*>(dense);
  const uint64_t both = (uint64_t)d32[bit >> 5] | ((uint64_t)d32[(bit >> 5) + 1] << 32);
  uint32_t v = (uint32_t)(both >> (bit & 31)) & 0x3FFFFFFFu;
  const int left = n_codes - 10 * w;
  if (left < 10) v &= (1u << (3 * left)) - 1u;
  return v;
}

struct QuantParams {
  const void* src[2];  // K, V: [B][n][H][D]
  uint8_t* codes[2];   // [B][H][T][R]; block-aligned words: [B][H][bh_words] words
  uint16_t* zero[2];   // [B][H][NB][D]
  uint16_t* scale[2];
  int32_t* status;     // nullable
  int64_t n_tiles;     // 2 * B * H
  int64_t T;           // rows per (b, h) in the cache
  int64_t off;         // first row of the block
  int32_t BH, H, n, NB, block, R;
  int32_t gs;          // threads per (tensor, b, h) tile
  int32_t rpt;         // rows per thread per pass
  int32_t word_layout; // block-aligned 3-bit words (then R is still the dense row size)
  int64_t bh_words;    // words per (b, h) cache (word layout)
  int64_t word_off;    // first word of the block in each (b, h) cache (word layout)
};

// the block's packed codes in the cache of (tensor kv, b*H + h)
__device__ __forceinline__ uint8_t* block_codes(const QuantParams& p, int kv, int64_t bh) {
  return p.word_layout ? p.codes[kv] + (bh * p.bh_words + p.word_off) * 4
                       : p.codes[kv] + (bh * p.T + p.off) * p.R;
}

// a dispatch holds at most 2^32 - 1 work-items
inline bool dispatch_fits(int64_t groups, int threads) {
  return groups * threads <= (int64_t)UINT32_MAX;
}

// The chunk-per-thread kernels (pack, unpack, dequantize) are launched in
// pieces of at most kMaxLaunchWGs workgroups; chunk0 is a piece's first chunk.
constexpr int64_t kMaxLaunchWGs = (int64_t)1 << 22;

struct PackParams {
  const uint8_t* codes;
  uint8_t* dst;
  int64_t n_rows, dst_stride, n_chunks;
  int64_t chunk0;
  int32_t row_len, bits, chunks_per_row, R;
  int32_t contiguous;  // dst rows back to back and row_len % 8 == 0
};

struct UnpackParams {
  const uint8_t* src;
  uint8_t* codes;
  int64_t n_rows, src_stride, n_chunks;
  int64_t chunk0;
  int32_t row_len, bits, chunks_per_row;
};

struct DequantParams {
  const uint8_t* codes;
  const uint16_t* zero;
  const uint16_t* scale;
  float* out;
  int64_t T_cache, T_out, n_chunks;
  int64_t chunk0;
  int32_t H, D, bits, R, NB;
  int32_t n_filled;
  int32_t block_end[KVQ_MAX_BLOCKS];  // exclusive prefix ends
  int32_t word_layout;                // block-aligned 3-bit words
  int64_t bh_words;
  int32_t block_pad[KVQ_MAX_BLOCKS];  // word layout: padding codes before block k
};

// Quantize-and-pack side of the fused quantize + attend launch: block `block`
// of K and V ([B][n][H][D]) goes into cache rows off .. off + n - 1 and stats
// slot `block` before the block's queries attend.
struct FuseParams {
  const void* src[2];  // K, V
  uint8_t* codes[2];   // writable views of the caches the attention reads
  uint16_t* zero[2];
  uint16_t* scale[2];
  int32_t* status;  // nullable
  int64_t off;
  int32_t block;
  int64_t word_off;  // block-aligned words: the block's first word
};

struct AttendParams {
  const uint16_t* q;  // [B][n][H][D] bf16
  const uint8_t* kcodes;
  const uint16_t* kzero;
  const uint16_t* kscale;
  const uint8_t* vcodes;
  const uint16_t* vzero;
  const uint16_t* vscale;
  float* out;         // [B][n][H][D]
  int64_t T_cache;    // rows per (b, h) in the cache
  int32_t B, H, n, NB, R;
  int32_t n_prefix;   // keys attended: off_k + n_k
  int32_t n_kblocks;  // blocks attended: k + 1
  int32_t q_tiles;    // query tiles per (b, h)
  float scale_log2;   // softmax scale * log2(e)
  int32_t block_end[KVQ_MAX_BLOCKS];
  // Block-aligned 3-bit words: each (b, h) cache holds bh_words words, the
  // prefix's blocks prefix_words of them; code (t, d) of a key t in block k
  // is code t D + d + block_pad[k] of the (b, h) stream, block_pad[k] = 10 W_k
  // - D off_k being the padding codes that the word boundaries of blocks
  // 0..k-1 add (W_k: words before block k).
  int32_t word_layout;
  int32_t prefix_words;
  int64_t bh_words;
  int32_t block_pad[KVQ_MAX_BLOCKS];
  FuseParams fz;  // used by the fused launch only
  // key-range launch only: ranges per query tile and the partials'
  // workspace, ws_o [splits][rows][D] and ws_ml [splits][rows][2] (rows = B n H)
  int32_t splits;
  int64_t ws_rows;
  float* ws_o;
  float* ws_ml;
};

hipError_t launch_quantize(const QuantParams& p, int head_dim, int bits, bool f32src,
                           hipStream_t s);
hipError_t launch_pack(const PackParams& p, hipStream_t s);
hipError_t launch_unpack(const UnpackParams& p, hipStream_t s);
// word-aligned stream of n codes (pack_mode 1)
hipError_t launch_pack_words(const uint8_t* codes, uint8_t* dst, int64_t n, int bits,
                             hipStream_t s);
hipError_t launch_unpack_words(const uint8_t* src, uint8_t* codes, int64_t n, int bits,
                               hipStream_t s);
hipError_t launch_dequantize(const DequantParams& p, hipStream_t s);
hipError_t launch_attend(const AttendParams& p, int head_dim, int bits, hipStream_t s);
// attention of blocks of more than 128 queries with the key prefix cut into
// p.splits ranges (p.splits >= 2), then the merge of the partials
hipError_t launch_attend_split(const AttendParams& p, int head_dim, int bits, hipStream_t s);
// quantize block k (q) then attend its queries (a): one launch where a fused
// kernel covers the shape, else the two launches in order
hipError_t launch_quantize_attend(const QuantParams& q, const AttendParams& a, int head_dim,
                                  int bits, bool f32src, hipStream_t s);
hipError_t launch_stream_copy(const void* src, void* dst, uint64_t n, hipStream_t s);
hipError_t launch_stream_read(const void* src, uint64_t n, uint32_t* sink, hipStream_t s);

}  // namespace kvq
