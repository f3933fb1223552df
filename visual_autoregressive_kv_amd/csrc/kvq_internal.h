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

struct QuantParams {
  const void* src[2];  // K, V: [B][n][H][D]
  uint8_t* codes[2];   // [B][H][T][R]
  uint16_t* zero[2];   // [B][H][NB][D]
  uint16_t* scale[2];
  int32_t* status;     // nullable
  int64_t n_tiles;     // 2 * B * H
  int64_t T;           // rows per (b, h) in the cache
  int64_t off;         // first row of the block
  int32_t BH, H, n, NB, block, R;
  int32_t gs;          // threads per (tensor, b, h) tile
  int32_t rpt;         // rows per thread per pass
};

struct PackParams {
  const uint8_t* codes;
  uint8_t* dst;
  int64_t n_rows, dst_stride, n_chunks;
  int32_t row_len, bits, chunks_per_row, R;
  int32_t contiguous;  // dst rows back to back and row_len % 8 == 0
};

struct UnpackParams {
  const uint8_t* src;
  uint8_t* codes;
  int64_t n_rows, src_stride, n_chunks;
  int32_t row_len, bits, chunks_per_row;
};

struct DequantParams {
  const uint8_t* codes;
  const uint16_t* zero;
  const uint16_t* scale;
  float* out;
  int64_t T_cache, T_out, n_chunks;
  int32_t H, D, bits, R, NB;
  int32_t n_filled;
  int32_t block_end[KVQ_MAX_BLOCKS];  // exclusive prefix ends
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
  int32_t stats_in_lds;  // prefix statistics staged in LDS as fp32
  int32_t block_end[KVQ_MAX_BLOCKS];
};

hipError_t launch_quantize(const QuantParams& p, int head_dim, int bits, bool f32src,
                           hipStream_t s);
hipError_t launch_pack(const PackParams& p, hipStream_t s);
hipError_t launch_unpack(const UnpackParams& p, hipStream_t s);
hipError_t launch_dequantize(const DequantParams& p, hipStream_t s);
hipError_t launch_attend(const AttendParams& p, int head_dim, int bits, hipStream_t s);
hipError_t launch_stream_copy(const void* src, void* dst, uint64_t n, hipStream_t s);

}  // namespace kvq
