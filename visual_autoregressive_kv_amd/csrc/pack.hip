// pack.hip -- standalone bit-packing (kvq_pack) plus the test-only unpack and
// dequantize kernels and the plain streaming copy used to measure HBM peak.
//
// Packing follows the cache-row layout of the fused quantizer: a row of codes is
// an LSB-first bit stream, code d at stream bits [bits*d, bits*d + bits); eight
// codes therefore fill exactly `bits` bytes.  One thread packs one 8-code chunk
// (one 64-bit load of 8 code bytes); when destination rows are back to back the
// workgroup's bytes are one contiguous span, staged in LDS and written with
// 128-bit stores, otherwise each chunk is written bytewise in place.
#include "kvq_internal.h"

#include <algorithm>

namespace kvq {
namespace {

constexpr int kWG = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint64_t pack8(uint64_t codes8, int bits, int count) {
  const uint32_t mask = (1u << bits) - 1u;
  uint64_t w = 0;
  for (int j = 0; j < count; ++j) w |= (uint64_t)((codes8 >> (8 * j)) & mask) << (bits * j);
  return w;
}

__global__ __launch_bounds__(kWG) void pack_kernel(PackParams p) {
  __shared__ __align__(16) uint8_t stage[kWG * 8 + 32];
  const int64_t first = p.chunk0 + (int64_t)blockIdx.x * kWG;  // the workgroup's first chunk
  const int64_t chunk = first + threadIdx.x;
  const bool ok = chunk < p.n_chunks;
  const int64_t row = ok ? chunk / p.chunks_per_row : 0;
  const int c = ok ? (int)(chunk - row * p.chunks_per_row) : 0;
  const int count = min(8, p.row_len - 8 * c);
  uint64_t w = 0;
  if (ok) {
    const uint8_t* src = p.codes + row * p.row_len + 8 * c;
    uint64_t codes8 = 0;
    if (count == 8 && ((reinterpret_cast<uintptr_t>(src) & 7) == 0)) {
      codes8 = *reinterpret_cast<const uint64_t*>(src);
    } else {
      for (int j = 0; j < count; ++j) codes8 |= (uint64_t)src[j] << (8 * j);
    }
    w = pack8(codes8, p.bits, count);
  }
  const int nb = ok ? (p.bits * count + 7) / 8 : 0;
  if (p.contiguous) {
    // the workgroup's chunks map to one contiguous span of dst
    const int64_t last = min(first + kWG, p.n_chunks);
    uint8_t* dst = p.dst + first * p.bits;
    const int nbytes = (int)((last - first) * p.bits);
    const int mis = (int)(reinterpret_cast<uintptr_t>(dst) & 15);
    uint8_t* sp = stage + mis + (int)(chunk - first) * p.bits;
    for (int j = 0; j < nb; ++j) sp[j] = (uint8_t)(w >> (8 * j));
    __syncthreads();
    const int head = min((16 - mis) & 15, nbytes);
    const int body = (nbytes - head) >> 4;
    const int tail = nbytes - head - (body << 4);
    const uint8_t* s0 = stage + mis;
    for (int k = threadIdx.x; k < body; k += kWG)
      *reinterpret_cast<u32x4*>(dst + head + 16 * k) =
          *reinterpret_cast<const u32x4*>(s0 + head + 16 * k);
    if ((int)threadIdx.x < head) dst[threadIdx.x] = s0[threadIdx.x];
    if ((int)threadIdx.x < tail) dst[head + 16 * body + threadIdx.x] = s0[head + 16 * body + threadIdx.x];
  } else if (ok) {
    uint8_t* dst = p.dst + row * p.dst_stride + (int64_t)c * p.bits;
    for (int j = 0; j < nb; ++j) dst[j] = (uint8_t)(w >> (8 * j));
  }
}

__global__ __launch_bounds__(kWG) void unpack_kernel(UnpackParams p) {
  const int64_t chunk = p.chunk0 + (int64_t)blockIdx.x * kWG + threadIdx.x;
  if (chunk >= p.n_chunks) return;
  const int64_t row = chunk / p.chunks_per_row;
  const int c = (int)(chunk - row * p.chunks_per_row);
  const int count = min(8, p.row_len - 8 * c);
  const int nb = (p.bits * count + 7) / 8;
  const uint8_t* src = p.src + row * p.src_stride + (int64_t)c * p.bits;
  uint64_t w = 0;
  for (int j = 0; j < nb; ++j) w |= (uint64_t)src[j] << (8 * j);
  const uint32_t mask = (1u << p.bits) - 1u;
  uint8_t* out = p.codes + row * p.row_len + 8 * c;
  for (int j = 0; j < count; ++j) out[j] = (uint8_t)((w >> (p.bits * j)) & mask);
}

// one thread = 8 channels of one cached token
__global__ __launch_bounds__(kWG) void dequant_kernel(DequantParams p) {
  const int64_t chunk = p.chunk0 + (int64_t)blockIdx.x * kWG + threadIdx.x;
  if (chunk >= p.n_chunks) return;
  const int cpr = p.D / 8;
  const int64_t rowid = chunk / cpr;  // (b*H + h) * T_out + t
  const int cg = (int)(chunk - rowid * cpr);
  const int64_t bh = rowid / p.T_out;
  const int64_t t = rowid - bh * p.T_out;
  int k = 0;
  while (k < p.n_filled - 1 && t >= p.block_end[k]) ++k;
  uint64_t w = 0;
  if (p.word_layout) {
    // block-aligned 3-bit words: the chunk starts at code gi of the (b, h)
    // stream and runs into the next word when fewer than 8 codes are left
    const uint32_t gi = (uint32_t)(t * p.D + 8 * cg + p.block_pad[k]);
    const uint32_t wi = gi / 10u;
    const int r = (int)(gi - 10u * wi);
    const uint32_t* words = reinterpret_cast<const uint32_t*>(p.codes) + bh * p.bh_words;
    w = words[wi] >> (3 * r);
    if (r > 2) w |= (uint64_t)words[wi + 1] << (30 - 3 * r);
  } else {
    const uint8_t* row = p.codes + (bh * p.T_cache + t) * p.R + (int64_t)cg * p.bits;
    for (int j = 0; j < p.bits; ++j) w |= (uint64_t)row[j] << (8 * j);
  }
  const uint32_t mask = (1u << p.bits) - 1u;
  const int64_t so = (bh * p.NB + k) * p.D + 8 * cg;
  float* out = p.out + rowid * p.D + 8 * cg;
  for (int j = 0; j < 8; ++j) {
    const float code = (float)((w >> (p.bits * j)) & mask);
    out[j] = __builtin_fmaf(code, h2f(p.scale[so + j]), h2f(p.zero[so + j]));
  }
}

// grid-stride 16-byte copy, 4 loads in flight per thread
__global__ __launch_bounds__(kWG) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * kWG;
  uint64_t i = (uint64_t)blockIdx.x * kWG + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4 a = __builtin_nontemporal_load(src + i);
    u32x4 b = __builtin_nontemporal_load(src + i + stride);
    u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Read-only stream: every 16-byte chunk is loaded once (4 per thread in
// flight, non-persistent grid); the loaded words are folded with xor and only
// a result equal to a fixed pattern (never in practice) is stored, so the
// loads cannot be dropped and almost nothing is written.
__global__ __launch_bounds__(kWG) void stream_read_kernel(const u32x4* __restrict__ src,
                                                         uint32_t* __restrict__ sink, uint64_t n16) {
  const uint64_t i0 = (uint64_t)blockIdx.x * kWG * 4 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t i = i0 + (uint64_t)k * kWG;
    if (i < n16) acc ^= __builtin_nontemporal_load(src + i);
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

// Word-aligned stream (pack_mode 1): word w holds codes w*cpw .. w*cpw + cpw - 1
// of the stream, cpw = floor(32 / bits), low bits first; one thread per word
// reads its codes (one per byte) and writes one 32-bit word.
__global__ __launch_bounds__(256) void pack_words_kernel(const uint8_t* __restrict__ codes,
                                                         uint32_t* __restrict__ dst, int64_t n,
                                                         int64_t words, int bits) {
  const int cpw = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i0 = w * cpw;
    uint32_t word = 0;
    for (int k = 0; k < cpw; ++k)
      if (i0 + k < n) word |= ((uint32_t)codes[i0 + k] & mask) << (bits * k);
    dst[w] = word;
  }
}

__global__ __launch_bounds__(256) void unpack_words_kernel(const uint32_t* __restrict__ src,
                                                           uint8_t* __restrict__ codes, int64_t n,
                                                           int64_t words, int bits) {
  const int cpw = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t word = src[w];
    const int64_t i0 = w * cpw;
    for (int k = 0; k < cpw; ++k)
      if (i0 + k < n) codes[i0 + k] = (uint8_t)((word >> (bits * k)) & mask);
  }
}

// one launch per piece of at most kMaxLaunchWGs workgroups, so a grid never
// exceeds the 32-bit work-item count of a dispatch
template <typename Params>
hipError_t launch_pieces(void (*kernel)(Params), const Params& p, hipStream_t s) {
  const int64_t wgs = (p.n_chunks + kWG - 1) / kWG;
  for (int64_t w0 = 0; w0 < wgs; w0 += kMaxLaunchWGs) {
    Params a = p;
    a.chunk0 = w0 * kWG;
    hipLaunchKernelGGL(kernel, dim3((unsigned)std::min(kMaxLaunchWGs, wgs - w0)), dim3(kWG), 0, s,
                       a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_pack(const PackParams& p, hipStream_t s) { return launch_pieces(pack_kernel, p, s); }

hipError_t launch_unpack(const UnpackParams& p, hipStream_t s) {
  return launch_pieces(unpack_kernel, p, s);
}

hipError_t launch_dequantize(const DequantParams& p, hipStream_t s) {
  return launch_pieces(dequant_kernel, p, s);
}

hipError_t launch_pack_words(const uint8_t* codes, uint8_t* dst, int64_t n, int bits,
                             hipStream_t s) {
  const int64_t words = (n + 32 / bits - 1) / (32 / bits);
  const int64_t grid = std::min<int64_t>((words + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_words_kernel, dim3((unsigned)grid), dim3(256), 0, s, codes,
                     reinterpret_cast<uint32_t*>(dst), n, words, bits);
  return hipGetLastError();
}

hipError_t launch_unpack_words(const uint8_t* src, uint8_t* codes, int64_t n, int bits,
                               hipStream_t s) {
  const int64_t words = (n + 32 / bits - 1) / (32 / bits);
  const int64_t grid = std::min<int64_t>((words + 255) / 256, 65536);
  hipLaunchKernelGGL(unpack_words_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(src), codes, n, words, bits);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, uint64_t n, hipStream_t s) {
  const uint64_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned grid = 256 * 16;  // 16 workgroups per CU
  hipLaunchKernelGGL(stream_copy_kernel, dim3(grid), dim3(kWG), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, uint64_t n, uint32_t* sink, hipStream_t s) {
  const uint64_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  const uint64_t groups = (n16 + 4 * kWG - 1) / (4 * kWG);
  if (!dispatch_fits((int64_t)groups, kWG)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)groups), dim3(kWG), 0, s,
                     static_cast<const u32x4*>(src), sink, n16);
  return hipGetLastError();
}

}  // namespace kvq
