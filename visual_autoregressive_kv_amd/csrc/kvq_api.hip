// kvq_api.hip -- the extern "C" boundary of libkvq (declared in include/kvq.h).
// Validates every argument on the host, computes the layout arithmetic and
// launches the gfx950 kernels on the caller's stream.  Allocates nothing.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kvq_internal.h"

namespace {

using namespace kvq;

constexpr int64_t kMaxElems = (int64_t)1 << 46;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int32_t row_bytes(int32_t bits, int32_t d) { return (bits * d + 7) / 8; }

int validate_layout(const kvq_layout* L) {
  if (!L) return KVQ_E_INVAL;
  if (L->batch < 1 || L->heads < 1) return KVQ_E_INVAL;
  if (L->head_dim < 8 || L->head_dim % 8 != 0) return KVQ_E_INVAL;
  if (L->bits < 1 || L->bits > 8) return KVQ_E_INVAL;
  if (L->n_blocks < 1 || L->n_blocks > KVQ_MAX_BLOCKS) return KVQ_E_INVAL;
  if (L->pack_mode < 0 || L->pack_mode > 2) return KVQ_E_INVAL;
  int64_t T = 0;
  for (int i = 0; i < L->n_blocks; ++i) {
    if (L->block_tokens[i] < 1) return KVQ_E_INVAL;
    T += L->block_tokens[i];
  }
  if (T > INT32_MAX) return KVQ_E_INVAL;
  const int64_t bh = (int64_t)L->batch * L->heads;
  if (bh > INT32_MAX / 2) return KVQ_E_INVAL;
  if (bh * T * L->head_dim > kMaxElems) return KVQ_E_INVAL;
  return KVQ_OK;
}

// Block-aligned words (pack_mode 2): words of blocks 0..block-1 in one (b, h)
// cache, each block's n_k * D codes in ceil(n_k * D / floor(32 / bits)) words.
int64_t words_before(const kvq_layout* L, int32_t block) {
  const int64_t cpw = 32 / L->bits;
  int64_t w = 0;
  for (int i = 0; i < block; ++i) w += ((int64_t)L->block_tokens[i] * L->head_dim + cpw - 1) / cpw;
  return w;
}

// pack_mode 2 with a width whose codes do not fill 32 bits (3 on the GPU): the
// kernels' word layout.  With 2-, 4- and 8-bit codes and head_dim a multiple of
// 64 every block's stream fills whole words and equals its dense rows byte for
// byte, so those run the dense-row kernels unchanged.
bool word_layout(const kvq_layout* L) { return L->pack_mode == 2 && 32 % L->bits != 0; }

// kernels are built for 2/3/4/8-bit codes and head_dim 64/128
int gpu_supported(const kvq_layout* L) {
  if (L->pack_mode == 1) return KVQ_E_UNSUPPORTED;  // one stream per (b, h): not block-writable
  if (L->bits != 2 && L->bits != 3 && L->bits != 4 && L->bits != 8) return KVQ_E_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return KVQ_E_UNSUPPORTED;
  // one (b, h)'s codes are addressed with 32-bit buffer offsets; block-aligned
  // words also with 32-bit code indices (plus a few tiles past the prefix)
  int64_t T = 0;
  for (int i = 0; i < L->n_blocks; ++i) T += L->block_tokens[i];
  if (T * row_bytes(L->bits, L->head_dim) > INT32_MAX) return KVQ_E_UNSUPPORTED;
  if (word_layout(L)) {
    const int64_t W = words_before(L, L->n_blocks) + 4096;
    if (4 * W > INT32_MAX || 10 * W > (int64_t)UINT32_MAX) return KVQ_E_UNSUPPORTED;
  }
  return KVQ_OK;
}

// Sequences x heads per decode call.  Below this bound every quantize and
// attention launch of a call that fits in HBM stays under 2^32 work-items per
// dispatch (the widest per pair, the small-block attention, takes 64).
constexpr int64_t kMaxDecodePairs = (int64_t)1 << 25;

int decode_pairs_ok(const kvq_layout* L) {
  return (int64_t)L->batch * L->heads < kMaxDecodePairs ? KVQ_OK : KVQ_E_UNSUPPORTED;
}

int64_t offset_of(const kvq_layout* L, int32_t block) {
  int64_t off = 0;
  for (int i = 0; i < block; ++i) off += L->block_tokens[i];
  return off;
}

int cache_ok(const kvq_cache& c) {
  return c.codes && c.zero && c.scale && aligned16(c.codes) && aligned16(c.zero) &&
         aligned16(c.scale);
}
int cache_ok(const kvq_cache_const& c) {
  return c.codes && c.zero && c.scale && aligned16(c.codes) && aligned16(c.zero) &&
         aligned16(c.scale);
}

// KVQ_DEBUG=1 in the environment: after every launch the call synchronizes
// its stream (unless the stream is being captured into a graph) and checks
// hipGetLastError, so a device fault or launch error is reported by the call
// that caused it, on stderr and as KVQ_E_DEVICE.  Off by default.
bool debug_mode() {
  static const bool on = [] {
    const char* v = getenv("KVQ_DEBUG");
    return v && v[0] && strcmp(v, "0") != 0;
  }();
  return on;
}

int device_status(hipError_t e, hipStream_t stream, const char* call) {
  if (e != hipSuccess) {
    if (debug_mode()) fprintf(stderr, "kvq: %s: launch failed: %s\n", call, hipGetErrorString(e));
    return KVQ_E_DEVICE;
  }
  if (debug_mode()) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) {
      hipError_t s = hipStreamSynchronize(stream);
      if (s == hipSuccess) s = hipGetLastError();
      if (s != hipSuccess) {
        fprintf(stderr, "kvq: %s: device error after the launch: %s\n", call,
                hipGetErrorString(s));
        return KVQ_E_DEVICE;
      }
    }
  }
  return KVQ_OK;
}

// threads per (tensor, b, h) tile and rows per thread for a block of n rows:
// the smallest power-of-two group (>= one row of chunks) that covers the block
// with at most 8 rows per thread; larger blocks stream in passes of 256 x 8
// (256 x 5 for block-aligned words, so that each pass starts on a word)
void pick_tiling(int n, int d, bool words, int32_t* gs, int32_t* rpt) {
  const int cpr = d / 8;
  for (int g = cpr; g <= 256; g <<= 1) {
    const int rps = g / cpr;
    const int r = (n + rps - 1) / rps;
    if (r <= 8) {
      *gs = g;
      *rpt = r;
      return;
    }
  }
  *gs = 256;
  *rpt = words ? 5 : 8;
}

// argument checks and launch descriptor of kvq_quantize_block
int make_quant_params(const kvq_layout* layout, int32_t block, int32_t src_dtype,
                      const void* k_src, const void* v_src, kvq_cache k_cache, kvq_cache v_cache,
                      int32_t* status_dev, QuantParams* out) {
  if (validate_layout(layout) != KVQ_OK) return KVQ_E_INVAL;
  if (block < 0 || block >= layout->n_blocks) return KVQ_E_INVAL;
  if (src_dtype != KVQ_F32 && src_dtype != KVQ_BF16) return KVQ_E_INVAL;
  if (!k_src || !v_src || !aligned16(k_src) || !aligned16(v_src)) return KVQ_E_INVAL;
  if (!cache_ok(k_cache) || !cache_ok(v_cache)) return KVQ_E_INVAL;
  if (status_dev && (reinterpret_cast<uintptr_t>(status_dev) & 3)) return KVQ_E_INVAL;
  int sup = gpu_supported(layout);
  if (sup == KVQ_OK) sup = decode_pairs_ok(layout);
  if (sup != KVQ_OK) return sup;
  QuantParams& p = *out;
  memset(&p, 0, sizeof(p));
  p.src[0] = k_src;
  p.src[1] = v_src;
  p.codes[0] = k_cache.codes;
  p.codes[1] = v_cache.codes;
  p.zero[0] = k_cache.zero;
  p.zero[1] = v_cache.zero;
  p.scale[0] = k_cache.scale;
  p.scale[1] = v_cache.scale;
  p.status = status_dev;
  p.BH = layout->batch * layout->heads;
  p.n_tiles = 2 * (int64_t)p.BH;
  p.H = layout->heads;
  p.n = layout->block_tokens[block];
  p.NB = layout->n_blocks;
  p.block = block;
  p.R = row_bytes(layout->bits, layout->head_dim);
  p.T = offset_of(layout, layout->n_blocks);
  p.off = offset_of(layout, block);
  p.word_layout = word_layout(layout);
  if (p.word_layout) {
    p.bh_words = words_before(layout, layout->n_blocks);
    p.word_off = words_before(layout, block);
  }
  pick_tiling(p.n, layout->head_dim, p.word_layout, &p.gs, &p.rpt);
  return KVQ_OK;
}

// argument checks and launch descriptor of kvq_attend_packed
int make_attend_params(const kvq_layout* layout, int32_t block, const uint16_t* q_bf16,
                       kvq_cache_const k_cache, kvq_cache_const v_cache, float scale,
                       float* out, AttendParams* dst) {
  if (validate_layout(layout) != KVQ_OK) return KVQ_E_INVAL;
  if (block < 0 || block >= layout->n_blocks) return KVQ_E_INVAL;
  if (!q_bf16 || !out || !aligned16(q_bf16) || !aligned16(out)) return KVQ_E_INVAL;
  if (!cache_ok(k_cache) || !cache_ok(v_cache)) return KVQ_E_INVAL;
  if (!(scale == scale) || isinf(scale)) return KVQ_E_INVAL;
  int sup = gpu_supported(layout);
  if (sup == KVQ_OK) sup = decode_pairs_ok(layout);
  if (sup != KVQ_OK) return sup;
  AttendParams& p = *dst;
  memset(&p, 0, sizeof(p));
  p.q = q_bf16;
  p.kcodes = k_cache.codes;
  p.kzero = k_cache.zero;
  p.kscale = k_cache.scale;
  p.vcodes = v_cache.codes;
  p.vzero = v_cache.zero;
  p.vscale = v_cache.scale;
  p.out = out;
  p.T_cache = offset_of(layout, layout->n_blocks);
  p.B = layout->batch;
  p.H = layout->heads;
  p.n = layout->block_tokens[block];
  p.NB = layout->n_blocks;
  p.R = row_bytes(layout->bits, layout->head_dim);
  p.n_prefix = (int32_t)offset_of(layout, block + 1);
  p.n_kblocks = block + 1;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)layout->head_dim);
  p.scale_log2 = (float)(sc * 1.4426950408889634);
  int64_t e = 0;
  for (int i = 0; i < layout->n_blocks; ++i) {
    e += layout->block_tokens[i];
    p.block_end[i] = (int32_t)e;
  }
  p.word_layout = word_layout(layout);
  if (p.word_layout) {
    const int64_t cpw = 32 / layout->bits;
    p.bh_words = words_before(layout, layout->n_blocks);
    p.prefix_words = (int32_t)words_before(layout, block + 1);
    for (int i = 0; i < layout->n_blocks; ++i)
      p.block_pad[i] =
          (int32_t)(cpw * words_before(layout, i) - layout->head_dim * offset_of(layout, i));
  }
  return KVQ_OK;
}

// Key ranges per query tile of kvq_attend_packed_split: enough workgroups for
// about four per CU of the 256 on a gfx950 device, at least 16 key tiles (512
// keys) per range, at most max_splits.  Blocks of at most 128 queries run the
// kernels without ranges.  Four per CU measured best on the next-frame video
// shape (40 heads x 1560 queries, 280 query tiles: 4 ranges), against 2, 3, 5,
// 6, 8 and 16: every range re-reads the queries and writes a partial output.
constexpr int32_t kMaxSplits = 64;
constexpr int64_t kSplitTargetWGs = 4 * 256;
constexpr int64_t kMinSplitTiles = 16;

int32_t pick_splits(const AttendParams& p, int32_t max_splits) {
  if (p.n <= 128) return 1;
  const int64_t wgs = (int64_t)p.B * p.H * ((p.n + 255) / 256);
  const int64_t tiles = ((int64_t)p.n_prefix + 31) / 32;
  int64_t sp = (kSplitTargetWGs + wgs - 1) / wgs;
  sp = std::min<int64_t>(sp, tiles / kMinSplitTiles);
  sp = std::min<int64_t>(sp, max_splits);
  return (int32_t)std::max<int64_t>(sp, 1);
}

// partial outputs (head_dim floats) plus (max, denominator) per range and row
uint64_t split_workspace_bytes(const kvq_layout* L, int32_t block, int32_t splits) {
  const uint64_t rows = (uint64_t)L->batch * (uint64_t)L->block_tokens[block] * (uint64_t)L->heads;
  return (uint64_t)splits * rows * ((uint64_t)L->head_dim + 2u) * 4u;
}

// Static scratch of kvq_attend_packed_split_noalloc.  In host code `scratch`
// is only a stand-in for the symbol: each GPU holds its own copy at its own
// address, looked up once per device (with that device current) and kept in
// scratch_ptr; kernels only ever see that address.
__device__ __align__(256) uint8_t scratch[KVQ_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// device address of the current GPU's scratch array, or nullptr on failure
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}

kvq_cache_const const_view(kvq_cache c) {
  kvq_cache_const r;
  r.codes = c.codes;
  r.zero = c.zero;
  r.scale = c.scale;
  return r;
}

}  // namespace

extern "C" {

const char* kvq_version(void) { return "kvq 0.1 (gfx950)"; }

int kvq_bytes(const kvq_layout* layout, int32_t n_filled, uint64_t* code_bytes,
              uint64_t* stat_bytes) {
  if (validate_layout(layout) != KVQ_OK) return KVQ_E_INVAL;
  if (n_filled < 0 || n_filled > layout->n_blocks || !code_bytes || !stat_bytes)
    return KVQ_E_INVAL;
  const uint64_t bh = (uint64_t)layout->batch * (uint64_t)layout->heads;
  const uint64_t T = (uint64_t)offset_of(layout, n_filled);
  if (layout->pack_mode == 1) {  // one word-aligned stream of T*D codes per (b, h)
    const uint64_t cpw = 32u / (uint64_t)layout->bits;
    const uint64_t n = T * (uint64_t)layout->head_dim;
    *code_bytes = bh * 4u * ((n + cpw - 1) / cpw);
  } else if (layout->pack_mode == 2) {  // one word-aligned stream per (b, h, block)
    *code_bytes = bh * 4u * (uint64_t)words_before(layout, n_filled);
  } else {
    *code_bytes = bh * T * (uint64_t)row_bytes(layout->bits, layout->head_dim);
  }
  *stat_bytes = bh * (uint64_t)n_filled * (uint64_t)layout->head_dim * 4u;
  return KVQ_OK;
}

int kvq_quantize_block(const kvq_layout* layout, int32_t block, int32_t src_dtype,
                       const void* k_src, const void* v_src, kvq_cache k_cache,
                       kvq_cache v_cache, int32_t* status_dev, hipStream_t stream) {
  QuantParams p;
  const int rc = make_quant_params(layout, block, src_dtype, k_src, v_src, k_cache, v_cache,
                                   status_dev, &p);
  if (rc != KVQ_OK) return rc;
  return device_status(
      launch_quantize(p, layout->head_dim, layout->bits, src_dtype == KVQ_F32, stream), stream,
      "kvq_quantize_block");
}

int kvq_pack(int32_t bits, int32_t pack_mode, const uint8_t* codes, int64_t n_rows,
             int32_t row_len, uint8_t* dst, int64_t dst_row_stride, hipStream_t stream) {
  if (bits < 1 || bits > 8 || n_rows < 0 || row_len < 1) return KVQ_E_INVAL;
  if (pack_mode == 1) {  // one word-aligned stream; no row stride
    if (dst_row_stride != 0) return KVQ_E_INVAL;
    if (n_rows == 0) return KVQ_OK;
    if (!codes || !dst || !aligned16(codes) || !aligned16(dst)) return KVQ_E_INVAL;
    if (n_rows > kMaxElems / row_len) return KVQ_E_INVAL;
    return device_status(launch_pack_words(codes, dst, n_rows * row_len, bits, stream),
                         stream, "kvq_pack");
  }
  if (pack_mode != 0) return KVQ_E_INVAL;
  const int32_t R = row_bytes(bits, row_len);
  if (dst_row_stride < R) return KVQ_E_INVAL;
  if (n_rows == 0) return KVQ_OK;
  if (!codes || !dst || !aligned16(codes) || !aligned16(dst)) return KVQ_E_INVAL;
  if (n_rows > kMaxElems / row_len) return KVQ_E_INVAL;
  PackParams p;
  memset(&p, 0, sizeof(p));
  p.codes = codes;
  p.dst = dst;
  p.n_rows = n_rows;
  p.dst_stride = dst_row_stride;
  p.row_len = row_len;
  p.bits = bits;
  p.chunks_per_row = (row_len + 7) / 8;
  p.n_chunks = n_rows * p.chunks_per_row;
  p.R = R;
  p.contiguous = (dst_row_stride == R) && (row_len % 8 == 0);
  return device_status(launch_pack(p, stream), stream, "kvq_pack");
}

int kvq_unpack(int32_t bits, int32_t pack_mode, const uint8_t* src, int64_t src_row_stride,
               int64_t n_rows, int32_t row_len, uint8_t* codes, hipStream_t stream) {
  if (bits < 1 || bits > 8 || n_rows < 0 || row_len < 1) return KVQ_E_INVAL;
  if (pack_mode == 1) {
    if (src_row_stride != 0) return KVQ_E_INVAL;
    if (n_rows == 0) return KVQ_OK;
    if (!codes || !src || !aligned16(codes) || !aligned16(src)) return KVQ_E_INVAL;
    if (n_rows > kMaxElems / row_len) return KVQ_E_INVAL;
    return device_status(launch_unpack_words(src, codes, n_rows * row_len, bits, stream),
                         stream, "kvq_unpack");
  }
  if (pack_mode != 0) return KVQ_E_INVAL;
  if (src_row_stride < row_bytes(bits, row_len)) return KVQ_E_INVAL;
  if (n_rows == 0) return KVQ_OK;
  if (!codes || !src || !aligned16(codes) || !aligned16(src)) return KVQ_E_INVAL;
  if (n_rows > kMaxElems / row_len) return KVQ_E_INVAL;
  UnpackParams p;
  memset(&p, 0, sizeof(p));
  p.src = src;
  p.codes = codes;
  p.n_rows = n_rows;
  p.src_stride = src_row_stride;
  p.row_len = row_len;
  p.bits = bits;
  p.chunks_per_row = (row_len + 7) / 8;
  p.n_chunks = n_rows * p.chunks_per_row;
  return device_status(launch_unpack(p, stream), stream, "kvq_unpack");
}

int kvq_dequantize(const kvq_layout* layout, int32_t n_filled, kvq_cache_const cache,
                   float* out, hipStream_t stream) {
  if (validate_layout(layout) != KVQ_OK) return KVQ_E_INVAL;
  if (n_filled < 0 || n_filled > layout->n_blocks) return KVQ_E_INVAL;
  if (!cache_ok(cache) || !out || !aligned16(out)) return KVQ_E_INVAL;
  const int sup = gpu_supported(layout);
  if (sup != KVQ_OK) return sup;
  DequantParams p;
  memset(&p, 0, sizeof(p));
  p.codes = cache.codes;
  p.zero = cache.zero;
  p.scale = cache.scale;
  p.out = out;
  p.H = layout->heads;
  p.D = layout->head_dim;
  p.bits = layout->bits;
  p.R = row_bytes(layout->bits, layout->head_dim);
  p.NB = layout->n_blocks;
  p.n_filled = n_filled;
  p.T_cache = offset_of(layout, layout->n_blocks);
  p.T_out = offset_of(layout, n_filled);
  int64_t e = 0;
  for (int i = 0; i < layout->n_blocks; ++i) {
    e += layout->block_tokens[i];
    p.block_end[i] = (int32_t)e;
  }
  p.word_layout = word_layout(layout);
  if (p.word_layout) {
    p.bh_words = words_before(layout, layout->n_blocks);
    for (int i = 0; i < layout->n_blocks; ++i)
      p.block_pad[i] = (int32_t)((32 / layout->bits) * words_before(layout, i) -
                                 layout->head_dim * offset_of(layout, i));
  }
  p.n_chunks = (int64_t)layout->batch * layout->heads * p.T_out * (p.D / 8);
  return device_status(launch_dequantize(p, stream), stream, "kvq_dequantize");
}

int kvq_attend_packed(const kvq_layout* layout, int32_t block, const uint16_t* q_bf16,
                      kvq_cache_const k_cache, kvq_cache_const v_cache, float scale,
                      float* out, hipStream_t stream) {
  AttendParams p;
  const int rc = make_attend_params(layout, block, q_bf16, k_cache, v_cache, scale, out, &p);
  if (rc != KVQ_OK) return rc;
  return device_status(launch_attend(p, layout->head_dim, layout->bits, stream),
                       stream, "kvq_attend_packed");
}

int kvq_attend_split_workspace(const kvq_layout* layout, int32_t block, int32_t max_splits,
                               uint64_t* bytes) {
  if (validate_layout(layout) != KVQ_OK) return KVQ_E_INVAL;
  if (block < 0 || block >= layout->n_blocks || !bytes) return KVQ_E_INVAL;
  if (max_splits < 1 || max_splits > kMaxSplits) return KVQ_E_INVAL;
  *bytes = split_workspace_bytes(layout, block, max_splits);
  return KVQ_OK;
}

int kvq_attend_packed_split(const kvq_layout* layout, int32_t block, const uint16_t* q_bf16,
                            kvq_cache_const k_cache, kvq_cache_const v_cache, float scale,
                            float* out, int32_t max_splits, void* workspace,
                            uint64_t workspace_bytes, hipStream_t stream) {
  AttendParams p;
  const int rc = make_attend_params(layout, block, q_bf16, k_cache, v_cache, scale, out, &p);
  if (rc != KVQ_OK) return rc;
  if (max_splits < 1 || max_splits > kMaxSplits) return KVQ_E_INVAL;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < split_workspace_bytes(layout, block, max_splits))
    return KVQ_E_INVAL;
  p.splits = pick_splits(p, max_splits);
  if (p.splits == 1) return device_status(launch_attend(p, layout->head_dim, layout->bits, stream),
                                          stream, "kvq_attend_packed_split");
  p.ws_rows = (int64_t)p.B * p.n * p.H;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.ws_o + (int64_t)p.splits * p.ws_rows * layout->head_dim;
  return device_status(launch_attend_split(p, layout->head_dim, layout->bits, stream),
                       stream, "kvq_attend_packed_split");
}

int kvq_attend_packed_split_noalloc(const kvq_layout* layout, int32_t block,
                                    const uint16_t* q_bf16, kvq_cache_const k_cache,
                                    kvq_cache_const v_cache, float scale, float* out,
                                    int32_t max_splits, hipStream_t stream) {
  AttendParams p;
  const int rc = make_attend_params(layout, block, q_bf16, k_cache, v_cache, scale, out, &p);
  if (rc != KVQ_OK) return rc;
  if (max_splits < 1 || max_splits > kMaxSplits) return KVQ_E_INVAL;
  if (split_workspace_bytes(layout, block, max_splits) > KVQ_STATIC_SCRATCH_BYTES)
    return KVQ_E_INVAL;
  p.splits = pick_splits(p, max_splits);
  if (p.splits == 1) return device_status(launch_attend(p, layout->head_dim, layout->bits, stream),
                                          stream, "kvq_attend_packed_split_noalloc");
  void* ws = device_scratch();
  if (!ws) return KVQ_E_DEVICE;
  p.ws_rows = (int64_t)p.B * p.n * p.H;
  p.ws_o = static_cast<float*>(ws);
  p.ws_ml = p.ws_o + (int64_t)p.splits * p.ws_rows * layout->head_dim;
  return device_status(launch_attend_split(p, layout->head_dim, layout->bits, stream),
                       stream, "kvq_attend_packed_split_noalloc");
}

int kvq_quantize_attend(const kvq_layout* layout, int32_t block, int32_t src_dtype,
                        const void* k_src, const void* v_src, const uint16_t* q_bf16,
                        kvq_cache k_cache, kvq_cache v_cache, float scale, float* out,
                        int32_t* status_dev, hipStream_t stream) {
  QuantParams qp;
  int rc = make_quant_params(layout, block, src_dtype, k_src, v_src, k_cache, v_cache,
                             status_dev, &qp);
  if (rc != KVQ_OK) return rc;
  AttendParams ap;
  rc = make_attend_params(layout, block, q_bf16, const_view(k_cache), const_view(v_cache), scale,
                          out, &ap);
  if (rc != KVQ_OK) return rc;
  return device_status(launch_quantize_attend(qp, ap, layout->head_dim, layout->bits,
                                              src_dtype == KVQ_F32, stream),
                                                  stream, "kvq_quantize_attend");
}

int kvq_stream_copy(const void* src, void* dst, uint64_t n_bytes, hipStream_t stream) {
  if (n_bytes % 16 != 0) return KVQ_E_INVAL;
  if (n_bytes == 0) return KVQ_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return KVQ_E_INVAL;
  return device_status(launch_stream_copy(src, dst, n_bytes, stream), stream, "kvq_stream_copy");
}

int kvq_stream_read(const void* src, uint64_t n_bytes, uint32_t* sink, hipStream_t stream) {
  if (n_bytes % 16 != 0) return KVQ_E_INVAL;
  if (n_bytes == 0) return KVQ_OK;
  if (!src || !sink || !aligned16(src)) return KVQ_E_INVAL;
  return device_status(launch_stream_read(src, n_bytes, sink, stream), stream, "kvq_stream_read");
}

}  // extern "C"
