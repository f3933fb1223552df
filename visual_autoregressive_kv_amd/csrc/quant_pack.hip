// quant_pack.hip -- fused VAR-Q quantize + bit-pack of one decoded block (gfx950).
//
// VAR-Q (abstract, "groups along the same two axes"): one asymmetric min/max
// grid per (sequence, block, head, channel) group; the block boundary is the
// one the decode loop hands over.  One workgroup pass streams a block's K and V
// from HBM exactly once:
//   1. every thread loads 8-channel chunks (128-bit loads) of its rows into
//      registers (a (tensor, b, h) tile of n_k x D values is spread over
//      `gs` threads, `rpt` rows each);
//   2. per-channel min/max: v_min3/v_max3 over row pairs, then an xor
//      butterfly over the lanes holding the same channels, then across waves
//      through LDS;
//   3. zero = binary16 rounded down from the min, step = binary16 rounded up
//      from fp32(max - zero)/(2^b - 1), reciprocal once per channel;
//   4. codes from the register copy: sub, mul, clamp (v_med3), and a
//      +2^23 add that rounds half-to-even and leaves the integer in the low
//      mantissa bits, summed straight into the packed word with shift-adds;
//   5. packed bytes staged in LDS (3-bit rows are 24 bytes: codes 2 and 5 of
//      each 8 straddle bytes and a block's rows may start 8 bytes off a
//      16-byte boundary) and written with coalesced 128-bit stores, never
//      touching bytes outside the block's rows.
// Tiles too large for registers (video frames) take two passes over HBM:
//   - many tiles: one workgroup per tile streams it twice (extremes, codes);
//   - few tiles (a batch of one video sequence has 2 x heads of them): every
//     tile is cut into register-sized token slices, one workgroup each, over
//     three launches: slice extremes (parked in the block's own code rows,
//     which the last launch overwrites), per-tile statistics, slice codes.
//     Min/max merge in any order, so the bytes are those of one pass.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWG = 256;
constexpr int kMaxRpt = 8;
// LDS staging of one pass of packed rows: up to kWG * kMaxRpt chunks of BITS
// bytes, plus room for every tile slot's 16-byte misalignment
template <int BITS>
constexpr int kStageBytes = kWG * kMaxRpt * (BITS > 4 ? BITS : 4) + 16 * 32;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool F32>
struct Chunk;
template <>
struct Chunk<false> {
  u32x4 w;  // 8 bf16; channel 2j in the low half of word j
};
template <>
struct Chunk<true> {
  f32x4 a, b;
};

template <bool F32>
__device__ __forceinline__ void load_chunk(Chunk<F32>& c, const void* base, int64_t elem) {
  if constexpr (F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
    c.a = __builtin_nontemporal_load(p);
    c.b = __builtin_nontemporal_load(p + 1);
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
    c.w = __builtin_nontemporal_load(p);
  }
}

__device__ __forceinline__ uint32_t word_of(const u32x4& w, int j) {
  return j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
}

// exact binary32 value of channel j
template <bool F32>
__device__ __forceinline__ float chan(const Chunk<F32>& c, int j) {
  if constexpr (F32) {
    const float v[8] = {c.a.x, c.a.y, c.a.z, c.a.w, c.b.x, c.b.y, c.b.z, c.b.w};
    return v[j];
  } else {
    uint32_t w = word_of(c.w, j >> 1);
    return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
}

// value used only for ordering: for odd bf16 channels the raw word, whose low
// 16 bits (the neighbouring channel) sit below the bf16 value's last bit and so
// never change its order against another bf16 value; masked off afterwards
template <bool F32>
__device__ __forceinline__ float chan_order(const Chunk<F32>& c, int j) {
  if constexpr (F32) {
    return chan<true>(c, j);
  } else {
    uint32_t w = word_of(c.w, j >> 1);
    return __uint_as_float((j & 1) ? w : (w << 16));
  }
}

template <bool F32>
__device__ __forceinline__ int nonfinite(const Chunk<F32>& c) {
  int bad = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) bad |= !__builtin_isfinite(chan<F32>(c, j));
  return bad;
}

// Per-thread extremes of the rows [row_base + i * rps] (i < nvalid) of 8 channels.
template <bool F32, bool CHECK>
__device__ __forceinline__ void extremes8(const Chunk<F32> (&v)[kMaxRpt], int nvalid, float (&mn)[8],
                                          float (&mx)[8], int& bad) {
#pragma unroll
  for (int i = 0; i < kMaxRpt; i += 2) {
    if (i < nvalid) {
      const int i2 = (i + 1 < nvalid) ? i + 1 : i;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = chan_order<F32>(v[i], j);
        const float c = chan_order<F32>(v[i2], j);
        mn[j] = min3f(mn[j], a, c);
        mx[j] = max3f(mx[j], a, c);
      }
      if constexpr (CHECK) bad |= nonfinite<F32>(v[i]) | nonfinite<F32>(v[i2]);
    }
  }
}

// Codes of the register rows of one pass, staged in LDS with the destination's
// 16-byte misalignment, then written with 128-bit stores plus byte-exact head
// and tail.  Every thread of the workgroup calls it (one barrier inside).
// BW (block-aligned 3-bit words): the pass starts on a word of the block's
// stream (a pass holds a multiple of 5 rows of 64 or 128 codes, i.e. of ten
// codes) and its words are formed from the dense staging, one per thread.
template <int D, int BITS, bool F32, bool BW>
__device__ __forceinline__ void pack_store(const Chunk<F32> (&v)[kMaxRpt], int nvalid, int r0, int rps,
                                           int cg, const float (&zf)[8], const float (&inv)[8],
                                           uint8_t* my_stage, uint8_t* dst, int rows_here, int R,
                                           int lt, int gs) {
  static_assert(!BW || BITS == 3, "block-aligned words are built for 3-bit codes");
  constexpr int CPR = D / 8;
  const int mis = BW ? 0 : (int)(reinterpret_cast<uintptr_t>(dst) & 15);
#pragma unroll
  for (int i = 0; i < kMaxRpt; ++i) {
    if (i < nvalid) {
      float xv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] = chan<F32>(v[i], j);
      const int chunk = (r0 + i * rps) * CPR + cg;  // within this pass
      store_chunk<BITS>(my_stage + mis + chunk * BITS, pack_chunk<BITS>(xv, zf, inv));
    }
  }
  __syncthreads();
  if constexpr (BW) {
    const int nc = rows_here * D;
    uint32_t* wd = reinterpret_cast<uint32_t*>(dst);
    for (int k = lt; k < (nc + 9) / 10; k += gs) wd[k] = word_from_dense3(my_stage, k, nc);
    return;
  }
  const int nbytes = rows_here * R;
  const int head = min((16 - mis) & 15, nbytes);
  const int body = (nbytes - head) >> 4;
  const int tail = nbytes - head - (body << 4);
  const uint8_t* sp = my_stage + mis;
  for (int k = lt; k < body; k += gs)
    *reinterpret_cast<u32x4*>(dst + head + 16 * k) = *reinterpret_cast<const u32x4*>(sp + head + 16 * k);
  if (lt < head) dst[lt] = sp[lt];
  if (lt < tail) dst[head + 16 * body + lt] = sp[head + 16 * body + lt];
}

template <int D, int BITS, bool F32, bool CHECK, bool STREAM, bool BW>
__global__ __launch_bounds__(kWG) void quant_pack_kernel(QuantParams p) {
  constexpr int CPR = D / 8;  // 8-channel chunks per row
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  __shared__ __align__(16) uint8_t stage[kStageBytes<BITS>];
  __shared__ float red_mn[kWG / kWave][CPR][8];
  __shared__ float red_mx[kWG / kWave][CPR][8];

  const int tid = threadIdx.x;
  const int gs = p.gs;
  const int rpt = p.rpt;
  const int slot = tid / gs;
  const int lt = tid - slot * gs;
  const int64_t tile = (int64_t)blockIdx.x * (kWG / gs) + slot;
  const bool tile_ok = tile < p.n_tiles;
  const int kv = tile_ok ? (int)(tile / p.BH) : 0;
  const int bh = tile_ok ? (int)(tile - (int64_t)kv * p.BH) : 0;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int cg = lt % CPR;
  const int r0 = lt / CPR;
  const int rps = gs / CPR;           // rows covered by one sweep of the tile's threads
  const int rows_per_pass = rps * rpt;
  const int n = tile_ok ? p.n : 0;
  const void* src = p.src[kv];
  const int64_t row_stride = (int64_t)p.H * D;            // elements between tokens
  const int64_t base = ((int64_t)b * p.n * p.H + h) * D + 8 * cg;
  const int slot_bytes = ((gs * rpt * BITS + 16) + 15) & ~15;
  uint8_t* my_stage = stage + slot * slot_bytes;

  Chunk<F32> v[kMaxRpt];
  float mn[8], mx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mn[j] = __uint_as_float(0x7F800000u);
    mx[j] = __uint_as_float(0xFF800000u);
  }
  int bad = 0;

  // ---- phase 1: load + per-thread extremes --------------------------------
  const int n_pass = STREAM ? (n + rows_per_pass - 1) / rows_per_pass : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    const int row_base = pass * rows_per_pass + r0;
    int nvalid = 0;
    if (row_base < n) nvalid = min(rpt, (n - row_base + rps - 1) / rps);
#pragma unroll
    for (int i = 0; i < kMaxRpt; ++i)
      if (i < nvalid) load_chunk<F32>(v[i], src, base + (int64_t)(row_base + i * rps) * row_stride);
    extremes8<F32, CHECK>(v, nvalid, mn, mx, bad);
  }

  // ---- phase 2: reduce across the tile's threads ---------------------------
  const int lanes = min(gs, kWave);
  for (int m = CPR; m < lanes; m <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mn[j] = fminf(mn[j], __shfl_xor(mn[j], m));
      mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], m));
    }
  }
  if (gs > kWave) {
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    if (lane < CPR) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        red_mn[wave][lane][j] = mn[j];
        red_mx[wave][lane][j] = mx[j];
      }
    }
    __syncthreads();
    const int wpt = gs / kWave;
    const int w0 = slot * wpt;
    for (int w = 0; w < wpt; ++w) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mn[j] = fminf(mn[j], red_mn[w0 + w][cg][j]);
        mx[j] = fmaxf(mx[j], red_mx[w0 + w][cg][j]);
      }
    }
  }

  // ---- phase 3: per-channel statistics -------------------------------------
  float zf[8], inv[8];
  uint16_t zb[8], sb[8];
  int flags = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float lo = mn[j], hi = mx[j];
    if (!F32 && (j & 1)) {
      lo = __uint_as_float(__float_as_uint(lo) & 0xFFFF0000u);
      hi = __uint_as_float(__float_as_uint(hi) & 0xFFFF0000u);
    }
    const GroupStats gs_ = group_stats<CHECK>(lo, hi, LEVELS, flags);
    zb[j] = gs_.zb;
    sb[j] = gs_.sb;
    zf[j] = gs_.zf;
    inv[j] = gs_.inv;
  }
  if (tile_ok && r0 == 0) {
    const int64_t so = (((int64_t)b * p.H + h) * p.NB + p.block) * D + 8 * cg;
    u32x4 zw, sw;
    zw.x = zb[0] | ((uint32_t)zb[1] << 16);
    zw.y = zb[2] | ((uint32_t)zb[3] << 16);
    zw.z = zb[4] | ((uint32_t)zb[5] << 16);
    zw.w = zb[6] | ((uint32_t)zb[7] << 16);
    sw.x = sb[0] | ((uint32_t)sb[1] << 16);
    sw.y = sb[2] | ((uint32_t)sb[3] << 16);
    sw.z = sb[4] | ((uint32_t)sb[5] << 16);
    sw.w = sb[6] | ((uint32_t)sb[7] << 16);
    *reinterpret_cast<u32x4*>(p.zero[kv] + so) = zw;
    *reinterpret_cast<u32x4*>(p.scale[kv] + so) = sw;
  }
  if constexpr (CHECK) {
    if (bad) flags |= KVQ_S_NONFINITE;
    if (tile_ok && flags) atomicOr(p.status, flags);
  }

  // ---- phase 4: codes, pack, stage, store ----------------------------------
  uint8_t* dst_tile = BW ? p.codes[kv] + ((int64_t)bh * p.bh_words + p.word_off) * 4
                        : p.codes[kv] + ((int64_t)bh * p.T + p.off) * p.R;
  for (int pass = 0; pass < n_pass; ++pass) {
    const int pass_row0 = pass * rows_per_pass;
    const int row_base = pass_row0 + r0;
    int nvalid = 0;
    if (row_base < n) nvalid = min(rpt, (n - row_base + rps - 1) / rps);
    if constexpr (STREAM) {
#pragma unroll
      for (int i = 0; i < kMaxRpt; ++i)
        if (i < nvalid)
          load_chunk<F32>(v[i], src, base + (int64_t)(row_base + i * rps) * row_stride);
    }
    uint8_t* dst = BW ? dst_tile + 4 * ((int64_t)pass_row0 * D / 10) : dst_tile + (int64_t)pass_row0 * p.R;
    const int rows_here = max(0, min(n - pass_row0, rows_per_pass));
    pack_store<D, BITS, F32, BW>(v, nvalid, r0, rps, cg, zf, inv, my_stage, dst, rows_here, p.R, lt, gs);
    if constexpr (STREAM) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Token-sliced path (few large tiles).  A slice is one register pass of a
// 256-thread workgroup: kSliceRows(D) rows (5 rows per thread for block-aligned
// words, so that every slice starts on a word).  Slice s of a tile parks its
// 2 x D float extremes at float offset 2 D s of the block's packed codes (at
// least 8 D bytes per slice for every supported width, checked by the host).
// ---------------------------------------------------------------------------
template <bool BW>
constexpr int kSliceRpt = BW ? 5 : kMaxRpt;
template <int D, bool BW>
constexpr int kSliceRows = (kWG / (D / 8)) * kSliceRpt<BW>;

__device__ __forceinline__ void tile_of(const QuantParams& p, int64_t tile, int& kv, int& bh, int& b,
                                        int& h) {
  kv = (int)(tile / p.BH);
  bh = (int)(tile - (int64_t)kv * p.BH);
  b = bh / p.H;
  h = bh - b * p.H;
}

// load this thread's rows of slice `slice` of a tile into registers
template <int D, bool F32, bool BW>
__device__ __forceinline__ int load_slice(const QuantParams& p, int kv, int b, int h, int slice,
                                          int tid, Chunk<F32> (&v)[kMaxRpt]) {
  constexpr int CPR = D / 8;
  constexpr int rps = kWG / CPR;
  const int cg = tid % CPR;
  const int row_base = slice * kSliceRows<D, BW> + tid / CPR;
  const int64_t row_stride = (int64_t)p.H * D;
  const int64_t base = ((int64_t)b * p.n * p.H + h) * D + 8 * cg;
  int nvalid = 0;
  if (row_base < p.n) nvalid = min(kSliceRpt<BW>, (p.n - row_base + rps - 1) / rps);
#pragma unroll
  for (int i = 0; i < kMaxRpt; ++i)
    if (i < nvalid) load_chunk<F32>(v[i], p.src[kv], base + (int64_t)(row_base + i * rps) * row_stride);
  return nvalid;
}

template <int D, bool F32, bool CHECK, bool BW>
__global__ __launch_bounds__(kWG) void slice_extremes_kernel(QuantParams p, int n_slices) {
  constexpr int CPR = D / 8;
  __shared__ float red_mn[kWG / kWave][CPR][8];
  __shared__ float red_mx[kWG / kWave][CPR][8];
  const int tid = threadIdx.x;
  const int64_t tile = blockIdx.x / n_slices;
  const int slice = (int)(blockIdx.x - tile * n_slices);
  int kv, bh, b, h;
  tile_of(p, tile, kv, bh, b, h);
  Chunk<F32> v[kMaxRpt];
  const int nvalid = load_slice<D, F32, BW>(p, kv, b, h, slice, tid, v);
  float mn[8], mx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mn[j] = __uint_as_float(0x7F800000u);
    mx[j] = __uint_as_float(0xFF800000u);
  }
  int bad = 0;
  extremes8<F32, CHECK>(v, nvalid, mn, mx, bad);
  for (int m = CPR; m < kWave; m <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mn[j] = fminf(mn[j], __shfl_xor(mn[j], m));
      mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], m));
    }
  }
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  if (lane < CPR) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      red_mn[wave][lane][j] = mn[j];
      red_mx[wave][lane][j] = mx[j];
    }
  }
  __syncthreads();
  if (tid < CPR) {
    float* ext = reinterpret_cast<float*>(block_codes(p, kv, bh)) + (int64_t)slice * 2 * D;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float lo = red_mn[0][tid][j], hi = red_mx[0][tid][j];
      for (int w = 1; w < kWG / kWave; ++w) {
        lo = fminf(lo, red_mn[w][tid][j]);
        hi = fmaxf(hi, red_mx[w][tid][j]);
      }
      ext[8 * tid + j] = lo;
      ext[D + 8 * tid + j] = hi;
    }
  }
  if constexpr (CHECK) {
    if (bad) atomicOr(p.status, KVQ_S_NONFINITE);
  }
}

// one workgroup per tile, thread = channel: merge the slices, statistics
template <int D, int BITS, bool F32, bool CHECK>
__global__ __launch_bounds__(D) void slice_stats_kernel(QuantParams p, int n_slices) {
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  const int ch = threadIdx.x;
  int kv, bh, b, h;
  tile_of(p, blockIdx.x, kv, bh, b, h);
  const float* ext = reinterpret_cast<const float*>(block_codes(p, kv, bh));
  float lo = __uint_as_float(0x7F800000u), hi = __uint_as_float(0xFF800000u);
#pragma unroll 8
  for (int sl = 0; sl < n_slices; ++sl) {
    lo = fminf(lo, ext[(int64_t)sl * 2 * D + ch]);
    hi = fmaxf(hi, ext[(int64_t)sl * 2 * D + D + ch]);
  }
  if (!F32 && (ch & 1)) {  // drop the neighbouring channel's bits (ordering keys)
    lo = __uint_as_float(__float_as_uint(lo) & 0xFFFF0000u);
    hi = __uint_as_float(__float_as_uint(hi) & 0xFFFF0000u);
  }
  int flags = 0;
  const GroupStats g = group_stats<CHECK>(lo, hi, LEVELS, flags);
  const int64_t so = (((int64_t)b * p.H + h) * p.NB + p.block) * D + ch;
  p.zero[kv][so] = g.zb;
  p.scale[kv][so] = g.sb;
  if constexpr (CHECK) {
    if (flags) atomicOr(p.status, flags);
  }
}

// codes of one slice from the tile's binary16 statistics (zero and reciprocal
// step rebuilt exactly as group_stats makes them)
template <int D, int BITS, bool F32, bool BW>
__global__ __launch_bounds__(kWG) void slice_pack_kernel(QuantParams p, int n_slices) {
  constexpr int CPR = D / 8;
  __shared__ __align__(16) uint8_t stage[kStageBytes<BITS>];
  const int tid = threadIdx.x;
  const int64_t tile = blockIdx.x / n_slices;
  const int slice = (int)(blockIdx.x - tile * n_slices);
  int kv, bh, b, h;
  tile_of(p, tile, kv, bh, b, h);
  Chunk<F32> v[kMaxRpt];
  const int nvalid = load_slice<D, F32, BW>(p, kv, b, h, slice, tid, v);
  const int cg = tid % CPR;
  const int64_t so = (((int64_t)b * p.H + h) * p.NB + p.block) * D + 8 * cg;
  const u32x4 zw = *reinterpret_cast<const u32x4*>(p.zero[kv] + so);
  const u32x4 sw = *reinterpret_cast<const u32x4*>(p.scale[kv] + so);
  float zf[8], inv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t zpair = word_of(zw, j >> 1), spair = word_of(sw, j >> 1);
    zf[j] = h2f((uint16_t)((j & 1) ? (zpair >> 16) : (zpair & 0xFFFFu)));
    const float sf = h2f((uint16_t)((j & 1) ? (spair >> 16) : (spair & 0xFFFFu)));
    inv[j] = (sf > 0.0f) ? 1.0f / sf : 0.0f;
  }
  const int row0 = slice * kSliceRows<D, BW>;
  uint8_t* dst = block_codes(p, kv, bh) + (BW ? 4 * ((int64_t)row0 * D / 10) : (int64_t)row0 * p.R);
  const int rows_here = min(p.n - row0, kSliceRows<D, BW>);
  pack_store<D, BITS, F32, BW>(v, nvalid, tid / CPR, kWG / CPR, cg, zf, inv, stage, dst, rows_here,
                               p.R, tid, kWG);
}

// tiles below which a block too large for registers is cut into slices
constexpr int64_t kSliceTiles = 1024;

template <int D, int BITS, bool F32, bool CHECK, bool BW>
hipError_t launch_sliced(const QuantParams& p, hipStream_t s) {
  const int n_slices = (p.n + kSliceRows<D, BW> - 1) / kSliceRows<D, BW>;
  // parked extremes must fit the block's packed codes
  const int64_t block_bytes = BW ? 4 * (((int64_t)p.n * D + 9) / 10) : (int64_t)p.n * p.R;
  if ((int64_t)n_slices * 8 * D > block_bytes) return hipErrorInvalidValue;
  if (!dispatch_fits(p.n_tiles * n_slices, kWG)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(p.n_tiles * n_slices));
  hipLaunchKernelGGL((slice_extremes_kernel<D, F32, CHECK, BW>), grid, dim3(kWG), 0, s, p, n_slices);
  hipLaunchKernelGGL((slice_stats_kernel<D, BITS, F32, CHECK>), dim3((unsigned)p.n_tiles), dim3(D), 0,
                     s, p, n_slices);
  hipLaunchKernelGGL((slice_pack_kernel<D, BITS, F32, BW>), grid, dim3(kWG), 0, s, p, n_slices);
  return hipGetLastError();
}

template <int D, int BITS, bool F32, bool BW>
hipError_t launch_t(const QuantParams& p, hipStream_t s) {
  const int tiles_per_wg = kWG / p.gs;
  const int64_t grid = (p.n_tiles + tiles_per_wg - 1) / tiles_per_wg;
  const bool stream = (int64_t)(p.gs / (D / 8)) * p.rpt < p.n;
  const bool check = p.status != nullptr;
  if (stream && p.n_tiles < kSliceTiles)
    return check ? launch_sliced<D, BITS, F32, true, BW>(p, s)
                 : launch_sliced<D, BITS, F32, false, BW>(p, s);
  if (!dispatch_fits(grid, kWG)) return hipErrorInvalidConfiguration;
  dim3 g((unsigned)grid), blk(kWG);
  if (check) {
    if (stream)
      hipLaunchKernelGGL((quant_pack_kernel<D, BITS, F32, true, true, BW>), g, blk, 0, s, p);
    else
      hipLaunchKernelGGL((quant_pack_kernel<D, BITS, F32, true, false, BW>), g, blk, 0, s, p);
  } else {
    if (stream)
      hipLaunchKernelGGL((quant_pack_kernel<D, BITS, F32, false, true, BW>), g, blk, 0, s, p);
    else
      hipLaunchKernelGGL((quant_pack_kernel<D, BITS, F32, false, false, BW>), g, blk, 0, s, p);
  }
  return hipGetLastError();
}

template <int D, int BITS, bool BW = false>
hipError_t launch_b(const QuantParams& p, bool f32src, hipStream_t s) {
  return f32src ? launch_t<D, BITS, true, BW>(p, s) : launch_t<D, BITS, false, BW>(p, s);
}

template <int D>
hipError_t launch_d(const QuantParams& p, int bits, bool f32src, hipStream_t s) {
  if (p.word_layout) return bits == 3 ? launch_b<D, 3, true>(p, f32src, s) : hipErrorInvalidValue;
  switch (bits) {
    case 2: return launch_b<D, 2>(p, f32src, s);
    case 3: return launch_b<D, 3>(p, f32src, s);
    case 4: return launch_b<D, 4>(p, f32src, s);
    case 8: return launch_b<D, 8>(p, f32src, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_quantize(const QuantParams& p, int head_dim, int bits, bool f32src,
                           hipStream_t s) {
  if (head_dim == 64) return launch_d<64>(p, bits, f32src, s);
  return launch_d<128>(p, bits, f32src, s);
}

}  // namespace kvq
