// attend.hip -- block-causal decode attention over the packed VAR-Q cache (gfx950).
//
// Block-by-block decoding (VAR-Q abstract): the n_k queries of block k attend
// to every cached token of blocks 0..k.  One workgroup owns up to 256 queries of
// one (sequence, head); its waves own 32 queries each.  (For long prefixes the
// same kernel can own one range of the prefix's key tiles instead, writing a
// partial result that attend_merge_kernel combines by log-sum-exp.)  The packed
// prefix is streamed once per workgroup in tiles of 32 keys, software-pipelined:
//   iteration j:  issue the buffer loads of tile j+2's packed codes,
//                 S^T of tile j from LDS (MFMA),
//                 dequantize tile j+1 (loaded one iteration earlier) into the
//                 other LDS buffer while those MFMAs run,
//                 softmax and O of tile j,
//                 one barrier.
//   (8-wave workgroups stagger this order between the two waves that share a
//   SIMD, so that one's VALU work runs beside the other's MFMAs.)
//   Dequantization (shared by the workgroup's waves through LDS):
//   - the (block, channel) statistics of the whole prefix are staged in LDS;
//     every thread owns fixed items (one key x 8 channels of K or of V) and
//     keeps its key's current block's binary16 statistics in registers,
//     refreshed only when the key crosses into the next block;
//   - k_hat = fma(code, s, z) in fp32 straight from the binary16 statistics
//     (v_fma_mix_f32; INT4 codes spread to bytes and converted with
//     v_cvt_f32_ubyteN); k_hat is split into a truncated bf16 high part and a
//     bf16 remainder, so two bf16 products reproduce it to ~2^-16;
//   - v_hat is rounded to fp16; lanes holding neighbouring keys swap halves
//     (DPP) so each writes dwords of (key 2m, key 2m+1) pairs into V^T, whose
//     odd dword row stride spreads them over the LDS banks.
//   Compute (per wave, 32 queries):
//   - S^T = K_hat Q^T with v_mfma_f32_32x32x16_bf16 (hi and lo accumulate into
//     one fp32 tile; the next k-step's operands are read from LDS while the
//     current MFMAs run): every lane holds 16 keys of one query, so the row
//     maximum is a per-lane reduction plus one v_permlane32_swap;
//   - online softmax in the log2 domain, p = exp2(fma(s, c, -m c)); the running
//     maximum only moves when a tile raises it by more than 2^8 (p then stays
//     <= 256, safe in fp16), which skips the accumulator rescale on almost every
//     tile; masking only on the last, partial tile;
//   - P (fp16, packed round-toward-zero) feeds O^T += V_hat^T P^T with
//     v_mfma_f32_32x32x16_f16 straight from registers: the 16 keys a lane holds
//     are exactly the contraction slots its lane group supplies; the softmax
//     denominator sums the same rounded P with v_dot2_f32_f16.
// Output is fp32 (bf16 output rounding alone would exceed the 2e-3 bound).
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int KT = 32;                  // keys per tile
constexpr int KPAD = 8;                 // K tile row padding (elements)
constexpr int VROW = KT / 2 + 1;        // V^T row stride in dwords (odd)
constexpr int kMaxWaves = 8;
constexpr float kRescaleLog2 = 8.0f;    // lazy-rescale slack, log2 units

// byte n of a 32-bit word to fp32 (one instruction)
template <int N>
__device__ __forceinline__ float ubyte_f32(uint32_t w) {
  float r;
  if constexpr (N == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(w));
  if constexpr (N == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(w));
  if constexpr (N == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(w));
  if constexpr (N == 3) asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(w));
  return r;
}

// two fp32 -> packed bf16 / fp16 pair, round to nearest even (low half = a)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  uint32_t r;
  asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// max / sum of a value and its copy 32 lanes away (lane ^ 32)
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// value of the neighbouring lane (lane ^ 1)
__device__ __forceinline__ uint32_t swap_adjacent(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1 /* quad_perm 1,0,3,2 */, 0xF, 0xF,
                                            false);
}

// Whether the top grid level z + L*s of any of 8 value groups can leave the
// binary16 range.  Binary32 input up to +-65504 can give a top level of up to
// about 65566 after the step is rounded up; the attention then forms v_hat / 2
// in binary16 (exact halving) and doubles its output, so v_hat never overflows.
template <int BITS>
__device__ __forceinline__ bool v_top_over_f16(const u32x4& zw, const u32x4& sw) {
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  const f16x8 z = __builtin_bit_cast(f16x8, zw), s = __builtin_bit_cast(f16x8, sw);
  bool over = false;
#pragma unroll
  for (int c = 0; c < 8; ++c) over |= __builtin_fmaf(LEVELS, (float)s[c], (float)z[c]) > 65504.0f;
  return over;
}

// the 8 codes of one packed chunk as fp32
template <int BITS>
__device__ __forceinline__ void codes_f32(uint32_t w, float c[8]) {
  if constexpr (BITS == 4) {
    const uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
    c[0] = ubyte_f32<0>(lo);
    c[1] = ubyte_f32<0>(hi);
    c[2] = ubyte_f32<1>(lo);
    c[3] = ubyte_f32<1>(hi);
    c[4] = ubyte_f32<2>(lo);
    c[5] = ubyte_f32<2>(hi);
    c[6] = ubyte_f32<3>(lo);
    c[7] = ubyte_f32<3>(hi);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = (float)((w >> (BITS * j)) & ((1u << BITS) - 1u));
  }
}

// 3- and 8-bit chunks need two dwords of a row, 2- and 4-bit chunks one
template <int BITS>
constexpr bool kTwoWords = BITS == 3 || BITS == 8;

// the 8 codes of one packed chunk as fp32: its bits start at bit `shift` of
// w0 and continue into w1 (3-bit codes; 8-bit codes 4-7 are all of w1)
template <int BITS>
__device__ __forceinline__ void chunk_f32(uint32_t w0, uint32_t w1, int shift, float c[8]) {
  static_assert(kWidthBuilt<BITS>, "code width not built");
  if constexpr (BITS == 4) {
    codes_f32<4>(w0, c);
  } else if constexpr (BITS == 8) {
    c[0] = ubyte_f32<0>(w0);
    c[1] = ubyte_f32<1>(w0);
    c[2] = ubyte_f32<2>(w0);
    c[3] = ubyte_f32<3>(w0);
    c[4] = ubyte_f32<0>(w1);
    c[5] = ubyte_f32<1>(w1);
    c[6] = ubyte_f32<2>(w1);
    c[7] = ubyte_f32<3>(w1);
  } else if constexpr (BITS == 2) {
    const uint32_t w = w0 >> shift;
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = (float)((w >> (2 * j)) & 3u);
  } else {
    const uint64_t v = (uint64_t)w0 | ((uint64_t)w1 << 32);
    codes_f32<BITS>((uint32_t)(v >> shift), c);
  }
}

// the 8 codes of a chunk of block-aligned 3-bit words: code sh / 3 of word w0
// onward, the chunk continuing into w1 past the word's ten codes
__device__ __forceinline__ void chunk_words3_f32(uint32_t w0, uint32_t w1, int sh, float c[8]) {
  codes_f32<3>((w0 >> sh) | (w1 << (30 - sh)), c);
}

// Word index and bit shift of the chunk that starts at code gi of a stream of
// block-aligned 3-bit words (gi / 10 by multiply-high: exact for 32-bit gi).
__device__ __forceinline__ uint32_t word_of_code(uint32_t gi, int& sh) {
  const uint32_t w = __umulhi(gi, 0xCCCCCCCDu) >> 3;
  sh = 3 * (int)(gi - 10u * w);
  return w;
}

// Raw buffer view of key tile j of one (b, h)'s packed prefix.  The hardware
// range check covers the per-lane offset only (not the scalar offset), so the
// tile's start goes into the base address and the record count is what is
// left of the prefix: loads past the prefix's end return 0 and never leave it;
// a tile past the prefix gets zero records, so its loads touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* prefix, int prefix_bytes,
                                                            int tile_bytes, int j) {
  const int off = j * tile_bytes;
  const int left = prefix_bytes > off ? prefix_bytes - off : 0;  // past the prefix: none
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(prefix + off), (short)0, left,
                                           0x00020000 /* 32-bit data format */);
}

// ---------------------------------------------------------------------------
// Fused launch, quantize side for a workgroup that owns one (sequence, head):
// the first half of the threads quantizes block k of K, the second half of V
// (bf16 input, the same group statistics and code arithmetic as the standalone
// quantize kernel).  Within a wave, L neighbouring lanes share one 8-channel
// chunk (L = 8, or 4 for a 2-wave workgroup at head_dim 128), so a wave covers
// 64 / L chunks and CW = D / 8 / (64 / L) waves cover a row; lane l of the
// half's wave w holds chunk (w % CW) * 64 / L + l / L of rows rl, rl + RG, ..
// (at most MAXR) with row lane rl = (w / CW) * L + l % L:
//   - per thread: v_min3 / v_max3 over row pairs (for the odd bf16 channel of
//     a word the raw word is the ordering key, masked afterwards);
//   - across the L lanes of a chunk: DPP steps (xor 1, xor 2 inside a quad,
//     then for L = 8 the mirror of the half-row);
//   - across the half's row waves: LDS; the half's first D threads then compute
//     every channel's statistics once (thread = channel);
//   - codes: every thread packs its rows into an LDS copy of the block's rows
//     (with the destination's 16-byte misalignment), which the half writes to
//     the cache with 128-bit stores plus byte-exact head and tail.
// The packed rows reach the cache before the caller's barrier, so the attention
// reads them back like older blocks.
// scratch: wg_quant_scratch<D, NW>() floats; stage_k, stage_v: 16 + 32 * NW * R bytes each.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// lanes sharing a chunk, chunks per wave, waves per row, row lanes, rows per thread
template <int D, int NW>
struct WgQuantShape {
  static constexpr int CPR = D / 8;
  static constexpr int WT = NW / 2;                         // waves per tensor
  static constexpr int L = (D == 128 && NW == 2) ? 4 : 8;   // lanes per chunk in a wave
  static constexpr int CPW = kWave / L;                     // chunks per wave
  static constexpr int CW = CPR / CPW;                      // waves per row
  static constexpr int RW = WT / CW;                        // row waves
  static constexpr int RG = RW * L;                         // row lanes per tensor
  static constexpr int MAXR = (NW * 32 + RG - 1) / RG;      // rows per thread (n <= NW * 32)
  static_assert(CPR % CPW == 0 && WT % CW == 0 && RW >= 1, "chunk layout must tile the row");
};
// scratch floats of quantize_block_wg: per tensor and row wave the channel
// extremes, then per tensor the channel zero points and reciprocal steps (no
// prologue below 2 waves)
template <int D, int NW>
__host__ __device__ constexpr int wg_quant_scratch() {
  if constexpr (NW < 2) {
    return 0;
  } else {
    return 2 * WgQuantShape<D, NW>::RW * 2 * D + 2 * 2 * D;
  }
}

template <int D, int BITS, int NW, bool CHECK, bool BW>
__device__ __forceinline__ void quantize_block_wg(const AttendParams& p, int b, int h, int tid,
                                                  _Float16* st_lds, float* scratch,
                                                  uint8_t* stage_k, uint8_t* stage_v, int& vover) {
  using S = WgQuantShape<D, NW>;
  static_assert((D == 64 || D == 128) && NW >= 2, "64- or 128-channel heads, a wave per tensor");
  constexpr int CPR = D / 8;
  constexpr int GT = NW * kWave / 2;  // threads per tensor
  constexpr int L = S::L;
  constexpr int RG = S::RG;
  constexpr int MAXR = S::MAXR;
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  const FuseParams& f = p.fz;
  const int n = p.n;
  const int lane = tid % kWave;
  const int tensor = tid / GT;
  const int u = tid % GT;
  const int wt = u / kWave;
  // (L and CW are powers of two: masks and shifts on the lane index)
  constexpr int LSH = L == 8 ? 3 : 2;
  const int c = (wt & (S::CW - 1)) * S::CPW + (lane >> LSH);
  const int rw = wt / S::CW;  // row wave
  const int rg = rw * L + (lane & (L - 1));
  const int64_t row_stride = (int64_t)p.H * D;
  const int64_t base = ((int64_t)b * n * p.H + h) * D + 8 * c;
  const uint16_t* src = static_cast<const uint16_t*>(f.src[tensor]);

  u32x4 w[MAXR];
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    const int r = rg + RG * i;
    if (r < n) w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + base + r * row_stride));
  }
  // exact value of channel j, and the key that orders it
  auto chan = [&](const u32x4& v, int j) {
    const uint32_t x = v[j >> 1];
    return __uint_as_float((j & 1) ? (x & 0xFFFF0000u) : (x << 16));
  };
  auto key = [&](const u32x4& v, int j) {
    const uint32_t x = v[j >> 1];
    return __uint_as_float((j & 1) ? x : (x << 16));
  };
  float mn[8], mx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mn[j] = __uint_as_float(0x7F800000u);
    mx[j] = __uint_as_float(0xFF800000u);
  }
  int bad = 0;
#pragma unroll
  for (int i = 0; i < MAXR; i += 2) {
    if (rg + RG * i < n) {
      const int i2 = (rg + RG * (i + 1) < n) ? i + 1 : i;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = key(w[i], j), e = key(w[i2], j);
        mn[j] = min3f(mn[j], a, e);
        mx[j] = max3f(mx[j], a, e);
      }
      if constexpr (CHECK) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // a bf16 is NaN or +-inf when its exponent bits are all set
          bad |= ((w[i][q] & 0x7F80u) == 0x7F80u) | ((w[i][q] & 0x7F800000u) == 0x7F800000u);
          bad |= ((w[i2][q] & 0x7F80u) == 0x7F80u) | ((w[i2][q] & 0x7F800000u) == 0x7F800000u);
        }
      }
    }
  }
  // the L lanes holding chunk c: xor 1 and xor 2 inside each quad, then for
  // L = 8 the mirror of each half-row (lane i with lane 7 - i)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mn[j] = min3f(mn[j], dpp_f32<0xB1>(mn[j]), mn[j]);
    mx[j] = max3f(mx[j], dpp_f32<0xB1>(mx[j]), mx[j]);
    mn[j] = min3f(mn[j], dpp_f32<0x4E>(mn[j]), mn[j]);
    mx[j] = max3f(mx[j], dpp_f32<0x4E>(mx[j]), mx[j]);
    if constexpr (L == 8) {
      mn[j] = min3f(mn[j], dpp_f32<0x141>(mn[j]), mn[j]);
      mx[j] = max3f(mx[j], dpp_f32<0x141>(mx[j]), mx[j]);
    }
  }
  float* red = scratch;                          // [tensor][row wave][min|max][D]
  float* zi = scratch + 2 * S::RW * 2 * D;       // [tensor][zero|reciprocal][D]
  if ((lane & (L - 1)) == 0) {
    float* rm = red + ((tensor * S::RW + rw) * 2 + 0) * D + 8 * c;
    float* rx = red + ((tensor * S::RW + rw) * 2 + 1) * D + 8 * c;
    *reinterpret_cast<f32x4*>(rm) = f32x4{mn[0], mn[1], mn[2], mn[3]};
    *reinterpret_cast<f32x4*>(rm + 4) = f32x4{mn[4], mn[5], mn[6], mn[7]};
    *reinterpret_cast<f32x4*>(rx) = f32x4{mx[0], mx[1], mx[2], mx[3]};
    *reinterpret_cast<f32x4*>(rx + 4) = f32x4{mx[4], mx[5], mx[6], mx[7]};
  }
  __syncthreads();
  int flags = 0;
  // the half's threads take one channel each (two for a 2-wave workgroup at
  // head_dim 128; a straight branch otherwise, which keeps the register
  // allocation of the tile loop free of spills)
  auto channel_stats = [&](int ch) {
    float lo = red[((tensor * S::RW) * 2 + 0) * D + ch];
    float hi = red[((tensor * S::RW) * 2 + 1) * D + ch];
#pragma unroll
    for (int wv = 1; wv < S::RW; ++wv) {
      lo = min3f(lo, red[((tensor * S::RW + wv) * 2 + 0) * D + ch], lo);
      hi = max3f(hi, red[((tensor * S::RW + wv) * 2 + 1) * D + ch], hi);
    }
    if (ch & 1) {  // the raw-word keys of odd channels
      lo = __uint_as_float(__float_as_uint(lo) & 0xFFFF0000u);
      hi = __uint_as_float(__float_as_uint(hi) & 0xFFFF0000u);
    }
    const GroupStats gst = group_stats<CHECK>(lo, hi, LEVELS, flags);
    const int64_t so = (((int64_t)b * p.H + h) * p.NB + f.block) * D + ch;
    f.zero[tensor][so] = gst.zb;
    f.scale[tensor][so] = gst.sb;
    _Float16* srow = st_lds + ((f.block * 2 + tensor) * 2) * D;
    srow[ch] = __builtin_bit_cast(_Float16, gst.zb);
    srow[D + ch] = __builtin_bit_cast(_Float16, gst.sb);
    zi[(tensor * 2 + 0) * D + ch] = gst.zf;
    zi[(tensor * 2 + 1) * D + ch] = gst.inv;
    if (tensor == 1) vover |= __builtin_fmaf(LEVELS, h2f(gst.sb), gst.zf) > 65504.0f;
  };
  if constexpr (D == kWave) {
    if (u < kWave) channel_stats(lane);  // the half's first wave: lane = channel
  } else if constexpr (GT >= D) {
    if (u < D) channel_stats(u);
  } else {
    for (int ch = u; ch < D; ch += GT) channel_stats(ch);
  }
  __syncthreads();
  float zf[8], inv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    zf[j] = zi[(tensor * 2 + 0) * D + 8 * c + j];
    inv[j] = zi[(tensor * 2 + 1) * D + 8 * c + j];
  }
  uint8_t* dst = BW ? f.codes[tensor] + (((int64_t)b * p.H + h) * p.bh_words + f.word_off) * 4
                    : f.codes[tensor] + (((int64_t)b * p.H + h) * p.T_cache + f.off) * p.R;
  const int mis = BW ? 0 : (int)(reinterpret_cast<uintptr_t>(dst) & 15);
  uint8_t* stg = (tensor == 0 ? stage_k : stage_v) + mis;
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    const int r = rg + RG * i;
    if (r < n) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = chan(w[i], j);
      const Packed8 pk = pack_chunk<BITS>(x, zf, inv);
      if constexpr (BITS != 3) {
        // chunks on BITS-byte boundaries go straight to the cache (a wave
        // writes 8 whole rows per store instruction)
        store_chunk<BITS>(dst + r * p.R + BITS * c, pk);
      } else {
        store_chunk<BITS>(stg + r * p.R + BITS * c, pk);
      }
    }
  }
  if constexpr (BW) {
    // block-aligned words: word k of the block's stream from the dense staging
    __syncthreads();
    const int nc = n * D;
    uint32_t* wd = reinterpret_cast<uint32_t*>(dst);
    for (int k = u; k < (nc + 9) / 10; k += GT) wd[k] = word_from_dense3(stg, k, nc);
  } else if constexpr (BITS == 3) {
    // 24-byte rows, 3 bytes per chunk, possibly 8 bytes off a 16-byte boundary:
    // the block's n * R bytes go out of LDS as 128-bit stores, byte-exact ends
    __syncthreads();
    const int nbytes = n * p.R;
    const int head = min((16 - mis) & 15, nbytes);
    const int body = (nbytes - head) >> 4;
    const int tail = nbytes - head - (body << 4);
    for (int k = u; k < body; k += GT)
      *reinterpret_cast<u32x4*>(dst + head + 16 * k) = *reinterpret_cast<const u32x4*>(stg + head + 16 * k);
    if (u < head) dst[u] = stg[u];
    if (u < tail) dst[head + 16 * body + u] = stg[head + 16 * body + u];
  }
  if constexpr (CHECK) {
    if (bad) flags |= KVQ_S_NONFINITE;
    if (flags) atomicOr(f.status, flags);
  }
  // the workgroup reads these rows back after the caller's barrier
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
}

// FUSE: 0 attention only; 1/2 quantize block k from bf16 first (2: with input
// checks); the launcher uses it with one query tile per (sequence, head).
// SPLIT: the workgroup attends only key-tile range sp of p.splits (whole
// tiles, balanced) and writes its unnormalized output, running maximum and
// denominator to the workspace for attend_merge_kernel (attention only).
// Register caps for residency: 2-wave workgroups at 3 waves per SIMD and 4-wave
// workgroups at 4 (a few dwords spill; measured faster on VAR-d20 than the
// extra dispatch rounds without the cap).  3- and 8-bit codes hold two words
// per item in flight and spill inside the tile loop at those caps, so their 2-
// and 4-wave workgroups run one wave per SIMD lower (measured faster: no spills).
__host__ __device__ constexpr int waves_per_eu(int nw, int bits) {
  const bool two_words = bits == 3 || bits == 8;
  return nw == 2 ? (two_words ? 2 : 3) : nw == 4 ? (two_words ? 3 : 4) : 1;
}

// BW: the cache holds block-aligned 3-bit words (BITS == 3); each item's word
// and shift are computed per tile from its key's block.
template <int D, int BITS, int NW, int FUSE, int SPLIT = 0, bool BW = false>
// Register caps chosen for residency (waves_per_eu below).
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu(waves_per_eu(NW, BITS)))) void attend_kernel(AttendParams p) {
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;              // k-steps of the QK^T contraction
  constexpr int MT = D / 32;              // 32-row tiles of O^T
  constexpr int NT = NW * kWave;          // threads
  constexpr int ITEMS = KT * CPR;         // (key, chunk) items per tensor per tile
  constexpr int MAXI = 2 * ITEMS / NT;    // items per thread per tile
  static_assert(2 * ITEMS % NT == 0 && ITEMS % kWave == 0, "items must split evenly");
  __shared__ __align__(16) __bf16 k_hi[2][KT][D + KPAD];
  __shared__ __align__(16) __bf16 k_lo[2][KT][D + KPAD];
  __shared__ __align__(16) uint32_t v_t[2][D][VROW];  // fp16 pairs (keys 2m, 2m+1)
  extern __shared__ __align__(16) _Float16 st[];     // [blk][tensor][z|s][D] when it fits
  __shared__ int blk_end[KVQ_MAX_BLOCKS];
  __shared__ int blk_pad[BW ? KVQ_MAX_BLOCKS : 1];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int g = lane >> 5;    // lane group: which 8 of each 16 contraction slots
  const int col = lane & 31;  // this lane's query (S^T / O^T column)
  static_assert(SPLIT == 0 || FUSE == 0, "key ranges are for the attention-only launch");
  static_assert(!BW || BITS == 3, "block-aligned words are built for 3-bit codes");
  // fused prologue: block rows staged in k_lo (K) and v_t (V), extremes in k_hi
  static_assert(FUSE == 0 || ((BITS != 3 || (sizeof(k_lo) >= 16 + NW * 32 * BITS * D / 8 &&
                                             sizeof(v_t) >= 16 + NW * 32 * BITS * D / 8)) &&
                              sizeof(k_hi) >= wg_quant_scratch<D, NW>() * sizeof(float)),
                "LDS too small for the quantize prologue");
  const int wg = SPLIT ? (int)(blockIdx.x / p.splits) : (int)blockIdx.x;
  const int sp = SPLIT ? (int)blockIdx.x - wg * p.splits : 0;
  const int bh = wg / p.q_tiles;
  const int qt = wg - bh * p.q_tiles;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int q = qt * NW * 32 + wave * 32 + col;
  const bool q_ok = q < p.n;
  const bool wave_live = qt * NW * 32 + wave * 32 < p.n;
  const int nkb = p.n_kblocks;
  const int64_t stat_base = (int64_t)bh * p.NB * D;
  const int n_prefix = p.n_prefix;
  const int n_tiles = (n_prefix + KT - 1) / KT;
  // this workgroup's key tiles [j_begin, j_end): all, or one balanced range
  const int j_begin = SPLIT ? (int)((int64_t)sp * n_tiles / p.splits) : 0;
  const int j_end = SPLIT ? (int)((int64_t)(sp + 1) * n_tiles / p.splits) : n_tiles;

  // Fused launch: quantize block k first (k_hi is free until tile 0 is
  // dequantized; the statistics slot of block k in LDS is filled here, the
  // copy below skips it; the barrier after the copy publishes everything).
  int vover = 0;  // a V group's top grid level leaves the binary16 range
  if constexpr (BW) {
    // block ends and paddings before any load: the loads' addresses need them
    for (int i = tid; i < nkb; i += NT) {
      blk_end[i] = p.block_end[i];
      blk_pad[i] = p.block_pad[i];
    }
    __syncthreads();
  }
  if constexpr (FUSE != 0) {
    quantize_block_wg<D, BITS, NW, FUSE == 2, BW>(p, b, h, tid, st,
                                              reinterpret_cast<float*>(&k_hi[0][0][0]),
                                              reinterpret_cast<uint8_t*>(&k_lo[0][0][0]),
                                              reinterpret_cast<uint8_t*>(&v_t[0][0][0]), vover);
  }

  // ---- item slots: (tensor, key, chunk), fixed for every tile ----------------
  // K items: key = rem / CPR (a row chunk); V items: key = rem % KT, so
  // neighbouring lanes hold neighbouring keys and can pair them.
  const uint8_t* kpfx = BW ? p.kcodes + (int64_t)bh * p.bh_words * 4 : p.kcodes + (int64_t)bh * p.T_cache * p.R;
  const uint8_t* vpfx = BW ? p.vcodes + (int64_t)bh * p.bh_words * 4 : p.vcodes + (int64_t)bh * p.T_cache * p.R;
  const int pfx_bytes = BW ? 4 * p.prefix_words : n_prefix * p.R;
  const int tile_bytes = KT * p.R;
  int s_tensor[MAXI], s_key[MAXI], s_cg[MAXI], s_voff[MAXI], s_shift[MAXI];
  // BW: block of each item's key at its latest load, and that block's padding
  int i_blk[MAXI], i_pad[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int it = tid + i * NT;
    s_tensor[i] = __builtin_amdgcn_readfirstlane((wave * kWave + i * NT) / ITEMS);
    const int rem = it - s_tensor[i] * ITEMS;
    s_key[i] = s_tensor[i] == 0 ? rem / CPR : rem % KT;
    s_cg[i] = s_tensor[i] == 0 ? rem % CPR : rem / KT;
    const int byte = BITS * s_cg[i];  // chunk cg starts at byte BITS*cg of a row
    s_voff[i] = s_key[i] * p.R + (byte & ~3);
    s_shift[i] = (byte & 3) * 8;
    i_blk[i] = 0;
    i_pad[i] = 0;
  }

  // Packed bits in flight: tile j lands in register set A (j even) or B (j
  // odd) two iterations before its dequantization, so the wait for one set
  // leaves the newer set's loads outstanding.
  uint32_t preA[MAXI], pre2A[MAXI], preB[MAXI], pre2B[MAXI];
  int shA[MAXI], shB[MAXI];  // BW: bit shift of each item's chunk in its first word
  // fused launch: block k's rows are written below; tile 0 is fetched before
  // that only if it ends before block k, tile 1 always after (block-aligned
  // words: a chunk ending in the last word of block k - 1 also loads block k's
  // first word, whose bits it does not use)
  const bool early0 = FUSE == 0 || (int)p.fz.off >= KT;
  auto issue_loads = [&](int j, uint32_t (&pre)[MAXI], uint32_t (&pre2)[MAXI], int (&sh)[MAXI]) {
    if constexpr (BW) {
      // the whole prefix in one view: loads past its words return 0
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kpfx, pfx_bytes, 0, 0);
      const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vpfx, pfx_bytes, 0, 0);
#pragma unroll
      for (int i = 0; i < MAXI; ++i) {
        const int t = j * KT + s_key[i];
        while (i_blk[i] + 1 < nkb && t >= blk_end[i_blk[i]]) {  // keys only move forward
          ++i_blk[i];
          i_pad[i] = blk_pad[i_blk[i]];
        }
        const int voff = 4 * (int)word_of_code((uint32_t)(t * D + 8 * s_cg[i] + i_pad[i]), sh[i]);
        const __amdgpu_buffer_rsrc_t r = s_tensor[i] == 0 ? rk : rv;
        pre[i] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
        pre2[i] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4, 0, 0);
      }
      return;
    }
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kpfx, pfx_bytes, tile_bytes, j);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vpfx, pfx_bytes, tile_bytes, j);
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const __amdgpu_buffer_rsrc_t r = s_tensor[i] == 0 ? rk : rv;
      pre[i] = __builtin_amdgcn_raw_buffer_load_b32(r, s_voff[i], 0, 0);
      if constexpr (kTwoWords<BITS>)
        pre2[i] = __builtin_amdgcn_raw_buffer_load_b32(r, s_voff[i] + 4, 0, 0);
      else
        pre2[i] = 0u;
    }
  };
  if (early0) issue_loads(j_begin, preA, pre2A, shA);

  // ---- block ends and statistics to LDS, Q operand to registers -------------
  if constexpr (!BW)
    for (int i = tid; i < nkb; i += NT) blk_end[i] = p.block_end[i];
  {  // 8 binary16 values per copy; a fused launch writes block k's
    const int nkb_copy = FUSE != 0 ? nkb - 1 : nkb;
    for (int i = tid; i < nkb_copy * 2 * CPR; i += NT) {
      const int blk = i / (2 * CPR);
      const int rem = i - blk * 2 * CPR;
      const int tensor = rem / CPR;
      const int cg = rem - tensor * CPR;
      const int64_t gi = stat_base + (int64_t)blk * D + 8 * cg;
      _Float16* row = st + ((blk * 2 + tensor) * 2) * D + 8 * cg;
      const u32x4 zw = *reinterpret_cast<const u32x4*>((tensor == 0 ? p.kzero : p.vzero) + gi);
      const u32x4 sw = *reinterpret_cast<const u32x4*>((tensor == 0 ? p.kscale : p.vscale) + gi);
      *reinterpret_cast<u32x4*>(row) = zw;
      *reinterpret_cast<u32x4*>(row + D) = sw;
      if (tensor == 1) vover |= v_top_over_f16<BITS>(zw, sw);
    }
  }
  bf16x8 qop[KS];
  {
    const uint16_t* qrow = p.q + (((int64_t)b * p.n + (q_ok ? q : 0)) * p.H + h) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (q_ok) w = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
      qop[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // blk_end, statistics and (fused) block k's rows visible; every workgroup of
  // a (sequence, head) sees the same statistics, so key ranges agree on vhalf
  const bool vhalf = __syncthreads_or(vover) != 0;
  if (!early0) issue_loads(j_begin, preA, pre2A, shA);
  issue_loads(j_begin + 1, preB, pre2B, shB);  // no records past the prefix: reads nothing

  // binary16 statistics (8 channels of z and s) of one block for one tensor,
  // from LDS only (a read that may also go to global memory compiles to a flat
  // load, whose wait would also drain the next tile's prefetch)
  auto load_stats = [&](int blk, int tensor, int cg, f16x8& z, f16x8& s) {
    const _Float16* zr = st + ((blk * 2 + tensor) * 2) * D + 8 * cg;
    z = *reinterpret_cast<const f16x8*>(zr);
    s = *reinterpret_cast<const f16x8*>(zr + D);
  };

  // per-slot cache of the current block's statistics
  int s_blk[MAXI], s_next[MAXI];
  f16x8 s_z[MAXI], s_s[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    s_blk[i] = 0;
    s_next[i] = blk_end[0];
    load_stats(0, s_tensor[i], s_cg[i], s_z[i], s_s[i]);
  }

  auto dequant = [&](int j, int buf, const uint32_t (&pre)[MAXI], const uint32_t (&pre2)[MAXI],
                     const int (&sh)[MAXI]) {
    const int t0 = j * KT;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int t = t0 + s_key[i];
      const int cg = s_cg[i];
      if (t < n_prefix && t >= s_next[i]) {  // crossed into a later block
        do {
          ++s_blk[i];
          s_next[i] = blk_end[s_blk[i]];
        } while (t >= s_next[i]);
        load_stats(s_blk[i], s_tensor[i], cg, s_z[i], s_s[i]);
      }
      // keys past the prefix read codes 0 (buffer range check) and keep the
      // last block's statistics: finite values whose scores are masked out
      float cf[8], x[8];
      if constexpr (BW)
        chunk_words3_f32(pre[i], pre2[i], sh[i], cf);
      else
        chunk_f32<BITS>(pre[i], pre2[i], s_shift[i], cf);
#pragma unroll
      for (int c = 0; c < 8; ++c) x[c] = __builtin_fmaf(cf[c], (float)s_s[i][c], (float)s_z[i][c]);
      if (s_tensor[i] != 0 && vhalf) {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] *= 0.5f;
      }
      if (s_tensor[i] == 0) {
        u32x4 hi, lo;
#pragma unroll
        for (int c = 0; c < 8; c += 2) {
          const uint32_t u0 = __float_as_uint(x[c]);
          const uint32_t u1 = __float_as_uint(x[c + 1]);
          hi[c >> 1] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);  // high halves
          lo[c >> 1] = pk_bf16(x[c] - __uint_as_float(u0 & 0xFFFF0000u),
                               x[c + 1] - __uint_as_float(u1 & 0xFFFF0000u));
        }
        *reinterpret_cast<u32x4*>(&k_hi[buf][s_key[i]][8 * cg]) = hi;
        *reinterpret_cast<u32x4*>(&k_lo[buf][s_key[i]][8 * cg]) = lo;
      } else {
        // channel pairs of this key as fp16; the even-key lane writes channels
        // 0-3 and the odd-key lane channels 4-7, each as (even, odd) key pairs
        const uint32_t h01 = pk_f16(x[0], x[1]), h23 = pk_f16(x[2], x[3]);
        const uint32_t h45 = pk_f16(x[4], x[5]), h67 = pk_f16(x[6], x[7]);
        const bool odd = s_key[i] & 1;
        // each lane sends the half its neighbour writes: the even key's
        // channels 4-7, the odd key's channels 0-3
        const uint32_t ra = swap_adjacent(odd ? h01 : h45);
        const uint32_t rb = swap_adjacent(odd ? h23 : h67);
        const uint32_t lo_e = odd ? ra : h01;  // even key, first channel pair
        const uint32_t hi_e = odd ? rb : h23;  // even key, second channel pair
        const uint32_t lo_o = odd ? h45 : ra;  // odd key, first channel pair
        const uint32_t hi_o = odd ? h67 : rb;  // odd key, second channel pair
        const int d0 = 8 * cg + (odd ? 4 : 0);
        uint32_t* vrow = &v_t[buf][d0][s_key[i] >> 1];
        vrow[0 * VROW] = __builtin_amdgcn_perm(lo_o, lo_e, 0x05040100u);  // channel d0
        vrow[1 * VROW] = __builtin_amdgcn_perm(lo_o, lo_e, 0x07060302u);  // d0 + 1
        vrow[2 * VROW] = __builtin_amdgcn_perm(hi_o, hi_e, 0x05040100u);  // d0 + 2
        vrow[3 * VROW] = __builtin_amdgcn_perm(hi_o, hi_e, 0x07060302u);  // d0 + 3
      }
    }
  };

  f32x16 o[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) o[i] = f32x16{};
  const float c = p.scale_log2;
  const float slack = kRescaleLog2 / c;  // in raw score units
  float m_run = -__builtin_inff();
  float negmc = 0.0f;  // -m_run * c
  float l_run = 0.0f;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  dequant(j_begin, 0, preA, pre2A, shA);
  __syncthreads();

  // tile j: cur holds tile j+1's packed bits (issued one iteration earlier),
  // tile j+2's loads go into nxt
  auto step = [&](int j, const uint32_t (&cur)[MAXI], const uint32_t (&cur2)[MAXI],
                  const int (&cursh)[MAXI], uint32_t (&nxt)[MAXI], uint32_t (&nxt2)[MAXI],
                  int (&nxtsh)[MAXI]) {
    const int t0 = j * KT;
    const int buf = (j - j_begin) & 1;
    const bool has_next = j + 1 < j_end;
    issue_loads(j + 2, nxt, nxt2, nxtsh);  // unconditional: past the prefix it reads nothing

    if (wave_live) {
      // Phase stagger (8-wave workgroups): waves w and w + 4 share a SIMD and
      // would otherwise reach a tile's MFMA and VALU phases together.  The upper
      // half dequantizes tile j + 1 before its QK^T, so its VALU work runs beside
      // the lower half's MFMAs; at head_dim 64 the lower half dequantizes after
      // its PV (at 128, whose QK^T is twice as long, beside its own QK^T MFMAs).
      // Every wave's arithmetic is unchanged, only its order.
      const bool dq_first = NW == 8 && wave >= NW / 2;
      const bool dq_last = NW == 8 && D == 64 && wave < NW / 2;
      if (dq_first && has_next) dequant(j + 1, buf ^ 1, cur, cur2, cursh);
      // ---- S^T = K_hat Q^T -------------------------------------------------
      f32x16 s = f32x16{};
      bf16x8 ah[2], al[2];  // operands of the current and the next k-step
      ah[0] = *reinterpret_cast<const bf16x8*>(&k_hi[buf][col][8 * g]);
      al[0] = *reinterpret_cast<const bf16x8*>(&k_lo[buf][col][8 * g]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
          ah[(ks + 1) & 1] = *reinterpret_cast<const bf16x8*>(&k_hi[buf][col][16 * (ks + 1) + 8 * g]);
          al[(ks + 1) & 1] = *reinterpret_cast<const bf16x8*>(&k_lo[buf][col][16 * (ks + 1) + 8 * g]);
        }
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[ks & 1], qop[ks], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[ks & 1], qop[ks], s, 0, 0, 0);
      }
      // keep the operand reads ahead of the MFMAs that consume them (the
      // register budget of 4 waves per SIMD otherwise serializes them)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // the next tile's dequantization runs while these MFMAs complete
      if (!dq_first && !dq_last && has_next) dequant(j + 1, buf ^ 1, cur, cur2, cursh);

      // ---- online softmax (log2 domain) -----------------------------------
      if (t0 + KT > n_prefix) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 8 * (r >> 2) + 4 * g + (r & 3);
          if (t0 + key >= n_prefix) s[r] = -__builtin_inff();
        }
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
      mx = fmaxf(mx, s[15]);
      mx = max_xor32(mx);
      const bool raise = mx > m_run + slack;
      if (__any(raise)) {
        const float m_new = raise ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < MT; ++i) o[i] *= alpha;
        m_run = m_new;
        negmc = -m_new * c;
      }
      f16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, negmc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], c, negmc));
        const f16x2 hp = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p0, p1));
        l_run = __builtin_amdgcn_fdot2(hp, ones, l_run, false);
        pb[r >> 3][(r & 7)] = hp[0];
        pb[r >> 3][(r & 7) + 1] = hp[1];
      }

      // ---- O^T += V_hat^T P^T ------------------------------------------------
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const uint32_t* vr = &v_t[buf][32 * i + col][0];
          u32x4 aw;
          aw[0] = vr[8 * kk + 2 * g];
          aw[1] = vr[8 * kk + 2 * g + 1];
          aw[2] = vr[8 * kk + 4 + 2 * g];
          aw[3] = vr[8 * kk + 4 + 2 * g + 1];
          o[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, aw), pb[kk],
                                                         o[i], 0, 0, 0);
        }
      }
      if (dq_last && has_next) dequant(j + 1, buf ^ 1, cur, cur2, cursh);
    }

    if (!wave_live && has_next) dequant(j + 1, buf ^ 1, cur, cur2, cursh);
    __syncthreads();
  };
  int j = j_begin;
  for (; j + 1 < j_end; j += 2) {
    step(j, preB, pre2B, shB, preA, pre2A, shA);
    step(j + 1, preA, pre2A, shA, preB, pre2B, shB);
  }
  if (j < j_end) step(j, preB, pre2B, shB, preA, pre2A, shA);

  const float l_tot = sum_xor32(l_run);
  const float oscale = vhalf ? 2.0f : 1.0f;  // undo the v_hat halving
  if constexpr (SPLIT) {
    // ---- partial result of this key range: O unnormalized, m c, l ----------
#pragma unroll
    for (int i = 0; i < MT; ++i) o[i] *= oscale;
    if (q_ok) {
      const int64_t row = ((int64_t)b * p.n + q) * p.H + h;
      float* orow = p.ws_o + ((int64_t)sp * p.ws_rows + row) * D;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<f32x4*>(orow + 32 * i + 8 * r4 + 4 * g) =
              f32x4{o[i][4 * r4 + 0], o[i][4 * r4 + 1], o[i][4 * r4 + 2], o[i][4 * r4 + 3]};
      }
      if (g == 0) {
        float* ml = p.ws_ml + ((int64_t)sp * p.ws_rows + row) * 2;
        ml[0] = m_run * c;  // log2 units: p = exp2(s c - ml[0])
        ml[1] = l_tot;
      }
    }
    return;
  }

  // ---- normalize and store (fp32) ----------------------------------------
  const float inv_l = oscale / l_tot;
  if (q_ok) {
    float* orow = p.out + (((int64_t)b * p.n + q) * p.H + h) * D;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v;
        v[0] = o[i][4 * r4 + 0] * inv_l;
        v[1] = o[i][4 * r4 + 1] * inv_l;
        v[2] = o[i][4 * r4 + 2] * inv_l;
        v[3] = o[i][4 * r4 + 3] * inv_l;
        *reinterpret_cast<f32x4*>(orow + 32 * i + 8 * r4 + 4 * g) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused launch, quantize side: one wave quantizes and packs one (sequence,
// head)'s block of at most 32 tokens for K and V, with the same group
// statistics and code arithmetic as the standalone quantize kernel.
//   Phase 1: lane c owns channel c: its extremes over the block's tokens (one
//   coalesced 128-byte row per token) and its statistics, computed once.
//   Phase 2: lane (token lane tl, chunk cg) packs the codes of channels 8 cg ..
//   8 cg + 7 of tokens tl, tl + 8, .. with the statistics read from LDS.
// The statistics and packed rows also go to LDS for the attention that
// follows in the same launch; the cache writes serve later blocks.
// ---------------------------------------------------------------------------
// LDS bytes per packed row of the fused block: R = 8 * BITS at head_dim 64,
// plus the 4 bytes a two-dword chunk read may touch past the row
template <int BITS>
constexpr int kFusedRowBytes = BITS == 8 ? 64 : 32;

template <int D, int BITS, bool F32, bool CHECK, bool BW>
__device__ __forceinline__ void quantize_block_wave(const AttendParams& p, int b, int h, int lane,
                                                    _Float16* st_lds, uint8_t* rows_lds,
                                                    float* scratch, int& vover) {
  static_assert(D == kWave, "the wave quantizer covers 64-channel heads, one channel per lane");
  constexpr int CPR = D / 8;
  constexpr int TL = kWave / CPR;  // token lanes of phase 2
  constexpr int MAXR = KT / TL;    // rows per lane in phase 2
  constexpr float LEVELS = (float)((1 << BITS) - 1);
  const FuseParams& f = p.fz;
  const int n = p.n;
  const int64_t row_stride = (int64_t)p.H * D;
  const int64_t base = ((int64_t)b * n * p.H + h) * D;
  int flags = 0;
#pragma unroll
  for (int tensor = 0; tensor < 2; ++tensor) {
    // ---- phase 1: channel `lane` over the block's tokens
    float mn = __uint_as_float(0x7F800000u), mx = __uint_as_float(0xFF800000u);
    int bad = 0;
#pragma unroll 8
    for (int t = 0; t < n; ++t) {
      float x;
      if constexpr (F32)
        x = static_cast<const float*>(f.src[tensor])[base + t * row_stride + lane];
      else
        x = __uint_as_float((uint32_t)static_cast<const uint16_t*>(f.src[tensor])[base + t * row_stride + lane] << 16);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
      if constexpr (CHECK) bad |= !__builtin_isfinite(x);
    }
    const GroupStats gst = group_stats<CHECK>(mn, mx, LEVELS, flags);
    if constexpr (CHECK) {
      if (bad) flags |= KVQ_S_NONFINITE;
    }
    const int64_t so = (((int64_t)b * p.H + h) * p.NB + f.block) * D + lane;
    f.zero[tensor][so] = gst.zb;
    f.scale[tensor][so] = gst.sb;
    _Float16* srow = st_lds + ((f.block * 2 + tensor) * 2) * D;
    srow[lane] = __builtin_bit_cast(_Float16, gst.zb);
    srow[D + lane] = __builtin_bit_cast(_Float16, gst.sb);
    scratch[lane] = gst.zf;
    scratch[D + lane] = gst.inv;
    if (tensor == 1) vover |= __builtin_fmaf(LEVELS, h2f(gst.sb), gst.zf) > 65504.0f;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // ---- phase 2: codes of (token, 8-channel chunk) items
    const int cg = lane % CPR;
    const int tl = lane / CPR;
    float zf[8], inv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      zf[j] = scratch[8 * cg + j];
      inv[j] = scratch[D + 8 * cg + j];
    }
    uint8_t* rows = f.codes[tensor] + (((int64_t)b * p.H + h) * p.T_cache + f.off) * p.R;
    uint8_t* lrows = rows_lds + tensor * KT * kFusedRowBytes<BITS>;
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
      const int t = tl + TL * i;
      if (t < n) {
        const int64_t e = base + t * row_stride + 8 * cg;
        float x[8];
        if constexpr (F32) {
          const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(f.src[tensor]) + e);
          const f32x4 a0 = src[0], a1 = src[1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[j] = a0[j];
            x[j + 4] = a1[j];
          }
        } else {
          const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(f.src[tensor]) + e);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(w[j] << 16);
            x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
          }
        }
        const Packed8 pk = pack_chunk<BITS>(x, zf, inv);
        if constexpr (!BW) store_chunk<BITS>(rows + (int64_t)t * p.R + BITS * cg, pk);
        store_chunk<BITS>(lrows + t * p.R + BITS * cg, pk);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // scratch reuse, LDS rows written
    if constexpr (BW) {
      // the LDS rows are the block's dense stream: its words, one per lane
      uint32_t* wd = reinterpret_cast<uint32_t*>(
          f.codes[tensor] + (((int64_t)b * p.H + h) * p.bh_words + f.word_off) * 4);
      const int nc = n * D;
      for (int k = lane; k < (nc + 9) / 10; k += kWave) wd[k] = word_from_dense3(lrows, k, nc);
    }
  }
  if constexpr (CHECK) {
    if (flags) atomicOr(f.status, flags);
  }
}

// ---------------------------------------------------------------------------
// Short blocks (up to 32·QT queries, the early scales; launched with QT = 1): one wave owns one
// (sequence, head) and all its queries, four independent waves share a
// workgroup, and no workgroup barrier is needed.  Each lane dequantizes its
// key's half-rows of K straight into the QK^T operand registers (the two lanes
// of a key cover its channels once); V goes through a wave-private LDS
// transpose in (even, odd) key-pair dwords.  The wave's statistics are staged
// in its own LDS region.  Within one wave LDS accesses complete in issue order,
// so the transpose needs no barrier.
// ---------------------------------------------------------------------------
constexpr int kSmallWaves = 4;
constexpr int kSmallStatsHalves = 2048;  // 4 KB per wave: up to 8 blocks at head_dim 64

// FUSE: 0 attention only; 1/2 quantize the block first from bf16 (2: with
// input checks); 3/4 the same from fp32.
// BW: block-aligned 3-bit words (BITS == 3), addressed per tile from the
// lane's key's block; block k's rows in a fused launch still come from LDS in
// the dense row form.
template <int D, int BITS, int QT, int FUSE, bool BW = false>
// 3 waves per SIMD: with 4-wave workgroups every VAR-d20 (sequence, head) is
// resident in one dispatch round
__global__ __launch_bounds__(kSmallWaves * kWave)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 1))) void attend_small_kernel(AttendParams p) {
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;
  constexpr int MT = D / 32;
  constexpr int VI = KT * CPR / kWave;  // V items (key, chunk) per lane per tile
  __shared__ __align__(16) uint32_t v_t_all[kSmallWaves][D][VROW];
  __shared__ __align__(16) _Float16 st_all[kSmallWaves][kSmallStatsHalves];
  __shared__ int bend_all[kSmallWaves][KVQ_MAX_BLOCKS];
  __shared__ int bpad_all[kSmallWaves][BW ? KVQ_MAX_BLOCKS : 1];
  static_assert(!BW || BITS == 3, "block-aligned words are built for 3-bit codes");
  // fused launch: the packed rows of block k (K then V) for the attention below
  __shared__ __align__(16) uint8_t rows_all[kSmallWaves][FUSE != 0 ? 2 * KT * kFusedRowBytes<BITS> : 16];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int g = lane >> 5;
  const int col = lane & 31;
  const int bh = blockIdx.x * kSmallWaves + wave;
  if (bh >= p.B * p.H) return;  // the whole wave leaves; nothing below synchronizes waves
  uint32_t(*v_t)[VROW] = v_t_all[wave];
  _Float16* st = st_all[wave];  // [blk][tensor][z|s][D]
  int* bend = bend_all[wave];
  int* bpad = bpad_all[wave];
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int nkb = p.n_kblocks;
  const int n_prefix = p.n_prefix;
  const int n_tiles = (n_prefix + KT - 1) / KT;
  const int64_t stat_base = (int64_t)bh * p.NB * D;

  const uint8_t* kpfx = BW ? p.kcodes + (int64_t)bh * p.bh_words * 4 : p.kcodes + (int64_t)bh * p.T_cache * p.R;
  const uint8_t* vpfx = BW ? p.vcodes + (int64_t)bh * p.bh_words * 4 : p.vcodes + (int64_t)bh * p.T_cache * p.R;
  const int pfx_bytes = BW ? 4 * p.prefix_words : n_prefix * p.R;
  const int tile_bytes = KT * p.R;
  // K: this lane's key is `col`, its chunks are 2 ks + g; V items: key = it % KT
  int k_voff[KS], k_shift[KS], v_key[VI], v_cg[VI], v_voff[VI], v_shift[VI];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int byte = BITS * (2 * ks + g);
    k_voff[ks] = col * p.R + (byte & ~3);
    k_shift[ks] = (byte & 3) * 8;
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int it = lane + i * kWave;
    v_key[i] = it % KT;  // == col: 64 lanes cover two whole 32-key columns
    v_cg[i] = it / KT;
    const int byte = BITS * v_cg[i];
    v_voff[i] = v_key[i] * p.R + (byte & ~3);
    v_shift[i] = (byte & 3) * 8;
  }
  uint32_t kpre[KS][2], vpre[VI][2];
  // BW: V item i is chunk 2 i + g of key `col`, the same chunk as K k-step i,
  // so one word index and shift serve both tensors
  static_assert(VI == KS, "V items and K k-steps pair up");
  int wsh_pre[KS] = {};
  int ib = 0, ipad = 0;  // BW: block of this lane's key at its latest load, its padding
  if constexpr (BW) {
    if (lane < nkb) {
      bend[lane] = p.block_end[lane];
      bpad[lane] = p.block_pad[lane];
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
  auto issue_loads = [&](int j) {
    if constexpr (BW) {
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kpfx, pfx_bytes, 0, 0);
      const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vpfx, pfx_bytes, 0, 0);
      const int t = j * KT + col;
      while (ib + 1 < nkb && t >= bend[ib]) {
        ++ib;
        ipad = bpad[ib];
      }
      const uint32_t gi0 = (uint32_t)(t * D + 8 * g + ipad);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int voff = 4 * (int)word_of_code(gi0 + 16u * ks, wsh_pre[ks]);
        kpre[ks][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, voff, 0, 0);
        kpre[ks][1] = __builtin_amdgcn_raw_buffer_load_b32(rk, voff + 4, 0, 0);
        vpre[ks][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff, 0, 0);
        vpre[ks][1] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff + 4, 0, 0);
      }
      return;
    }
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kpfx, pfx_bytes, tile_bytes, j);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vpfx, pfx_bytes, tile_bytes, j);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kpre[ks][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, k_voff[ks], 0, 0);
      kpre[ks][1] = kTwoWords<BITS> ? __builtin_amdgcn_raw_buffer_load_b32(rk, k_voff[ks] + 4, 0, 0) : 0u;
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      vpre[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, v_voff[i], 0, 0);
      vpre[i][1] = kTwoWords<BITS> ? __builtin_amdgcn_raw_buffer_load_b32(rv, v_voff[i] + 4, 0, 0) : 0u;
    }
  };
  issue_loads(0);

  // the launcher only picks this kernel when every statistic fits the wave's
  // LDS; a fused launch writes block k's own statistics there itself
  const int nkb_copy = FUSE != 0 ? nkb - 1 : nkb;
  int vover = 0;  // a V group's top grid level leaves the binary16 range
  for (int i = lane; i < nkb_copy * 2 * CPR; i += kWave) {
    const int blk = i / (2 * CPR);
    const int rem = i - blk * 2 * CPR;
    const int tensor = rem / CPR;
    const int cg = rem - tensor * CPR;
    const int64_t gi = stat_base + (int64_t)blk * D + 8 * cg;
    _Float16* row = st + ((blk * 2 + tensor) * 2) * D + 8 * cg;
    const u32x4 zw = *reinterpret_cast<const u32x4*>((tensor == 0 ? p.kzero : p.vzero) + gi);
    const u32x4 sw = *reinterpret_cast<const u32x4*>((tensor == 0 ? p.kscale : p.vscale) + gi);
    *reinterpret_cast<u32x4*>(row) = zw;
    *reinterpret_cast<u32x4*>(row + D) = sw;
    if (tensor == 1) vover |= v_top_over_f16<BITS>(zw, sw);
  }
  if (!BW && lane < nkb) bend[lane] = p.block_end[lane];
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  bf16x8 qop[QT][KS];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int q = 32 * t + col;
    const bool ok = q < p.n;
    const uint16_t* qrow = p.q + (((int64_t)b * p.n + (ok ? q : 0)) * p.H + h) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (ok) w = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
      qop[t][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const bool live1 = QT > 1 && 32 < p.n;
  // Fused launch: quantize block k now (its loads overlap the ones above).
  // Rows of block k then come from LDS (keys off .. off + n - 1).
  const uint8_t* qrows = rows_all[wave];
  if constexpr (FUSE != 0)
    quantize_block_wave<D, BITS, FUSE >= 3, FUSE == 2 || FUSE == 4, BW>(
        p, b, h, lane, st, rows_all[wave], reinterpret_cast<float*>(&v_t[0][0]), vover);
  const bool vhalf = __any(vover);

  // Every K and V item of a lane is key `col` of the tile, so one block index
  // per lane follows the tiles; it only moves forward.
  int blk = 0;
  int blk_next = nkb > 1 ? bend[0] : INT32_MAX;
  auto stats = [&](int tensor, int cg, f16x8& z, f16x8& s) {
    const _Float16* zr = st + ((blk * 2 + tensor) * 2) * D + 8 * cg;
    z = *reinterpret_cast<const f16x8*>(zr);
    s = *reinterpret_cast<const f16x8*>(zr + D);
  };

  f32x16 o[QT][MT];
  float m_run[QT], negmc[QT], l_run[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
#pragma unroll
    for (int i = 0; i < MT; ++i) o[t][i] = f32x16{};
    m_run[t] = -__builtin_inff();
    negmc[t] = 0.0f;
    l_run[t] = 0.0f;
  }
  const float c = p.scale_log2;
  const float slack = kRescaleLog2 / c;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  for (int j = 0; j < n_tiles; ++j) {
    const int t0 = j * KT;
    uint32_t kc[KS][2], vc[VI][2];
    int wsh[KS];  // BW: shifts of this tile's chunks
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kc[ks][0] = kpre[ks][0];
      kc[ks][1] = kpre[ks][1];
      wsh[ks] = wsh_pre[ks];
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      vc[i][0] = vpre[i][0];
      vc[i][1] = vpre[i][1];
    }
    if (j + 1 < n_tiles) issue_loads(j + 1);
    // this lane's key; past the prefix its codes read 0 and dequantize to
    // finite values under the last block's statistics, masked in the scores
    const int tk = t0 + col;
    const bool live = tk < n_prefix;
    if constexpr (FUSE != 0) {
      const int r = tk - (int)p.fz.off;  // row within block k
      if (r >= 0 && live) {
        const uint8_t* kr = qrows + r * p.R;
        const uint8_t* vr = qrows + KT * kFusedRowBytes<BITS> + r * p.R;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int bo = k_voff[ks] - col * p.R;  // byte offset within the row
          kc[ks][0] = *reinterpret_cast<const uint32_t*>(kr + bo);
          if constexpr (kTwoWords<BITS>) kc[ks][1] = *reinterpret_cast<const uint32_t*>(kr + bo + 4);
        }
#pragma unroll
        for (int i = 0; i < VI; ++i) {
          const int bo = v_voff[i] - col * p.R;
          vc[i][0] = *reinterpret_cast<const uint32_t*>(vr + bo);
          if constexpr (kTwoWords<BITS>) vc[i][1] = *reinterpret_cast<const uint32_t*>(vr + bo + 4);
        }
        if constexpr (BW) {
          // dense LDS rows: the chunk's 24 bits as a word read from bit 0
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            kc[ks][0] = (uint32_t)(((uint64_t)kc[ks][1] << 32 | kc[ks][0]) >> k_shift[ks]);
            kc[ks][1] = 0u;
            vc[ks][0] = (uint32_t)(((uint64_t)vc[ks][1] << 32 | vc[ks][0]) >> v_shift[ks]);
            vc[ks][1] = 0u;
            wsh[ks] = 0;
          }
        }
      }
    }
    while (tk >= blk_next) {
      ++blk;
      blk_next = blk + 1 < nkb ? bend[blk] : INT32_MAX;
    }

    // ---- V: dequantize, pair keys across neighbouring lanes, transpose --------
    // (the previous tile's reads of v_t by other lanes precede these writes)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      f16x8 z, sc;
      stats(1, v_cg[i], z, sc);
      float cf[8], x[8];
      if constexpr (BW)
        chunk_words3_f32(vc[i][0], vc[i][1], wsh[i], cf);
      else
        chunk_f32<BITS>(vc[i][0], vc[i][1], v_shift[i], cf);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(cf[e], (float)sc[e], (float)z[e]);
      if (vhalf) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= 0.5f;
      }
      const uint32_t h01 = pk_f16(x[0], x[1]), h23 = pk_f16(x[2], x[3]);
      const uint32_t h45 = pk_f16(x[4], x[5]), h67 = pk_f16(x[6], x[7]);
      const bool odd = v_key[i] & 1;
      const uint32_t ra = swap_adjacent(odd ? h01 : h45);
      const uint32_t rb = swap_adjacent(odd ? h23 : h67);
      const uint32_t lo_e = odd ? ra : h01, hi_e = odd ? rb : h23;
      const uint32_t lo_o = odd ? h45 : ra, hi_o = odd ? h67 : rb;
      uint32_t* vrow = &v_t[8 * v_cg[i] + (odd ? 4 : 0)][v_key[i] >> 1];
      vrow[0 * VROW] = __builtin_amdgcn_perm(lo_o, lo_e, 0x05040100u);
      vrow[1 * VROW] = __builtin_amdgcn_perm(lo_o, lo_e, 0x07060302u);
      vrow[2 * VROW] = __builtin_amdgcn_perm(hi_o, hi_e, 0x05040100u);
      vrow[3 * VROW] = __builtin_amdgcn_perm(hi_o, hi_e, 0x07060302u);
    }

    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // V writes before PV reads

    // ---- S^T = K_hat Q^T, K_hat made in registers ------------------------------
    f32x16 s[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) s[t] = f32x16{};
    {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        f16x8 z, sc;
        stats(0, 2 * ks + g, z, sc);
        float cf[8], x[8];
        if constexpr (BW)
          chunk_words3_f32(kc[ks][0], kc[ks][1], wsh[ks], cf);
        else
          chunk_f32<BITS>(kc[ks][0], kc[ks][1], k_shift[ks], cf);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(cf[e], (float)sc[e], (float)z[e]);
        u32x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t u0 = __float_as_uint(x[e]);
          const uint32_t u1 = __float_as_uint(x[e + 1]);
          hi[e >> 1] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
          lo[e >> 1] = pk_bf16(x[e] - __uint_as_float(u0 & 0xFFFF0000u),
                               x[e + 1] - __uint_as_float(u1 & 0xFFFF0000u));
        }
        const bf16x8 ah = __builtin_bit_cast(bf16x8, hi), al = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          if (qt == 0 || live1) {
            s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qop[qt][ks], s[qt], 0, 0, 0);
            s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qop[qt][ks], s[qt], 0, 0, 0);
          }
        }
      }
    }

    // ---- softmax and O^T += V_hat^T P^T ----------------------------------------
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      if (qt == 1 && !live1) continue;
      f32x16& sv = s[qt];
      if (t0 + KT > n_prefix) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 8 * (r >> 2) + 4 * g + (r & 3);
          if (t0 + key >= n_prefix) sv[r] = -__builtin_inff();
        }
      }
      float mx = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, sv[r]), sv[r + 1]);
      mx = fmaxf(mx, sv[15]);
      mx = max_xor32(mx);
      const bool raise = mx > m_run[qt] + slack;
      if (__any(raise)) {
        const float m_new = raise ? mx : m_run[qt];
        const float alpha = __builtin_amdgcn_exp2f((m_run[qt] - m_new) * c);
        l_run[qt] *= alpha;
#pragma unroll
        for (int i = 0; i < MT; ++i) o[qt][i] *= alpha;
        m_run[qt] = m_new;
        negmc[qt] = -m_new * c;
      }
      f16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], c, negmc[qt]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r + 1], c, negmc[qt]));
        const f16x2 hp = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p0, p1));
        l_run[qt] = __builtin_amdgcn_fdot2(hp, ones, l_run[qt], false);
        pb[r >> 3][(r & 7)] = hp[0];
        pb[r >> 3][(r & 7) + 1] = hp[1];
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const uint32_t* vr = &v_t[32 * i + col][0];
          u32x4 aw;
          aw[0] = vr[8 * kk + 2 * g];
          aw[1] = vr[8 * kk + 2 * g + 1];
          aw[2] = vr[8 * kk + 4 + 2 * g];
          aw[3] = vr[8 * kk + 4 + 2 * g + 1];
          o[qt][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, aw), pb[kk],
                                                             o[qt][i], 0, 0, 0);
        }
      }
    }
  }

  // ---- normalize and store (fp32) ----------------------------------------
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float inv_l = (vhalf ? 2.0f : 1.0f) / sum_xor32(l_run[qt]);
    const int q = 32 * qt + col;
    if (q < p.n) {
      float* orow = p.out + (((int64_t)b * p.n + q) * p.H + h) * D;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 v;
          v[0] = o[qt][i][4 * r4 + 0] * inv_l;
          v[1] = o[qt][i][4 * r4 + 1] * inv_l;
          v[2] = o[qt][i][4 * r4 + 2] * inv_l;
          v[3] = o[qt][i][4 * r4 + 3] * inv_l;
          *reinterpret_cast<f32x4*>(orow + 32 * i + 8 * r4 + 4 * g) = v;
        }
      }
    }
  }
}

template <int D, int BITS, int QT, int FUSE = 0, bool BW = false>
hipError_t launch_small(const AttendParams& p, hipStream_t s) {
  AttendParams a = p;
  a.q_tiles = 1;
  const int64_t grid = ((int64_t)p.B * p.H + kSmallWaves - 1) / kSmallWaves;
  if (!dispatch_fits(grid, kSmallWaves * kWave)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attend_small_kernel<D, BITS, QT, FUSE, BW>), dim3((unsigned)grid),
                     dim3(kSmallWaves * kWave), 0, s, a);
  return hipGetLastError();
}

template <int D, int BITS, int NW, int FUSE = 0, int SPLIT = 0, bool BW = false>
hipError_t launch_nw(const AttendParams& p, hipStream_t s) {
  AttendParams a = p;
  a.q_tiles = (p.n + NW * 32 - 1) / (NW * 32);
  // every block's statistics in LDS: at most 64 blocks x 4 x D binary16
  // (32 KB at head_dim 64, 64 KB at 128)
  const size_t dyn = (size_t)p.n_kblocks * 4 * D * sizeof(_Float16);
  const int64_t grid = (int64_t)p.B * p.H * a.q_tiles * (SPLIT ? p.splits : 1);
  if (!dispatch_fits(grid, NW * kWave)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attend_kernel<D, BITS, NW, FUSE, SPLIT, BW>), dim3((unsigned)grid),
                     dim3(NW * kWave), dyn, s, a);
  return hipGetLastError();
}

// waves per workgroup: enough 32-query waves for the block, rounded to 1/2/4/8
template <int D, int BITS, bool BW = false>
hipError_t launch_t(const AttendParams& p, hipStream_t s) {
  // Up to 32 queries the one-wave kernel wins; from 33 on, measured on VAR-d20,
  // sharing each tile's dequantization among the block's waves does better.
  if (p.n <= 32 && p.n_kblocks * 4 * D <= kSmallStatsHalves)
    return launch_small<D, BITS, 1, 0, BW>(p, s);
  const int waves = (min(p.n, kMaxWaves * 32) + 31) / 32;
  if (waves <= 1) return launch_nw<D, BITS, 1, 0, 0, BW>(p, s);
  if (waves <= 2) return launch_nw<D, BITS, 2, 0, 0, BW>(p, s);
  if (waves <= 4) return launch_nw<D, BITS, 4, 0, 0, BW>(p, s);
  return launch_nw<D, BITS, 8, 0, 0, BW>(p, s);
}

}  // namespace

// head_dim x code width dispatch of a launcher template L<D, BITS>
#define KVQ_DISPATCH(L, head_dim, bits, ...)            \
  do {                                                  \
    switch ((head_dim) * 16 + (bits)) {                 \
      case 64 * 16 + 2: return L<64, 2>(__VA_ARGS__);   \
      case 64 * 16 + 3: return L<64, 3>(__VA_ARGS__);   \
      case 64 * 16 + 4: return L<64, 4>(__VA_ARGS__);   \
      case 64 * 16 + 8: return L<64, 8>(__VA_ARGS__);   \
      case 128 * 16 + 2: return L<128, 2>(__VA_ARGS__); \
      case 128 * 16 + 3: return L<128, 3>(__VA_ARGS__); \
      case 128 * 16 + 4: return L<128, 4>(__VA_ARGS__); \
      case 128 * 16 + 8: return L<128, 8>(__VA_ARGS__); \
      default: return hipErrorInvalidValue;             \
    }                                                   \
  } while (0)

// block-aligned 3-bit words: launcher template L<D, 3, true>
#define KVQ_DISPATCH_WORDS(L, head_dim, bits, ...)         \
  do {                                                     \
    if ((bits) != 3) return hipErrorInvalidValue;          \
    if ((head_dim) == 64) return L<64, 3, true>(__VA_ARGS__); \
    if ((head_dim) == 128) return L<128, 3, true>(__VA_ARGS__); \
    return hipErrorInvalidValue;                           \
  } while (0)

hipError_t launch_attend(const AttendParams& p, int head_dim, int bits, hipStream_t s) {
  if (p.word_layout) KVQ_DISPATCH_WORDS(launch_t, head_dim, bits, p, s);
  KVQ_DISPATCH(launch_t, head_dim, bits, p, s);
}

namespace {
// Merge of the key-range partials written by attend_kernel<.., SPLIT = 1>:
// with M = max_s ml_s (log2 units), out = sum_s 2^(ml_s - M) O_s divided by
// sum_s 2^(ml_s - M) l_s, the log-sum-exp combination of softmax pieces.  One
// thread per 4 channels of one output row (sequence, query, head).
template <int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(AttendParams p) {
  constexpr int C4 = D / 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / C4;
  if (row >= p.ws_rows) return;
  const int c4 = (int)(t - row * C4);
  float m = -__builtin_inff();
  for (int sp = 0; sp < p.splits; ++sp) m = fmaxf(m, p.ws_ml[((int64_t)sp * p.ws_rows + row) * 2]);
  f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
  float den = 0.0f;
  for (int sp = 0; sp < p.splits; ++sp) {
    const int64_t r = (int64_t)sp * p.ws_rows + row;
    const float w = __builtin_amdgcn_exp2f(p.ws_ml[r * 2] - m);
    den = __builtin_fmaf(w, p.ws_ml[r * 2 + 1], den);
    const f32x4 o = *reinterpret_cast<const f32x4*>(p.ws_o + r * D + 4 * c4);
#pragma unroll
    for (int k = 0; k < 4; ++k) num[k] = __builtin_fmaf(w, o[k], num[k]);
  }
  const float inv = 1.0f / den;
  *reinterpret_cast<f32x4*>(p.out + row * D + 4 * c4) =
      f32x4{num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv};
}

template <int D, int BITS, bool BW = false>
hipError_t launch_split_t(const AttendParams& p, hipStream_t s) {
  const int64_t merge_grid = (p.ws_rows * (D / 4) + 255) / 256;
  if (!dispatch_fits(merge_grid, 256)) return hipErrorInvalidConfiguration;
  const hipError_t e = launch_nw<D, BITS, kMaxWaves, 0, 1, BW>(p, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attend_merge_kernel<D>), dim3((unsigned)merge_grid), dim3(256), 0, s, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attend_split(const AttendParams& p, int head_dim, int bits, hipStream_t s) {
  if (p.word_layout) KVQ_DISPATCH_WORDS(launch_split_t, head_dim, bits, p, s);
  KVQ_DISPATCH(launch_split_t, head_dim, bits, p, s);
}

namespace {
template <int BITS, bool BW = false>
hipError_t launch_small_fused(const AttendParams& a, bool f32, bool check, hipStream_t s) {
  if (f32)
    return check ? launch_small<64, BITS, 1, 4, BW>(a, s) : launch_small<64, BITS, 1, 3, BW>(a, s);
  return check ? launch_small<64, BITS, 1, 2, BW>(a, s) : launch_small<64, BITS, 1, 1, BW>(a, s);
}
}  // namespace

static void fill_fuse(AttendParams& p, const QuantParams& q) {
  for (int t = 0; t < 2; ++t) {
    p.fz.src[t] = q.src[t];
    p.fz.codes[t] = q.codes[t];
    p.fz.zero[t] = q.zero[t];
    p.fz.scale[t] = q.scale[t];
  }
  p.fz.status = q.status;
  p.fz.off = q.off;
  p.fz.block = q.block;
  p.fz.word_off = q.word_off;
}

template <int D, int BITS, bool BW = false>
static hipError_t launch_wg_fused_d(const AttendParams& p, int waves, bool check, hipStream_t s) {
  if (waves <= 2)
    return check ? launch_nw<D, BITS, 2, 2, 0, BW>(p, s) : launch_nw<D, BITS, 2, 1, 0, BW>(p, s);
  if (waves <= 4)
    return check ? launch_nw<D, BITS, 4, 2, 0, BW>(p, s) : launch_nw<D, BITS, 4, 1, 0, BW>(p, s);
  return check ? launch_nw<D, BITS, 8, 2, 0, BW>(p, s) : launch_nw<D, BITS, 8, 1, 0, BW>(p, s);
}

template <int BITS, bool BW = false>
static hipError_t launch_wg_fused(const AttendParams& p, int head_dim, int waves, bool check,
                                  hipStream_t s) {
  return head_dim == 64 ? launch_wg_fused_d<64, BITS, BW>(p, waves, check, s)
                        : launch_wg_fused_d<128, BITS, BW>(p, waves, check, s);
}

hipError_t launch_quantize_attend(const QuantParams& q, const AttendParams& a, int head_dim,
                                  int bits, bool f32src, hipStream_t s) {
  const bool small = head_dim == 64 && a.n <= KT && a.n_kblocks * 4 * 64 <= kSmallStatsHalves;
  if (small) {
    AttendParams p = a;
    fill_fuse(p, q);
    const bool check = q.status != nullptr;
    if (a.word_layout)
      return bits == 3 ? launch_small_fused<3, true>(p, f32src, check, s) : hipErrorInvalidValue;
    switch (bits) {
      case 2: return launch_small_fused<2>(p, f32src, check, s);
      case 3: return launch_small_fused<3>(p, f32src, check, s);
      case 4: return launch_small_fused<4>(p, f32src, check, s);
      case 8: return launch_small_fused<8>(p, f32src, check, s);
      default: return hipErrorInvalidValue;
    }
  }
  // larger blocks: the workgroup kernels with one query tile per (sequence, head)
  const int waves = (a.n + 31) / 32;
  if ((head_dim == 64 || head_dim == 128) && !f32src && a.n <= kMaxWaves * 32 && waves >= 2) {
    AttendParams p = a;
    fill_fuse(p, q);
    const bool check = q.status != nullptr;
    if (a.word_layout)
      return bits == 3 ? launch_wg_fused<3, true>(p, head_dim, waves, check, s)
                       : hipErrorInvalidValue;
    switch (bits) {
      case 2: return launch_wg_fused<2>(p, head_dim, waves, check, s);
      case 3: return launch_wg_fused<3>(p, head_dim, waves, check, s);
      case 4: return launch_wg_fused<4>(p, head_dim, waves, check, s);
      case 8: return launch_wg_fused<8>(p, head_dim, waves, check, s);
      default: return hipErrorInvalidValue;
    }
  }
  const hipError_t e = launch_quantize(q, head_dim, bits, f32src, s);
  if (e != hipSuccess) return e;
  return launch_attend(a, head_dim, bits, s);
}

}  // namespace kvq
