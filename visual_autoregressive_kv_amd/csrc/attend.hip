// attend.hip -- block-causal decode attention over the packed VAR-Q cache (gfx950).
//
// Block-by-block decoding (VAR-Q abstract): the n_k queries of block k attend
// to every cached token of blocks 0..k.  One workgroup owns up to 256 queries of
// one (sequence, head); its waves own 32 queries each.  The packed prefix is
// streamed once per workgroup in tiles of 32 keys:
//   - the workgroup unpacks a tile's K and V codes and dequantizes them in
//     registers, k_hat = fma(code, s, z) with the (block, channel) statistics;
//     k_hat is split into a truncated bf16 high part and a bf16 remainder so
//     the two bf16 products reproduce it to ~2^-16; v_hat is rounded to fp16;
//     the results go to LDS (V transposed);
//   - each wave computes S^T = K_hat Q^T with v_mfma_f32_32x32x16_bf16 (hi and lo
//     accumulate into one fp32 tile), so every lane holds 16 keys of a single
//     query and the row maximum is a per-lane reduction plus one exchange;
//   - online softmax in the log2 domain; the running maximum is only moved when
//     a tile raises it by more than 2^8 (probabilities then stay <= 256, safe
//     in fp16), which skips the accumulator rescale on almost every tile;
//   - P (fp16, packed round-toward-zero) feeds O^T += V_hat^T P^T with
//     v_mfma_f32_32x32x16_f16 straight from registers: the 16 keys a lane holds
//     are exactly the 8+8 contraction slots its lane group supplies, so only
//     V's LDS reads follow that key order.
// Output is fp32 (bf16 output rounding alone would exceed the 2e-3 bound).
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = 32;       // keys per tile
constexpr int KPAD = 8;      // LDS row padding (elements)
constexpr int kMaxWaves = 8;
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int BITS>
__device__ __forceinline__ uint32_t load_code_bits(const uint8_t* row, int cg) {
  if constexpr (BITS == 4) {
    return *reinterpret_cast<const uint32_t*>(row + 4 * cg);
  } else {
    const int byte = 3 * cg;
    const int w = byte & ~3;
    const int shift = (byte & 3) * 8;
    uint64_t v = *reinterpret_cast<const uint32_t*>(row + w);
    if (shift > 8) v |= (uint64_t)(*reinterpret_cast<const uint32_t*>(row + w + 4)) << 32;
    return (uint32_t)(v >> shift) & 0xFFFFFFu;
  }
}

template <int D, int BITS>
__global__ __launch_bounds__(kMaxWaves * kWave) void attend_kernel(AttendParams p) {
  constexpr int CPR = D / 8;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  constexpr int KS = D / 16;  // k-steps of the QK^T contraction
  constexpr int MT = D / 32;  // 32-row tiles of O^T
  __shared__ __align__(16) __bf16 k_hi[KT][D + KPAD];
  __shared__ __align__(16) __bf16 k_lo[KT][D + KPAD];
  __shared__ __align__(16) _Float16 v_t[D][KT + KPAD];
  __shared__ int blk_end[KVQ_MAX_BLOCKS];

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int g = lane >> 5;    // lane group: which 8 of each 16 contraction slots
  const int col = lane & 31;  // this lane's query (S^T / O^T column)
  const int bh = blockIdx.x / p.q_tiles;
  const int qt = blockIdx.x - bh * p.q_tiles;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int q = qt * (nthreads / kWave) * 32 + wave * 32 + col;
  const bool q_ok = q < p.n;

  for (int i = tid; i < p.n_kblocks; i += nthreads) blk_end[i] = p.block_end[i];

  // Q^T operand: 8 bf16 per k-step, kept in registers for the whole prefix
  bf16x8 qop[KS];
  {
    const uint16_t* qrow = p.q + (((int64_t)b * p.n + q) * p.H + h) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (q_ok) w = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
      qop[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  const uint8_t* kc = p.kcodes + (int64_t)bh * p.T_cache * p.R;
  const uint8_t* vc = p.vcodes + (int64_t)bh * p.T_cache * p.R;
  const int64_t stat_base = (int64_t)bh * p.NB * D;

  for (int t0 = 0; t0 < p.n_prefix; t0 += KT) {
    __syncthreads();  // previous tile consumed (and blk_end visible)
    // ---- unpack + dequantize one tile of K and V into LDS ----------------
    for (int c = tid; c < 2 * KT * CPR; c += nthreads) {
      const int tensor = c / (KT * CPR);
      const int rem = c - tensor * (KT * CPR);
      const int key = rem / CPR;
      const int cg = rem - key * CPR;
      const int t = t0 + key;
      float x[8];
      if (t < p.n_prefix) {
        int blk = 0;
        while (blk < p.n_kblocks - 1 && t >= blk_end[blk]) ++blk;
        const uint8_t* row = (tensor == 0 ? kc : vc) + (int64_t)t * p.R;
        const uint32_t bits = load_code_bits<BITS>(row, cg);
        const int64_t so = stat_base + (int64_t)blk * D + 8 * cg;
        const u32x4 zw = *reinterpret_cast<const u32x4*>((tensor == 0 ? p.kzero : p.vzero) + so);
        const u32x4 sw = *reinterpret_cast<const u32x4*>((tensor == 0 ? p.kscale : p.vscale) + so);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t zj = (j & 1) ? (zw[j >> 1] >> 16) : (zw[j >> 1] & 0xFFFFu);
          const uint32_t sj = (j & 1) ? (sw[j >> 1] >> 16) : (sw[j >> 1] & 0xFFFFu);
          const float code = (float)((bits >> (BITS * j)) & MASK);
          x[j] = __builtin_fmaf(code, h2f((uint16_t)sj), h2f((uint16_t)zj));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = 0.0f;
      }
      if (tensor == 0) {
        u32x4 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const uint32_t u0 = __float_as_uint(x[j]) & 0xFFFF0000u;
          const uint32_t u1 = __float_as_uint(x[j + 1]) & 0xFFFF0000u;
          const float r0 = x[j] - __uint_as_float(u0);
          const float r1 = x[j + 1] - __uint_as_float(u1);
          hi[j >> 1] = (u0 >> 16) | u1;
          const __bf16 l0 = (__bf16)r0;
          const __bf16 l1 = (__bf16)r1;
          lo[j >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, l0) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        }
        *reinterpret_cast<u32x4*>(&k_hi[key][8 * cg]) = hi;
        *reinterpret_cast<u32x4*>(&k_lo[key][8 * cg]) = lo;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v_t[8 * cg + j][key] = (_Float16)x[j];
      }
    }
    __syncthreads();

    // ---- S^T = K_hat Q^T ---------------------------------------------------
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&k_hi[col][16 * ks + 8 * g]);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(&k_lo[col][16 * ks + 8 * g]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qop[ks], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qop[ks], s, 0, 0, 0);
    }

    // ---- online softmax (log2 domain) -------------------------------------
    float mt = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * g + (r & 3);
      const float v = (t0 + key < p.n_prefix) ? s[r] * p.scale_log2 : -__builtin_inff();
      s[r] = v;
      mt = fmaxf(mt, v);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = (mt > m_run + kRescaleSlack) ? mt : m_run;
    if (__any(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < MT; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    f16x8 pb[2];
    float lsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(s[r] - m_run);
      const float p1 = __builtin_amdgcn_exp2f(s[r + 1] - m_run);
      lsum += p0 + p1;
      const f16x2 hp = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p0, p1));
      pb[r >> 3][(r & 7)] = hp[0];
      pb[r >> 3][(r & 7) + 1] = hp[1];
    }
    l_run += lsum;

    // ---- O^T += V_hat^T P^T --------------------------------------------------
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int d = 32 * i + col;
        const f16x4 a0 = *reinterpret_cast<const f16x4*>(&v_t[d][16 * kk + 4 * g]);
        const f16x4 a1 = *reinterpret_cast<const f16x4*>(&v_t[d][16 * kk + 8 + 4 * g]);
        const f16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        o[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[kk], o[i], 0, 0, 0);
      }
    }
  }

  // ---- normalize and store (fp32) ----------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv_l = 1.0f / l_tot;
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

template <int D, int BITS>
hipError_t launch_t(const AttendParams& p, hipStream_t s) {
  const int rows = min(p.n, kMaxWaves * 32);
  const int waves = (rows + 31) / 32;
  AttendParams a = p;
  a.q_tiles = (p.n + waves * 32 - 1) / (waves * 32);
  const int64_t grid = (int64_t)p.B * p.H * a.q_tiles;
  hipLaunchKernelGGL((attend_kernel<D, BITS>), dim3((unsigned)grid), dim3(waves * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const AttendParams& p, int head_dim, int bits, hipStream_t s) {
  if (head_dim == 64) return bits == 4 ? launch_t<64, 4>(p, s) : launch_t<64, 3>(p, s);
  return bits == 4 ? launch_t<128, 4>(p, s) : launch_t<128, 3>(p, s);
}

}  // namespace kvq
