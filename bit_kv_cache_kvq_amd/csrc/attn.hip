// jb_attn: Jensen-bias-corrected chunk attention over a quantized KV cache (gfx950).
//
// Paper: "Quantized Keys Steal Attention" (arXiv 2605.26266). Abstract and §1: the
// current chunk's queries attend to a cached window of earlier chunks (quantized, §3)
// and to their own chunk (not quantized); a correction b, computed on the fly from the
// cached keys' step sizes and the query, is subtracted from every cached-key score
// before the softmax (Fig. 3 caption: uniform rounding noise inflates E[e^score]);
// Fig. 2: the cached/current attention masses P_S and P_R. b is the second-order
// Taylor form s^2 sum_c q'_c^2 Delta_c^2 / 24 of that inflation (per token:
// s^2 |q|^2 Delta_j^2 / 24).
//
// Kernel design (one workgroup = 8 waves = 256 queries of one head; a wave owns 32
// queries and streams 64-key tiles through a two-stage LDS pipeline, one barrier per
// tile, the next tile's global loads in flight during the current tile's math):
//  * Scores are computed transposed, S^T = K Q^T, so keys are the MFMA M dimension and
//    each lane owns one query: per-query softmax state lives in one lane (and its
//    partner lane l^32, which holds the other half of each key block).
//  * Cached QK^T runs on int8 MFMA (v_mfma_i32_32x32x32_i8): the rotated query
//    q' = H q is a 16-bit fixed-point integer (scale sigma) split into signed hi/lo
//    bytes, the key operand is the raw 2- or 4-bit code, unpacked in registers with
//    shifts and masks; integer accumulation is exact: S = 256 S_hi + S_lo.
//  * The zero point and the correction enter through one fp16 MFMA per 32x32 block whose
//    key operand is (z_j, z_j, Delta_j, Delta_j) and whose query operand is the hi/lo
//    fp16 split of (-A sum(q_fixed), -G): bias_ij = -A z_j sum(q_fixed) - G Delta_j.
//    Logit in log2 units: x = Delta_j (A S + bias), A = s sigma log2 e,
//    G = s^2 |q'|^2 / 24 log2 e.
//  * Softmax with a lazy running max m: p = exp2(Delta_j * inner - m) in one fma and one
//    exp; the exact max and the rescale run only when a tile's p exceeds 2^8 (or for a
//    ragged tile), so P values stay below 2^8 and in fp16 range.
//  * PV runs on fp16 MFMA: P~ = p Delta^V_j rounded to fp16, times (code - z) exact in
//    fp16, unpacked once per workgroup into LDS (channel-major rows). A fixed key
//    permutation inside each 32-key block lets P~ feed the B operand straight from the
//    score registers.
//  * The cached PV sum lives in the rotated basis; it is un-rotated once (an FWHT across
//    the accumulator registers) before the current chunk is processed with bf16 QK^T
//    and fp16 PV. One online softmax (shared running max, separate sums l_S, l_R)
//    covers both phases.
#include <math.h>

#include "common.h"

namespace kvq {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kQFix = 32639.f;  // |q_fixed| <= 32639 keeps hi = (q+128)>>8 in int8
constexpr float kLazy = 256.f;    // 2^8: largest p allowed before the running max is raised

struct Params {
  int B, H, n_q, n_r, chunk_len, n_chunks, cp;
  int n_qblk;
  const uint16_t* q;
  const uint16_t* k_cur;
  const uint16_t* v_cur;
  const uint32_t* k_codes;
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint32_t* v_codes;
  const uint16_t* v_scale;
  const uint16_t* v_zero;
  float s;
  int correction;
  int k_had, v_had;
  float* o;
  float* mass_s;
  float* mass_r;
};

// Key position (0..31) inside a 32-key block held by M-row r of the S^T accumulator.
// The order makes each 8-value slice of a lane's accumulator registers line up with
// the PV operand order (positions p = 2j + e <-> key j + 8e in every 16-key group).
__device__ __host__ inline int mrow_key(int r) {
  const int b = r & 3, h = (r >> 2) & 1, a = (r >> 3) & 1, vh = (r >> 4) & 1;
  return 16 * vh + 4 * h + 2 * a + (b >> 1) + 8 * (b & 1);
}
__device__ __host__ inline int key_mrow(int k) {
  const int vh = (k >> 4) & 1, b1 = (k >> 3) & 1, h = (k >> 2) & 1, a = (k >> 1) & 1, b0 = k & 1;
  return (2 * b0 + b1) + 4 * h + 8 * a + 16 * vh;
}

// Channel offset (0..15) inside a 16-channel slice for byte b of unpacked dword j.
template <int BITS>
__device__ __host__ constexpr int kperm(int j, int b) {
  return BITS == 2 ? 4 * b + j : 8 * (j >> 1) + 2 * b + (j & 1);
}

__device__ inline float half_bits_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

__device__ inline uint32_t pack_f16x2(float lo, float hi) {
  f16x2 r;
  r[0] = (_Float16)lo;
  r[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ inline float xor32(float v) { return __shfl_xor(v, 32); }
__device__ inline float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// Map a linear workgroup id to (query block, head) so that all query blocks of a head
// run on the same XCD (workgroups are dealt to the 8 XCDs round-robin), keeping that
// head's cache window in one L2.
__device__ inline void xcd_map(int L, int total, int n_qblk, int& qb, int& bh) {
  const int per = (total + 7) / 8;
  int tall = total % 8;
  if (tall == 0) tall = 8;
  const int xcd = L % 8, local = L / 8;
  const int w = xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
  qb = w % n_qblk;
  bh = w / n_qblk;
}

template <int D, int BITS>
struct TileBuf {
  static constexpr int KW = D * BITS / 32;  // key words per token
  static constexpr int VROW = kBN + 8;      // fp16 per value row (padded against bank conflicts)
  alignas(16) uint32_t k_words[kBN][KW];    // cached keys, natural token order
  alignas(16) _Float16 v[D][VROW];          // (code - z) or current-chunk values, channel-major
  alignas(16) uint16_t kr[kBN][D + 8];      // current-chunk keys (bf16), natural order
  alignas(16) float dk[kBN];                // per key, M-row order
  alignas(16) float dv[kBN];
  alignas(16) float mask[kBN];
  alignas(16) uint2 kb[kBN];                // bias operand: (z, z), (Delta, Delta) as fp16
};

template <int D, int BITS>
struct Smem {
  TileBuf<D, BITS> buf[2];
  alignas(16) uint32_t zv_pair[2][kBN / 2];  // (-1024 - z) fp16 pairs of a tile's value tokens
};

template <int D, int BITS, bool MASS_ONLY>
__global__ __launch_bounds__(kThreads) void jb_attn_kernel(const Params p) {
  constexpr int HALF = D / 2;
  constexpr int KSTEPS = D / 32;  // int8 K-steps of 32 channels
  constexpr int CBLK = D / 32;    // 32-channel output blocks
  constexpr int CPW = 32 / BITS;
  constexpr int KW = D * BITS / 32;    // key words per token
  constexpr int VWPC = kBN / CPW;      // value words per channel per 64-token block
  constexpr int KWT = kBN * KW;        // key words per tile
  constexpr int VWT = D * VWPC;        // value words per tile
  __shared__ Smem<D, BITS> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  int qb, bh;
  xcd_map(blockIdx.x, gridDim.x, p.n_qblk, qb, bh);
  const int qi = qb * kBM + wave * 32 + col;  // this lane's query
  const bool q_ok = qi < p.n_q;

  // ---------------- prologue: rotated query as 16-bit fixed point, hi/lo bytes --------
  i32x4 qhi[KSTEPS], qlo[KSTEPS];
  f16x8 qbias;  // B operand of the bias MFMA
  float A;
  {
    float qv[HALF];
    const uint16_t* qrow = p.q + ((size_t)bh * p.n_q + (q_ok ? qi : 0)) * D + HALF * h;
#pragma unroll
    for (int u = 0; u < HALF / 8; u++) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (q_ok) w = reinterpret_cast<const uint4*>(qrow)[u];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        qv[8 * u + 2 * e] = __uint_as_float(ww[e] << 16);
        qv[8 * u + 2 * e + 1] = __uint_as_float(ww[e] & 0xFFFF0000u);
      }
    }
    if (p.k_had) {
#pragma unroll
      for (int hh = 1; hh < HALF; hh <<= 1)
#pragma unroll
        for (int i = 0; i < HALF; i++)
          if ((i & hh) == 0) {
            const float a = qv[i], b = qv[i + hh];
            qv[i] = a + b;
            qv[i + hh] = a - b;
          }
      const float c = rsqrtf((float)D);
#pragma unroll
      for (int i = 0; i < HALF; i++) {
        const float pv = xor32(qv[i]);
        qv[i] = (h ? (pv - qv[i]) : (qv[i] + pv)) * c;
      }
    }
    float ss = 0.f, mxa = 0.f;
#pragma unroll
    for (int i = 0; i < HALF; i++) {
      ss += qv[i] * qv[i];
      mxa = fmaxf(mxa, fabsf(qv[i]));
    }
    ss += xor32(ss);
    mxa = fmaxf(mxa, xor32(mxa));
    const float inv = mxa > 0.f ? kQFix / mxa : 0.f;
    const float sigma = mxa > 0.f ? mxa / kQFix : 0.f;
    int qs = 0;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; kk++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        uint32_t whi = 0, wlo = 0;
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int qf = (int)__builtin_rintf(qv[16 * kk + kperm<BITS>(j, b)] * inv);
          const int hi = (qf + 128) >> 8;
          const int lo = qf - (hi << 8);
          qs += qf;
          whi |= (uint32_t)(hi & 0xFF) << (8 * b);
          wlo |= (uint32_t)(lo & 0xFF) << (8 * b);
        }
        qhi[kk][j] = (int)whi;
        qlo[kk][j] = (int)wlo;
      }
    qs += __shfl_xor(qs, 32);
    A = p.s * sigma * kLog2e;
    const float G = p.correction ? p.s * p.s * ss * (1.f / 24.f) * kLog2e : 0.f;
    // bias = z_j * (-A qs) + Delta_j * (-G), each factor split into fp16 hi + lo
    const float bz = -A * (float)qs, bd = -G;
    const _Float16 bz_hi = (_Float16)bz, bd_hi = (_Float16)bd;
    const _Float16 bz_lo = (_Float16)(bz - (float)bz_hi), bd_lo = (_Float16)(bd - (float)bd_hi);
#pragma unroll
    for (int e = 0; e < 8; e++) qbias[e] = (_Float16)0.f;
    if (h == 0) {
      qbias[0] = bz_hi;
      qbias[1] = bz_lo;
      qbias[2] = bd_hi;
      qbias[3] = bd_lo;
    }
  }

  float m_run = -INFINITY, l_s = 0.f, l_r = 0.f;
  f32x16 acc[CBLK];
#pragma unroll
  for (int c = 0; c < CBLK; c++)
#pragma unroll
    for (int v = 0; v < 16; v++) acc[c][v] = 0.f;

  // Exact max + rescale for a tile whose logits x (log2 units, masked) are given; the
  // returned x hold p = exp2(x - m_run).
  auto exact_tile = [&](float (&x)[2][16]) {
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
      for (int v = 0; v < 16; v++) mx = fmaxf(mx, x[mb][v]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run) != 0) {
      const float sc = exp2_(m_run - m_new);
      l_s *= sc;
      l_r *= sc;
      if (!MASS_ONLY) {
#pragma unroll
        for (int c = 0; c < CBLK; c++)
#pragma unroll
          for (int v = 0; v < 16; v++) acc[c][v] *= sc;
      }
      m_run = m_new;
    }
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
      for (int v = 0; v < 16; v++) x[mb][v] = exp2_(x[mb][v] - m_run);
  };

  // PV for one tile: B operand = P (fp16 pairs from the score registers), A = value rows in LDS.
  auto pv_tile = [&](const TileBuf<D, BITS>& tb, const uint32_t (&pb)[4][4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(pb[ks][0], pb[ks][1], pb[ks][2], pb[ks][3]));
#pragma unroll
      for (int c = 0; c < CBLK; c++) {
        const f16x8 aop = *reinterpret_cast<const f16x8*>(&tb.v[32 * c + col][16 * ks + 8 * h]);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop, acc[c], 0, 0, 0);
      }
    }
  };

  // ---------------- phase 1: cached window ----------------
  const int tiles_per_chunk = p.cp / kBN;
  const int n_tiles = p.n_chunks * tiles_per_chunk;
  const size_t n_tot = (size_t)p.n_chunks * p.cp;
  const uint32_t* kc_base = p.k_codes + (size_t)bh * n_tot * KW;
  const uint32_t* vc_base = p.v_codes + (size_t)bh * (n_tot / kBN) * VWT;
  const uint16_t* ks_base = p.k_scale + (size_t)bh * n_tot;
  const uint16_t* kz_base = p.k_zero + (size_t)bh * n_tot;
  const uint16_t* vs_base = p.v_scale + (size_t)bh * n_tot;
  const uint16_t* vz_base = p.v_zero + (size_t)bh * n_tot;


  // ---- prefetch registers: key words, one 16-token group of value words, per-key fp16 ----
  constexpr int KPT = KWT >= kThreads ? KWT / kThreads : 1;  // key words per thread (contiguous)
  constexpr int WPG = BITS / 2;                                // value words per 16-token group
  constexpr int VGT = D * (kBN / 16);                          // value groups per tile (<= kThreads)
  static_assert(KWT <= 2 * kThreads && VGT <= kThreads, "tile staging assumes at most 2 words per thread");
  uint32_t kwr[KPT], vwr[WPG];
  uint32_t pk_dk = 0, pk_zk = 0, pk_dv = 0;  // per-key fp16 bits (threads < kBN)
  uint32_t pz0 = 0, pz1 = 0;                 // value zero points of a token pair (threads < kBN/2)
#pragma unroll
  for (int e = 0; e < KPT; e++) kwr[e] = 0;
#pragma unroll
  for (int e = 0; e < WPG; e++) vwr[e] = 0;

  auto load_tile = [&](int T) {
    const size_t tok0 = (size_t)T * kBN;
    if (tid * KPT < KWT) {
      const uint32_t* src = kc_base + tok0 * KW + tid * KPT;
      if constexpr (KPT == 2) {
        const uint2 w = *reinterpret_cast<const uint2*>(src);
        kwr[0] = w.x;
        kwr[KPT - 1] = w.y;
      } else {
        kwr[0] = src[0];
      }
    }
    if (!MASS_ONLY && tid < VGT) {
      const uint32_t* src = vc_base + (size_t)T * VWT + tid * WPG;
      if constexpr (WPG == 2) {
        const uint2 w = *reinterpret_cast<const uint2*>(src);
        vwr[0] = w.x;
        vwr[WPG - 1] = w.y;
      } else {
        vwr[0] = src[0];
      }
    }
    if (tid < kBN) {
      pk_dk = ks_base[tok0 + tid];
      pk_zk = kz_base[tok0 + tid];
      if (!MASS_ONLY) pk_dv = vs_base[tok0 + tid];
    }
  };
  auto load_zv = [&](int T) {
    if (!MASS_ONLY && tid < kBN / 2) {
      const size_t tok0 = (size_t)T * kBN;
      const int g = tid >> 3, j = tid & 7;
      pz0 = vz_base[tok0 + 16 * g + j];
      pz1 = vz_base[tok0 + 16 * g + j + 8];
    }
  };
  auto store_zv = [&](int slot) {
    if (!MASS_ONLY && tid < kBN / 2)
      sm.zv_pair[slot][tid] = pack_f16x2(-1024.f - half_bits_to_f32(pz0), -1024.f - half_bits_to_f32(pz1));
  };
  // Key words, per-key values and the unpacked value tile of tile T (its zero-point
  // pairs must already be visible in zv_pair[T & 1]).
  auto store_tile = [&](int T, TileBuf<D, BITS>& tb) {
    if (tid * KPT < KWT) {
      uint32_t* dst = &tb.k_words[0][0] + tid * KPT;
      if constexpr (KPT == 2)
        *reinterpret_cast<uint2*>(dst) = make_uint2(kwr[0], kwr[KPT - 1]);
      else
        dst[0] = kwr[0];
    }
    if (tid < kBN) {
      const int r = 32 * (tid >> 5) + key_mrow(tid & 31);
      const int nvalid = min(kBN, p.chunk_len - (T % tiles_per_chunk) * kBN);
      tb.dk[r] = half_bits_to_f32(pk_dk);
      tb.dv[r] = half_bits_to_f32(pk_dv);
      tb.mask[r] = tid < nvalid ? 0.f : -INFINITY;
      tb.kb[r] = make_uint2((pk_zk & 0xFFFFu) | (pk_zk << 16), (pk_dk & 0xFFFFu) | (pk_dk << 16));
    }
    if (!MASS_ONLY && tid < VGT) {
      const int ch = tid >> 2, g = tid & 3;  // 16-token group g of channel ch
      const uint4* zp = reinterpret_cast<const uint4*>(&sm.zv_pair[T & 1][8 * g]);
      const uint4 z0 = zp[0], z1 = zp[1];
      const uint32_t zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
      uint32_t a[8];
      if constexpr (BITS == 2) {
        const uint32_t w = vwr[0];
#pragma unroll
        for (int j = 0; j < 8; j++) a[j] = ((w >> (2 * j)) & 0x00030003u) | 0x64006400u;
      } else {
        // t0 = [w0.b0 w0.b1 w1.b0 w1.b1], t1 = [w0.b2 w0.b3 w1.b2 w1.b3]
        const uint32_t w0 = vwr[0], w1 = vwr[WPG - 1];
        const uint32_t t0 = (w0 & 0xFFFFu) | (w1 << 16);
        const uint32_t t1 = (w0 >> 16) | (w1 & 0xFFFF0000u);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          a[j] = ((t0 >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
          a[4 + j] = ((t1 >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        }
      }
      uint32_t res[8];
#pragma unroll
      for (int j = 0; j < 8; j++)
        res[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a[j]) + __builtin_bit_cast(f16x2, zz[j]));
      uint4* dst = reinterpret_cast<uint4*>(&tb.v[ch][16 * g]);
      dst[0] = make_uint4(res[0], res[1], res[2], res[3]);
      dst[1] = make_uint4(res[4], res[5], res[6], res[7]);
    }
  };

  // Lazy softmax over one tile: inner scores are turned into p = exp2(scale*inner - m)
  // by one fma and one exp when that keeps every p <= 2^8; otherwise (and for ragged
  // tiles, which need the mask) the exact max path runs. scl[mb][v] multiplies inner.
  auto softmax_tile = [&](const f32x16 (&inner)[2], const float (&scl)[2][16], bool ragged,
                          const float* mask_rows, float (&pv)[2][16]) {
    bool fast = !ragged;
    if (fast) {
      float pmax = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int v = 0; v < 16; v++) {
          pv[mb][v] = exp2_(fmaf(scl[mb][v], inner[mb][v], -m_run));
          pmax = fmaxf(pmax, pv[mb][v]);
        }
      pmax = fmaxf(pmax, xor32(pmax));
      fast = __ballot(!(pmax <= kLazy)) == 0;
    }
    if (!fast) {
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int v = 0; v < 16; v++) {
          pv[mb][v] = scl[mb][v] * inner[mb][v];
          if (ragged) pv[mb][v] += mask_rows[32 * mb + (v & 3) + 8 * (v >> 2) + 4 * h];
        }
      exact_tile(pv);
    }
  };

  auto compute_cached = [&](int T, const TileBuf<D, BITS>& tb) {
    const int nvalid = min(kBN, p.chunk_len - (T % tiles_per_chunk) * kBN);
    i32x16 shi[2], slo[2];
    f32x16 inner[2];
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      const int key = 32 * mb + mrow_key(col);
      uint32_t kw[KW / 2];
      if constexpr (KW / 2 == 4) {
        const uint4 w = *reinterpret_cast<const uint4*>(&tb.k_words[key][(KW / 2) * h]);
        kw[0] = w.x; kw[1] = w.y; kw[2] = w.z; kw[3] = w.w;
      } else if constexpr (KW / 2 == 8) {
        const uint4 w0 = *reinterpret_cast<const uint4*>(&tb.k_words[key][(KW / 2) * h]);
        const uint4 w1 = *reinterpret_cast<const uint4*>(&tb.k_words[key][(KW / 2) * h + 4]);
        kw[0] = w0.x; kw[1] = w0.y; kw[2] = w0.z; kw[3] = w0.w;
        kw[4 % (KW / 2)] = w1.x; kw[5 % (KW / 2)] = w1.y; kw[6 % (KW / 2)] = w1.z; kw[7 % (KW / 2)] = w1.w;
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(&tb.k_words[key][(KW / 2) * h]);
        kw[0] = w.x; kw[1 % (KW / 2)] = w.y;
      }
#pragma unroll
      for (int kk = 0; kk < KSTEPS; kk++) {
        i32x4 aop;
        if constexpr (BITS == 2) {
          const uint32_t w = kw[kk];
#pragma unroll
          for (int j = 0; j < 4; j++) aop[j] = (int)((w >> (2 * j)) & 0x03030303u);
        } else {
          const uint32_t w0 = kw[2 * kk], w1 = kw[2 * kk + 1];
          aop[0] = (int)(w0 & 0x0F0F0F0Fu);
          aop[1] = (int)((w0 >> 4) & 0x0F0F0F0Fu);
          aop[2] = (int)(w1 & 0x0F0F0F0Fu);
          aop[3] = (int)((w1 >> 4) & 0x0F0F0F0Fu);
        }
        if (kk == 0) {
          const i32x16 z = {};
          shi[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, qhi[kk], z, 0, 0, 0);
          slo[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, qlo[kk], z, 0, 0, 0);
        } else {
          shi[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, qhi[kk], shi[mb], 0, 0, 0);
          slo[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, qlo[kk], slo[mb], 0, 0, 0);
        }
      }
      const uint2 kb = tb.kb[32 * mb + col];
      const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(kb.x, kb.y, 0u, 0u));
      const f32x16 zf = {};
      inner[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bop, qbias, zf, 0, 0, 0);
    }
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
      for (int v = 0; v < 16; v++) inner[mb][v] = fmaf(A, (float)((shi[mb][v] << 8) + slo[mb][v]), inner[mb][v]);
    float dk[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const float4 d4 = *reinterpret_cast<const float4*>(&tb.dk[32 * mb + 8 * v4 + 4 * h]);
        dk[mb][4 * v4] = d4.x; dk[mb][4 * v4 + 1] = d4.y; dk[mb][4 * v4 + 2] = d4.z; dk[mb][4 * v4 + 3] = d4.w;
      }
    float pv[2][16];
    softmax_tile(inner, dk, nvalid < kBN, tb.mask, pv);
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
      for (int v = 0; v < 16; v++) l_s += pv[mb][v];
    if (!MASS_ONLY) {
      uint32_t pb[4][4];
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int v4 = 0; v4 < 4; v4++) {
          const float4 dv4 = *reinterpret_cast<const float4*>(&tb.dv[32 * mb + 8 * v4 + 4 * h]);
          const int v = 4 * v4;
          const int ks = 2 * mb + (v4 >> 1), slot = 2 * (v4 & 1);
          pb[ks][slot] = pack_f16x2(pv[mb][v] * dv4.x, pv[mb][v + 1] * dv4.y);
          pb[ks][slot + 1] = pack_f16x2(pv[mb][v + 2] * dv4.z, pv[mb][v + 3] * dv4.w);
        }
      pv_tile(tb, pb);
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    load_zv(0);
    store_zv(0);
    if (n_tiles > 1) {
      load_zv(1);
      store_zv(1);
    }
    __syncthreads();
    store_tile(0, sm.buf[0]);
    __syncthreads();
    for (int T = 0; T < n_tiles; T++) {
      const int cur = T & 1;
      const bool has_next = T + 1 < n_tiles;
      if (has_next) load_tile(T + 1);
      if (T + 2 < n_tiles) load_zv(T + 2);
      compute_cached(T, sm.buf[cur]);
      if (has_next) store_tile(T + 1, sm.buf[cur ^ 1]);
      if (T + 2 < n_tiles) store_zv(cur);  // tile T+2 uses slot (T+2) & 1 == cur
      __syncthreads();
    }
  }

  // ---------------- phase switch: un-rotate the cached PV sum ----------------
  if (!MASS_ONLY && p.v_had && n_tiles > 0) {
    // acc[c][v] holds channel 32c + (v&3) + 8(v>>2) + 4h of this lane's query.
#pragma unroll
    for (int bit = 0; bit < 4; bit++) {  // channel bits 0,1 (v bits 0,1) and 3,4 (v bits 2,3)
#pragma unroll
      for (int c = 0; c < CBLK; c++)
#pragma unroll
        for (int v = 0; v < 16; v++)
          if ((v & (1 << bit)) == 0) {
            const float a = acc[c][v], b = acc[c][v | (1 << bit)];
            acc[c][v] = a + b;
            acc[c][v | (1 << bit)] = a - b;
          }
    }
#pragma unroll
    for (int c = 0; c < CBLK; c++)  // channel bit 2: the partner lane
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const float pv = xor32(acc[c][v]);
        acc[c][v] = h ? (pv - acc[c][v]) : (acc[c][v] + pv);
      }
#pragma unroll
    for (int cb = 1; cb < CBLK; cb <<= 1)  // channel bits 5, 6: the 32-channel block
#pragma unroll
      for (int c = 0; c < CBLK; c++)
        if ((c & cb) == 0)
#pragma unroll
          for (int v = 0; v < 16; v++) {
            const float a = acc[c][v], b = acc[c | cb][v];
            acc[c][v] = a + b;
            acc[c | cb][v] = a - b;
          }
    const float cn = rsqrtf((float)D);
#pragma unroll
    for (int c = 0; c < CBLK; c++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[c][v] *= cn;
  }

  // ---------------- phase 2: current chunk (bf16, no correction) ----------------
  if (p.n_r > 0) {
    bf16x8 qb16[D / 16];
    {
      const uint16_t* qrow = p.q + ((size_t)bh * p.n_q + (q_ok ? qi : 0)) * D + HALF * h;
#pragma unroll
      for (int t = 0; t < D / 16; t++) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (q_ok) w = reinterpret_cast<const uint4*>(qrow)[t];
        qb16[t] = __builtin_bit_cast(bf16x8, w);
      }
    }
    const float sl = p.s * kLog2e;
    const uint16_t* kr_base = p.k_cur + (size_t)bh * p.n_r * D;
    const uint16_t* vr_base = p.v_cur + (size_t)bh * p.n_r * D;
    const int n_rt = (p.n_r + kBN - 1) / kBN;
    constexpr int SEGS = D / 8;              // 16-byte segments per row
    constexpr int ITEMS = (kBN / 2) * SEGS;  // (token pair, segment) items per tile
    static_assert(ITEMS <= kThreads, "one staging item per thread");
    // thread item: tokens (16g + j, 16g + j + 8) -- adjacent value positions -- and one segment
    const int seg = tid % SEGS, pr = tid / SEGS;
    const int tokA = 16 * (pr >> 3) + (pr & 7), tokB = tokA + 8;
    uint4 rka = make_uint4(0, 0, 0, 0), rkb = rka, rva = rka, rvb = rka;
    auto load_cur = [&](int T) {
      if (tid >= ITEMS) return;
      const int t0 = T * kBN;
      const bool okA = t0 + tokA < p.n_r, okB = t0 + tokB < p.n_r;
      rka = rkb = rva = rvb = make_uint4(0, 0, 0, 0);
      if (okA) {
        rka = reinterpret_cast<const uint4*>(kr_base + (size_t)(t0 + tokA) * D)[seg];
        if (!MASS_ONLY) rva = reinterpret_cast<const uint4*>(vr_base + (size_t)(t0 + tokA) * D)[seg];
      }
      if (okB) {
        rkb = reinterpret_cast<const uint4*>(kr_base + (size_t)(t0 + tokB) * D)[seg];
        if (!MASS_ONLY) rvb = reinterpret_cast<const uint4*>(vr_base + (size_t)(t0 + tokB) * D)[seg];
      }
    };
    auto store_cur = [&](int T, TileBuf<D, BITS>& tb) {
      if (tid < kBN) {
        const int nvalid = min(kBN, p.n_r - T * kBN);
        tb.mask[32 * (tid >> 5) + key_mrow(tid & 31)] = tid < nvalid ? 0.f : -INFINITY;
      }
      if (tid >= ITEMS) return;
      *reinterpret_cast<uint4*>(&tb.kr[tokA][8 * seg]) = rka;
      *reinterpret_cast<uint4*>(&tb.kr[tokB][8 * seg]) = rkb;
      if (!MASS_ONLY) {
        const uint32_t wa[4] = {rva.x, rva.y, rva.z, rva.w}, wb[4] = {rvb.x, rvb.y, rvb.z, rvb.w};
        const int pos = 16 * (pr >> 3) + 2 * (pr & 7);  // positions of tokA, tokB: pos, pos + 1
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float a0 = __uint_as_float(wa[e] << 16), a1 = __uint_as_float(wa[e] & 0xFFFF0000u);
          const float b0 = __uint_as_float(wb[e] << 16), b1 = __uint_as_float(wb[e] & 0xFFFF0000u);
          *reinterpret_cast<uint32_t*>(&tb.v[8 * seg + 2 * e][pos]) = pack_f16x2(a0, b0);
          *reinterpret_cast<uint32_t*>(&tb.v[8 * seg + 2 * e + 1][pos]) = pack_f16x2(a1, b1);
        }
      }
    };
    auto compute_cur = [&](int T, const TileBuf<D, BITS>& tb) {
      const int nvalid = min(kBN, p.n_r - T * kBN);
      f32x16 sc[2];
#pragma unroll
      for (int mb = 0; mb < 2; mb++) {
        const int key = 32 * mb + mrow_key(col);
#pragma unroll
        for (int t = 0; t < D / 16; t++) {
          const bf16x8 aop = *reinterpret_cast<const bf16x8*>(&tb.kr[key][HALF * h + 8 * t]);
          if (t == 0) {
            const f32x16 z = {};
            sc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qb16[t], z, 0, 0, 0);
          } else {
            sc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qb16[t], sc[mb], 0, 0, 0);
          }
        }
      }
      float slv[2][16];
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int v = 0; v < 16; v++) slv[mb][v] = sl;
      float pv[2][16];
      softmax_tile(sc, slv, nvalid < kBN, tb.mask, pv);
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int v = 0; v < 16; v++) l_r += pv[mb][v];
      if (!MASS_ONLY) {
        uint32_t pb[4][4];
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
          for (int v4 = 0; v4 < 4; v4++) {
            const int v = 4 * v4;
            const int ks = 2 * mb + (v4 >> 1), slot = 2 * (v4 & 1);
            pb[ks][slot] = pack_f16x2(pv[mb][v], pv[mb][v + 1]);
            pb[ks][slot + 1] = pack_f16x2(pv[mb][v + 2], pv[mb][v + 3]);
          }
        pv_tile(tb, pb);
      }
    };
    load_cur(0);
    store_cur(0, sm.buf[0]);
    __syncthreads();
    for (int T = 0; T < n_rt; T++) {
      const bool has_next = T + 1 < n_rt;
      if (has_next) load_cur(T + 1);
      compute_cur(T, sm.buf[T & 1]);
      if (has_next) store_cur(T + 1, sm.buf[(T + 1) & 1]);
      __syncthreads();
    }
  }

  // ---------------- epilogue ----------------
  l_s += xor32(l_s);
  l_r += xor32(l_r);
  const float tot = l_s + l_r;
  if (!q_ok) return;
  const float inv = 1.f / tot;
  if (!MASS_ONLY) {
    float* orow = p.o + ((size_t)bh * p.n_q + qi) * D;
#pragma unroll
    for (int c = 0; c < CBLK; c++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const int ch = 32 * c + 8 * v4 + 4 * h;
        *reinterpret_cast<float4*>(orow + ch) = make_float4(acc[c][4 * v4] * inv, acc[c][4 * v4 + 1] * inv,
                                                            acc[c][4 * v4 + 2] * inv, acc[c][4 * v4 + 3] * inv);
      }
  }
  if (h == 0 && p.mass_s) {
    p.mass_s[(size_t)bh * p.n_q + qi] = l_s * inv;
    p.mass_r[(size_t)bh * p.n_q + qi] = l_r * inv;
  }
}

int validate_attn(const jb_attn_args* a, bool mass_only) {
  if (!a) return KVQ_ERR_NULL;
  const kvq_format& kf = a->k_fmt;
  const kvq_format& vf = a->v_fmt;
  if (kf.bits != 2 && kf.bits != 4) return KVQ_ERR_UNSUPPORTED;
  if (vf.bits != kf.bits) return KVQ_ERR_UNSUPPORTED;
  if (kf.role != KVQ_ROLE_KEY || vf.role != KVQ_ROLE_VALUE) return KVQ_ERR_UNSUPPORTED;
  if (vf.granularity != KVQ_PER_TOKEN) return KVQ_ERR_UNSUPPORTED;
  if (kf.granularity != KVQ_PER_TOKEN) return KVQ_ERR_UNSUPPORTED;  // per-channel keys: see jb_attn_fwd
  if ((kf.hadamard | vf.hadamard) & ~1) return KVQ_ERR_UNSUPPORTED;
  if (a->correction != JB_CORR_NONE && a->correction != JB_CORR_TAYLOR) return KVQ_ERR_UNSUPPORTED;
  if (a->d != 64 && a->d != 128) return KVQ_ERR_SHAPE;
  if (a->B < 1 || a->H < 1 || a->n_q < 1 || a->n_r < 0 || a->chunk_len < 1 || a->n_chunks < 0)
    return KVQ_ERR_SHAPE;
  if ((long long)a->n_chunks * a->chunk_len + a->n_r < 1) return KVQ_ERR_SHAPE;
  if (!(a->softmax_scale >= 0.f) || isinf(a->softmax_scale)) return KVQ_ERR_SHAPE;
  const long long nqblk = (a->n_q + kBM - 1) / kBM;
  if (nqblk * a->B * a->H > 0x7FFFFFFFLL) return KVQ_ERR_SHAPE;
  if (!a->q) return KVQ_ERR_NULL;
  if (a->n_r > 0 && (!a->k_cur || (!mass_only && !a->v_cur))) return KVQ_ERR_NULL;
  if (a->n_chunks > 0) {
    if (!a->k_codes || !a->k_scale || !a->k_zero) return KVQ_ERR_NULL;
    if (!mass_only && (!a->v_codes || !a->v_scale || !a->v_zero)) return KVQ_ERR_NULL;
    if (!aligned16(a->k_codes) || !aligned16(a->k_scale) || !aligned16(a->k_zero)) return KVQ_ERR_ALIGN;
    if (!mass_only && (!aligned16(a->v_codes) || !aligned16(a->v_scale) || !aligned16(a->v_zero)))
      return KVQ_ERR_ALIGN;
  }
  if (mass_only) {
    if (!a->mass_s || !a->mass_r) return KVQ_ERR_NULL;
  } else {
    if (!a->o) return KVQ_ERR_NULL;
    if (!a->mass_s != !a->mass_r) return KVQ_ERR_NULL;
    if (!aligned16(a->o)) return KVQ_ERR_ALIGN;
  }
  if (!aligned16(a->q)) return KVQ_ERR_ALIGN;
  if (a->n_r > 0 && (!aligned16(a->k_cur) || (!mass_only && !aligned16(a->v_cur)))) return KVQ_ERR_ALIGN;
  return KVQ_OK;
}

template <int D, int BITS, bool MASS_ONLY>
int launch_attn(const jb_attn_args* a, hipStream_t st) {
  Params p;
  p.B = a->B;
  p.H = a->H;
  p.n_q = a->n_q;
  p.n_r = a->n_r;
  p.chunk_len = a->chunk_len;
  p.n_chunks = a->n_chunks;
  p.cp = chunk_pad(a->chunk_len);
  p.n_qblk = (a->n_q + kBM - 1) / kBM;
  p.q = a->q;
  p.k_cur = a->k_cur;
  p.v_cur = a->v_cur;
  p.k_codes = a->k_codes;
  p.k_scale = a->k_scale;
  p.k_zero = a->k_zero;
  p.v_codes = a->v_codes;
  p.v_scale = a->v_scale;
  p.v_zero = a->v_zero;
  p.s = a->softmax_scale > 0.f ? a->softmax_scale : 1.f / sqrtf((float)D);
  p.correction = a->correction;
  p.k_had = a->k_fmt.hadamard;
  p.v_had = a->v_fmt.hadamard;
  p.o = MASS_ONLY ? nullptr : a->o;
  p.mass_s = a->mass_s;
  p.mass_r = a->mass_r;
  const unsigned grid = (unsigned)(p.n_qblk * a->B * a->H);
  jb_attn_kernel<D, BITS, MASS_ONLY><<<grid, kThreads, 0, st>>>(p);
  return launch_status();
}

template <bool MASS_ONLY>
int dispatch(const jb_attn_args* a, void* stream) {
  const int st = validate_attn(a, MASS_ONLY);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a->d == 128)
    return a->k_fmt.bits == 2 ? launch_attn<128, 2, MASS_ONLY>(a, s) : launch_attn<128, 4, MASS_ONLY>(a, s);
  return a->k_fmt.bits == 2 ? launch_attn<64, 2, MASS_ONLY>(a, s) : launch_attn<64, 4, MASS_ONLY>(a, s);
}

}  // namespace
}  // namespace kvq

extern "C" int jb_attn_fwd(const jb_attn_args* a, void* stream) { return kvq::dispatch<false>(a, stream); }

extern "C" int jb_attn_mass(const jb_attn_args* a, void* stream) { return kvq::dispatch<true>(a, stream); }

extern "C" size_t jb_attn_workspace_bytes(const jb_attn_args* a) {
  (void)a;
  return 0;
}
