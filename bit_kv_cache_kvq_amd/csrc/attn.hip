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
// queries and streams 64-key tiles):
//  * Scores are computed transposed, S^T = K Q^T, so keys are the MFMA M dimension and
//    each lane owns one query: per-query softmax state lives in one lane (and its
//    partner lane l^32, which holds the other half of each key block).
//  * Cached QK^T runs on int8 MFMA (v_mfma_i32_32x32x32_i8): the rotated query
//    q' = H q is a 16-bit fixed-point integer split into signed hi/lo bytes, the key
//    operand is the raw 2- or 4-bit code, unpacked in registers with shifts and masks.
//    Integer accumulation is exact; the zero point enters as -z_j * sum(q_fixed).
//    Logit (log2 units): x = Delta_j (A S - G Delta_j), A = s sigma log2(e),
//    G = s^2 |q'|^2 / 24 log2(e).
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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kQFix = 32639.f;  // |q_fixed| <= 32639 keeps hi = (q+128)>>8 in int8

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

__device__ inline float half_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ inline uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ inline float xor32(float v) { return __shfl_xor(v, 32); }

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
struct Smem {
  static constexpr int KW = D * BITS / 32;           // key words per token
  static constexpr int VROW = kBN + 8;               // fp16 per V row (padded)
  uint32_t k_words[kBN][KW];
  _Float16 v[D][VROW];                               // (code - z) or current-chunk values
  uint16_t kr[kBN][D + 8];                           // current-chunk keys (bf16)
  float dk[kBN];                                     // per key, M-row order
  int zk[kBN];
  float dv[kBN];
  float mask[kBN];
  uint32_t zv_pair[kBN / 2];                         // (-1024 - z) fp16 pairs, natural order
};

template <int D, int BITS, bool MASS_ONLY>
__global__ __launch_bounds__(kThreads) void jb_attn_kernel(const Params p) {
  constexpr int HALF = D / 2;
  constexpr int KSTEPS = D / 32;        // int8 K-steps of 32 channels
  constexpr int CBLK = D / 32;          // 32-channel output blocks
  constexpr int CPW = 32 / BITS;
  constexpr int KW = D * BITS / 32;     // key words per token
  constexpr int VWPC = kBN / CPW;       // value words per channel per 64-token block
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
  float A, G;
  int nqsum;
  {
    float qv[HALF];
    const uint16_t* qrow = p.q + ((size_t)bh * p.n_q + (q_ok ? qi : 0)) * D + HALF * h;
#pragma unroll
    for (int u = 0; u < HALF / 8; u++) {
      uint4 w = q_ok ? reinterpret_cast<const uint4*>(qrow)[u] : make_uint4(0, 0, 0, 0);
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
    nqsum = -qs;
    A = p.s * sigma * kLog2e;
    G = p.correction ? p.s * p.s * ss * (1.f / 24.f) * kLog2e : 0.f;
  }

  float m_run = -INFINITY, l_s = 0.f, l_r = 0.f;
  f32x16 acc[CBLK];
#pragma unroll
  for (int c = 0; c < CBLK; c++)
#pragma unroll
    for (int v = 0; v < 16; v++) acc[c][v] = 0.f;

  // Online-softmax step over one 64-key tile whose scores (log2 units) are in x[2][16].
  // Returns p in x; updates m_run and rescales acc and the sums when the max grows.
  auto softmax_tile = [&](float (&x)[2][16]) {
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
      for (int v = 0; v < 16; v++) mx = fmaxf(mx, x[mb][v]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run) != 0) {
      const float sc = __builtin_amdgcn_exp2f(m_run - m_new);
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
      for (int v = 0; v < 16; v++) x[mb][v] = __builtin_amdgcn_exp2f(x[mb][v] - m_run);
  };

  // PV for one tile: B operand = P (fp16 pairs from the score registers), A = V rows in LDS.
  auto pv_tile = [&](const uint32_t (&pb)[4][4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(pb[ks][0], pb[ks][1], pb[ks][2], pb[ks][3]));
#pragma unroll
      for (int c = 0; c < CBLK; c++) {
        const f16x8 aop = *reinterpret_cast<const f16x8*>(&sm.v[32 * c + col][16 * ks + 8 * h]);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop, acc[c], 0, 0, 0);
      }
    }
  };

  // ---------------- phase 1: cached window ----------------
  const int n_tiles = p.n_chunks * (p.cp / kBN);
  const size_t n_tot = (size_t)p.n_chunks * p.cp;
  const uint32_t* kc_base = p.k_codes + (size_t)bh * n_tot * KW;
  const uint32_t* vc_base = p.v_codes + (size_t)bh * (n_tot / kBN) * (D * VWPC);
  const uint16_t* ks_base = p.k_scale + (size_t)bh * n_tot;
  const uint16_t* kz_base = p.k_zero + (size_t)bh * n_tot;
  const uint16_t* vs_base = p.v_scale + (size_t)bh * n_tot;
  const uint16_t* vz_base = p.v_zero + (size_t)bh * n_tot;

  for (int T = 0; T < n_tiles; T++) {
    const int off = (T * kBN) % p.cp;
    const int nvalid = min(kBN, p.chunk_len - off);
    const size_t tok0 = (size_t)T * kBN;
    __syncthreads();  // the previous tile's LDS reads are complete
    // stage packed key words (natural token order)
    for (int e = tid; e < kBN * KW; e += kThreads) (&sm.k_words[0][0])[e] = kc_base[tok0 * KW + e];
    if (tid < kBN) {
      const int j = tid;
      const int r = 32 * (j >> 5) + key_mrow(j & 31);
      const float dk = half_bits_to_f32(ks_base[tok0 + j]);
      const float zk = half_bits_to_f32(kz_base[tok0 + j]);
      const float dv = MASS_ONLY ? 0.f : half_bits_to_f32(vs_base[tok0 + j]);
      sm.dk[r] = dk;
      sm.zk[r] = (int)zk;
      sm.dv[r] = dv;
      sm.mask[r] = j < nvalid ? 0.f : -INFINITY;
    }
    if (!MASS_ONLY && tid < kBN / 2) {
      // pair (j, j+8) of each 16-token group: halves hold -(1024 + z)
      const int g = tid >> 3, j = tid & 7;
      const float z0 = half_bits_to_f32(vz_base[tok0 + 16 * g + j]);
      const float z1 = half_bits_to_f32(vz_base[tok0 + 16 * g + j + 8]);
      sm.zv_pair[tid] = pack_f16x2(-1024.f - z0, -1024.f - z1);
    }
    __syncthreads();
    if (!MASS_ONLY) {
      // unpack value codes into (code - z) fp16, channel-major rows, pair-interleaved
      const uint32_t* vblk = vc_base + (size_t)T * (D * VWPC);
      for (int e = tid; e < D * (kBN / 16); e += kThreads) {
        const int ch = e / (kBN / 16), g = e % (kBN / 16);  // 16-token group g of channel ch
        uint32_t out[8];
        if (BITS == 2) {
          const uint32_t w = vblk[ch * VWPC + g];
#pragma unroll
          for (int j = 0; j < 8; j++) out[j] = ((w >> (2 * j)) & 0x00030003u) | 0x64006400u;
        } else {
          const uint32_t w0 = vblk[ch * VWPC + 2 * g], w1 = vblk[ch * VWPC + 2 * g + 1];
          // t0 = [w0.b0 w0.b1 w1.b0 w1.b1], t1 = [w0.b2 w0.b3 w1.b2 w1.b3]
          const uint32_t t0 = (w0 & 0xFFFFu) | (w1 << 16);
          const uint32_t t1 = (w0 >> 16) | (w1 & 0xFFFF0000u);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            out[j] = ((t0 >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
            out[4 + j] = ((t1 >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
          }
        }
        uint32_t res[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          typedef _Float16 h2 __attribute__((ext_vector_type(2)));
          const h2 a = __builtin_bit_cast(h2, out[j]);
          const h2 z = __builtin_bit_cast(h2, sm.zv_pair[8 * g + j]);
          res[j] = __builtin_bit_cast(uint32_t, a + z);
        }
        uint4* dst = reinterpret_cast<uint4*>(&sm.v[ch][16 * g]);
        dst[0] = make_uint4(res[0], res[1], res[2], res[3]);
        dst[1] = make_uint4(res[4], res[5], res[6], res[7]);
      }
      __syncthreads();
    }

    // ---- QK^T on int8 MFMA ----
    i32x16 shi[2], slo[2];
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      const int key = 32 * mb + mrow_key(col);
      uint32_t kw[KW / 2];
#pragma unroll
      for (int e = 0; e < KW / 2; e++) kw[e] = sm.k_words[key][(KW / 2) * h + e];
#pragma unroll
      for (int v = 0; v < 16; v++) {
        shi[mb][v] = 0;
        slo[mb][v] = 0;
      }
#pragma unroll
      for (int kk = 0; kk < KSTEPS; kk++) {
        i32x4 aop;
        if (BITS == 2) {
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
        shi[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, qhi[kk], shi[mb], 0, 0, 0);
        slo[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, qlo[kk], slo[mb], 0, 0, 0);
      }
    }
    // ---- logits with the correction ----
    float x[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const int r0 = 32 * mb + 8 * v4 + 4 * h;
        const float4 dk4 = *reinterpret_cast<const float4*>(&sm.dk[r0]);
        const int4 zk4 = *reinterpret_cast<const int4*>(&sm.zk[r0]);
        const float dk[4] = {dk4.x, dk4.y, dk4.z, dk4.w};
        const int zk[4] = {zk4.x, zk4.y, zk4.z, zk4.w};
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int v = 4 * v4 + b;
          const int si = (shi[mb][v] << 8) + slo[mb][v] + zk[b] * nqsum;
          const float f = (float)si;
          x[mb][v] = dk[b] * fmaf(A, f, -G * dk[b]);
        }
      }
    if (nvalid < kBN) {
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int v = 0; v < 16; v++) x[mb][v] += sm.mask[32 * mb + (v & 3) + 8 * (v >> 2) + 4 * h];
    }
    softmax_tile(x);
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
      for (int v = 0; v < 16; v++) l_s += x[mb][v];
    if (!MASS_ONLY) {
      uint32_t pb[4][4];
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int v4 = 0; v4 < 4; v4++) {
          const float4 dv4 = *reinterpret_cast<const float4*>(&sm.dv[32 * mb + 8 * v4 + 4 * h]);
          const int v = 4 * v4;
          const int ks = 2 * mb + (v4 >> 1), slot = 2 * (v4 & 1);
          pb[ks][slot] = pack_f16x2(x[mb][v] * dv4.x, x[mb][v + 1] * dv4.y);
          pb[ks][slot + 1] = pack_f16x2(x[mb][v + 2] * dv4.z, x[mb][v + 3] * dv4.w);
        }
      pv_tile(pb);
    }
  }

  // ---------------- phase switch: un-rotate the cached PV sum ----------------
  if (!MASS_ONLY && p.v_had && n_tiles > 0) {
    // acc[c][v] holds channel 32c + (v&3) + 8(v>>2) + 4h of this lane's query.
#pragma unroll
    for (int bit = 0; bit < 2; bit++)  // channel bits 0,1: v bits 0,1
#pragma unroll
      for (int c = 0; c < CBLK; c++)
#pragma unroll
        for (int v = 0; v < 16; v++)
          if ((v & (1 << bit)) == 0) {
            const float a = acc[c][v], b = acc[c][v | (1 << bit)];
            acc[c][v] = a + b;
            acc[c][v | (1 << bit)] = a - b;
          }
#pragma unroll
    for (int c = 0; c < CBLK; c++)  // channel bit 2: the partner lane
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const float pv = xor32(acc[c][v]);
        acc[c][v] = h ? (pv - acc[c][v]) : (acc[c][v] + pv);
      }
#pragma unroll
    for (int bit = 2; bit < 4; bit++)  // channel bits 3,4: v bits 2,3
#pragma unroll
      for (int c = 0; c < CBLK; c++)
#pragma unroll
        for (int v = 0; v < 16; v++)
          if ((v & (1 << bit)) == 0) {
            const float a = acc[c][v], b = acc[c][v | (1 << bit)];
            acc[c][v] = a + b;
            acc[c][v | (1 << bit)] = a - b;
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
        const uint4 w = q_ok ? reinterpret_cast<const uint4*>(qrow)[t] : make_uint4(0, 0, 0, 0);
        qb16[t] = __builtin_bit_cast(bf16x8, w);
      }
    }
    const float sl = p.s * kLog2e;
    const uint16_t* kr_base = p.k_cur + (size_t)bh * p.n_r * D;
    const uint16_t* vr_base = p.v_cur + (size_t)bh * p.n_r * D;
    const int n_rt = (p.n_r + kBN - 1) / kBN;
    for (int T = 0; T < n_rt; T++) {
      const int t0 = T * kBN;
      const int nvalid = min(kBN, p.n_r - t0);
      __syncthreads();
      for (int e = tid; e < kBN * (D / 8); e += kThreads) {
        const int tok = e / (D / 8), seg = e % (D / 8);
        const bool ok = tok < nvalid;
        const uint4 kw = ok ? reinterpret_cast<const uint4*>(kr_base + (size_t)(t0 + tok) * D)[seg]
                            : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(&sm.kr[tok][8 * seg]) = kw;
        if (!MASS_ONLY) {
          const uint4 vw = ok ? reinterpret_cast<const uint4*>(vr_base + (size_t)(t0 + tok) * D)[seg]
                              : make_uint4(0, 0, 0, 0);
          const uint32_t ww[4] = {vw.x, vw.y, vw.z, vw.w};
          // position of token tok in its 16-token group: key j + 8e sits at 2j + e
          const int g = tok >> 4, in = tok & 15;
          const int pos = 16 * g + 2 * (in & 7) + (in >> 3);
#pragma unroll
          for (int e2 = 0; e2 < 4; e2++) {
            sm.v[8 * seg + 2 * e2][pos] = (_Float16)__uint_as_float(ww[e2] << 16);
            sm.v[8 * seg + 2 * e2 + 1][pos] = (_Float16)__uint_as_float(ww[e2] & 0xFFFF0000u);
          }
        }
      }
      if (tid < kBN) {
        const int j = tid;
        sm.mask[32 * (j >> 5) + key_mrow(j & 31)] = j < nvalid ? 0.f : -INFINITY;
      }
      __syncthreads();
      f32x16 sc[2];
#pragma unroll
      for (int mb = 0; mb < 2; mb++) {
        const int key = 32 * mb + mrow_key(col);
#pragma unroll
        for (int v = 0; v < 16; v++) sc[mb][v] = 0.f;
#pragma unroll
        for (int t = 0; t < D / 16; t++) {
          const bf16x8 aop = *reinterpret_cast<const bf16x8*>(&sm.kr[key][HALF * h + 8 * t]);
          sc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qb16[t], sc[mb], 0, 0, 0);
        }
      }
      float x[2][16];
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int v = 0; v < 16; v++) x[mb][v] = sc[mb][v] * sl;
      if (nvalid < kBN) {
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
          for (int v = 0; v < 16; v++) x[mb][v] += sm.mask[32 * mb + (v & 3) + 8 * (v >> 2) + 4 * h];
      }
      softmax_tile(x);
#pragma unroll
      for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int v = 0; v < 16; v++) l_r += x[mb][v];
      if (!MASS_ONLY) {
        uint32_t pb[4][4];
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
          for (int v4 = 0; v4 < 4; v4++) {
            const int v = 4 * v4;
            const int ks = 2 * mb + (v4 >> 1), slot = 2 * (v4 & 1);
            pb[ks][slot] = pack_f16x2(x[mb][v], x[mb][v + 1]);
            pb[ks][slot + 1] = pack_f16x2(x[mb][v + 2], x[mb][v + 3]);
          }
        pv_tile(pb);
      }
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
