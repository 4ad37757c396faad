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
// Kernel design. A workgroup is 8 waves (two per SIMD) and 256 queries of one head; a
// wave owns 32 queries and walks 32-key blocks (two per 64-key tile), first over the
// cached window, then over the current chunk.
//  * Scores are computed transposed, S^T = K Q^T: keys are the MFMA M dimension and
//    each lane owns one query (lane l^32 holds the other half of every 32-key block),
//    so the softmax state of a query lives in one lane pair.
//  * Cached QK^T with per-token keys runs on the scaled MFMA
//    (v_mfma_scale_f32_32x32x64_f8f6f4): the key operand is the raw code, as fp4 e2m1
//    (2-bit codes, value code / 2 with a key scale of 2) or fp6 e2m3 (4-bit codes),
//    unpacked once per workgroup into LDS; the rotated query q' = H q enters as three
//    fp6 e2m3 passes (a rounding, then roundings of what is left), each with a
//    power-of-two scale per lane and 32 channels, summed in one fp32 accumulator.
//    Group-wise keys of 64 channels run the same contraction with one accumulator per
//    group; group-wise keys of 32 channels (and group-wise keys with the exact
//    correction) are dequantized to fp16 in the staging and meet the query as fp16
//    hi + lo parts on fp16 MFMA.
//  * The zero point, the correction, the reference max and the padding mask enter
//    through one fp16 MFMA per block whose key operand holds Delta_j z_j, Delta_j^2
//    (hi/lo fp16 pairs), 1 and the mask, and whose query operand holds -A times the
//    query's channel sum (as the QK^T operands hold it), -G, -m and a large negative
//    constant. In log2 units the logit is x = (Delta_j A) S + c with A = s log2 e and
//    G = s^2 |q'|^2 / 24 log2 e, so a score costs one fma and one exp2.
//  * Keys quantized per channel over token groups (Delta_gc, z_gc) run QK^T on int8
//    MFMA (v_mfma_i32_32x32x32_i8): at each group's first tile the wave rescales its
//    rotated query by the group's steps, q~ = q' Delta_g, quantizes it to 16-bit
//    fixed point (one scale a_ch per wave) split into signed bytes hi, lo (the int32
//    sum 256 S_hi + S_lo is exact), and folds the group's zero-point and correction
//    terms into a per-query constant carried by the bias MFMA; the logit is
//    x = a_ch S + c. The rotated queries stay in LDS (16-bit fixed point) for the
//    whole cached window.
//  * The reference max m starts at the first block's maximum plus a headroom of 2^2 (a
//    larger headroom pushes keys a few binades below the max into fp16 subnormals) and
//    stays fixed while every p = exp2(x) fits fp16 (checked by the fp16 row sum of each
//    block); only a block that passes 2^15 raises m and rescales the accumulator, in a
//    rare wave-uniform branch.
//  * PV on fp16 MFMA: P = fp16(p) straight from the score registers (a fixed key
//    permutation inside each 32-key block makes the score layout the B operand); the
//    value tile in LDS holds fp16((code - z) Delta^V), exact in the subtraction. The
//    sums l_S, l_R add the same fp16 P.
//  * The cached PV sum is in the rotated basis and is un-rotated once (an FWHT across
//    the accumulator registers) before the current chunk, which runs on bf16 QK^T
//    (exact products) and fp16 PV.
//  * Keys and per-key parameters are staged two tiles ahead, values one tile ahead
//    (a three-slot LDS ring), by all eight waves, with one barrier per tile; the two
//    waves of a SIMD overlap each other's matrix-core and VALU work in part.
//  * A grid too small for the device splits each query block's tiles into shares whose
//    partial records a second kernel merges; several calls may share one launch; with
//    at most 32 queries a one-wave kernel streams shares of the cached window instead
//    (few queries: the cache stream, not the matrix cores, bounds the call).
//  * Options: the exact correction sum_c log(sinh(x_c) / x_c), x_c = s q'_c Delta_c / 2
//    (an ablation of the second-order form), randomized rotations H diag(s), and a
//    window stride larger than the chunks attended (a ring of chunk slots).
#include <math.h>

#include <algorithm>
#include <mutex>

#include <type_traits>

#include "common.h"

namespace kvq {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x6 __attribute__((ext_vector_type(6)));
typedef unsigned u32x6 __attribute__((ext_vector_type(6)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStreams = 1;             // 32-query streams per wave
constexpr int kNS = kWaves * kStreams;  // streams per workgroup
constexpr int kBM = 32 * kNS;           // queries per workgroup
constexpr int kBN = 64;                 // keys per tile
static_assert(kBM == kQueryBlock && kBN == kKeyTile, "the host plan and the kernels use one geometry");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPmax = 32768.f;     // largest fp16 row sum of a block accepted in a pass
constexpr float kHeadroom = 2.f;     // first reference max: the first block's max + 2 (log2 units)
constexpr float kMaskLogit = 65504.f;  // subtracted from padded keys' logits (log2 units)
constexpr float kD2Scale = 64.f;     // Delta^2 is carried as Delta^2 / 64 (fp16 range)

constexpr float kQFix = 32639.f;  // |q_f| <= 32639 keeps hi = (q_f + 128) >> 8 in int8
constexpr float kRoundMagic = 12582912.f;  // 1.5 2^23: adding it rounds |x| < 2^22 to an integer

struct Params {
  int B, H, n_q, n_r, chunk_len, n_chunks, cp;
  int n_wchunks;  // chunks per head in the window arrays (their per-head stride), >= n_chunks
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
  uint32_t k_sg[4], v_sg[4];  // randomized rotations H diag(s): bit c set -> channel c negated
  int k_group;  // tokens per key channel group (per-channel keys), else 0
  int n_split;  // workgroups per query block, each over a contiguous share of the tiles
  float* part;  // n_split > 1: partial records [n_split][B*H][n_q][D + 4], else null
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

// fp16 hi/lo split of x: hi = fp16(x), lo = fp16(x - hi).
__device__ inline void split16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

__device__ inline float xor32(float v) { return __shfl_xor(v, 32); }

// XOR mask that negates channels j and j+1 (j even) of a bf16 pair word, for the sign
// bits w of channels j0 .. j0+31 (j - j0 = bit index): the randomized rotation's diag(s).
__device__ inline uint32_t pair_sign_xor(uint32_t w, int bit) {
  const uint32_t b = w >> bit;
  return ((b & 1u) << 15) | (((b >> 1) & 1u) << 31);
}

// log(sinh(x) / x), the logarithm of E[e^(2 x u)] for u uniform on [-1/2, 1/2]: its
// power series through x^10 (coefficients 2^2n B_2n / (2n (2n)!), omitted terms below
// 1.7e-7 for |x| < 1), else |x| - log(2|x|) + log(1 - e^(-2|x|)).
__device__ inline float log_sinhc(float x) {
  const float a = fabsf(x), u = a * a;
  if (a < 1.f)
    return u * (1.f / 6 - u * (1.f / 180 - u * (1.f / 2835 - u * (1.f / 37800 - u * (1.f / 467775)))));
  return a - __logf(2.f * a) + __logf(1.f - __expf(-2.f * a));
}

// Raw buffer descriptor over [base, base + bytes): loads take a per-lane 32-bit offset
// and a wave-uniform offset (scalar register), so no 64-bit per-lane addresses are kept.
// Loads past the end return 0.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// C += A B on the scaled MFMA: A (keys) fp4 e2m1 (FA = 4) or fp6 e2m3 (FA = 2) with E8M0
// scale 2^1, B fp6 e2m3 with the E8M0 scale in byte SEL of sb (per lane, for its 32
// elements).
template <int FA, int SEL>
__device__ inline f32x16 mfma_kq(i32x8 a, i32x8 b, f32x16 c, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, 2, 0, 128, SEL, (int)sb);
}

// Element e of a 32-element operand slice (one lane's K half of a 64-channel K-step) is
// channel kslot<BITS>(e) of the 32: 2-bit keys, the fp4 nibbles come from the packed codes
// as (w & 0x33333333, (w >> 2) & 0x33333333) per 16 channels; 4-bit keys are converted
// to fp6 in channel order.
__device__ __host__ constexpr int kperm6(int e) { return 16 * (e >> 4) + 2 * (e & 7) + ((e >> 3) & 1); }
template <int BITS>
__device__ __host__ constexpr int kslot(int e) { return BITS == 2 ? kperm6(e) : e; }

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

template <int D>
struct SmemSlots {
  static constexpr int VROW = kBN + 8;  // fp16 per value row (padded against bank conflicts)
  static constexpr int KROW = D + 16;   // bytes per unpacked key row
  typedef uint8_t KCodes[kBN][KROW];    // cached key codes (kperm order per 16 channels)
  union KSlot {
    KCodes c;
    uint16_t kr[kBN][D + 8];  // current-chunk keys (bf16), natural order
  };
  struct PSlot {
    float dka[kNS][kBN];  // Delta_j A of each stream (cached; 0 for padding), M-row order
    uint4 kb[kBN][2];     // bias operand rows (16 fp16), M-row order
    float spare[2 * kBN];  // unused; without it c40 measured 2% slower (LDS placement)
  };
  struct ZSlot {
    uint32_t zv[kBN / 2];   // (-1024 - z^V) fp16 pairs, token pair (j, j+8) order
    uint32_t dvp[kBN / 2];  // (Delta^V_j, Delta^V_j+8) fp16 pairs
  };
  // Group-wise keys and values (NG channel groups per token): one zero-point / step pair
  // table per value channel group.
  template <int NG>
  struct ZSlotG {
    uint32_t zv[NG][kBN / 2];
    uint32_t dvp[NG][kBN / 2];
  };
};

// The LDS of a workgroup: a three-slot ring of key, value and parameter tiles (TG > 0:
// keys and values quantized in groups of TG channels per token).
template <int D, bool PERCH = false, int TG = 0>
struct Smem : SmemSlots<D> {
  using T = SmemSlots<D>;
  using PS = typename T::PSlot;
  using ZS = std::conditional_t<(TG > 0), typename T::template ZSlotG<(TG > 0 ? D / TG : 1)>, typename T::ZSlot>;
  alignas(16) typename T::KSlot k[3];     // cached codes, or fp16 keys (group-wise, current)
  alignas(16) _Float16 v[3][D][T::VROW];  // value rows: fp16((code - z) Delta^V) or current values
  alignas(16) PS prm[3];
  alignas(16) ZS z[3];
  alignas(16) float a_stream[kNS];
};

// Per-channel keys also keep each stream's rotated queries in LDS during the cached tiles,
// as 16-bit fixed point (32 queries x D per wave; the 16-byte chunks of a row are swizzled
// by the query index against bank conflicts), behind three packed code slots; the current
// chunk's key slots overlay both.
template <int D>
struct Smem<D, true, 0> : SmemSlots<D> {
  using T = SmemSlots<D>;
  union {
    typename T::KSlot k[3];
    struct {
      typename T::KCodes c[3];
      int16_t qf[kNS * 32 * D];
    } pc;
  };
  alignas(16) _Float16 v[3][D][T::VROW];
  alignas(16) typename T::PSlot prm[3];
  alignas(16) typename T::ZSlot z[3];
  alignas(16) float a_stream[kNS];
  __device__ typename T::KCodes& kc(int s) { return pc.c[s]; }
};

#define KVQ_INLINE __attribute__((always_inline))

// The rotated query of one lane (qv[i]: channel HALF h + i of its query) as three fp6
// e2m3 roundings per 64-channel K-step, for the scaled-MFMA QK^T: K-step k6 holds
// channels 32 k6 + kslot<BITS>(e), e < 32; pass 0 rounds them with a power-of-two scale
// 2^ex > max|.| / 7.5, passes 1 and 2 round what is left the same way. Writes the
// operands q6[k6][pass] and their E8M0 scale bytes (passes 0 and 1 of K-step k6 in bytes
// 2 k6 and 2 k6 + 1 of sc[0], pass 2 in byte k6 of sc[1]); returns the lane's sum of the
// rounded channels per K-step (the _slices form) or in all (encode_query_fp6).
// The rounding is the hardware conversion (32 floats / scale to packed e2m3, to nearest
// even, saturating at 7.5; packed element 2j from the first operand's j-th value, 2j + 1
// from the second's) and its inverse gives the rounded values. Every pass reads its
// sources again after the conversion (the residual), which keeps them out of the
// conversion's result registers: it writes part of its result before it has read all
// of its sources.
template <int HALF, int BITS>
__device__ KVQ_INLINE void encode_query_fp6_slices(const float (&qv)[HALF], i32x8 (&q6)[HALF / 32][3], uint32_t (&sc)[2],
                                                   float (&ksum)[HALF / 32]) {
  sc[0] = 0u;
  sc[1] = 0u;
#pragma unroll
  for (int k6 = 0; k6 < HALF / 32; k6++) {
    float qsum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i++) qsum += qv[32 * k6 + i];
    f32x16 s0, s1;  // element 2j: channel 32 k6 + kslot(2j); 2j + 1: kslot(2j + 1)
#pragma unroll
    for (int j = 0; j < 16; j++) {
      s0[j] = qv[32 * k6 + kslot<BITS>(2 * j)];
      s1[j] = qv[32 * k6 + kslot<BITS>(2 * j + 1)];
    }
#pragma unroll
    for (int pass = 0; pass < 3; pass++) {
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < 16; j++) mx = fmaxf(mx, fmaxf(fabsf(s0[j]), fabsf(s1[j])));
      // 2^ex > mx / 7.5 (the fp32 exponent of mx / 7.5, plus one)
      const int ex = min(max((int)((__float_as_uint(mx * (1.f / 7.5f)) >> 23) & 255u) - 126, -126), 126);
      const float scl = __uint_as_float((uint32_t)(127 + ex) << 23);
      const i32x6 c = __builtin_bit_cast(i32x6, __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(s0, s1, scl));
      const f32x32 v = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(__builtin_bit_cast(u32x6, c), scl);
#pragma unroll
      for (int j = 0; j < 16; j++) {
        s0[j] -= v[2 * j];
        s1[j] -= v[2 * j + 1];
      }
      q6[k6][pass] = i32x8{c[0], c[1], c[2], c[3], c[4], c[5], 0, 0};
      if (pass < 2)
        sc[0] |= (uint32_t)(ex + 127) << (8 * (2 * k6 + pass));
      else
        sc[1] |= (uint32_t)(ex + 127) << (8 * k6);
    }
    // the sum of the rounded channels: the sum of q' minus what the passes left
#pragma unroll
    for (int j = 0; j < 16; j++) qsum -= s0[j] + s1[j];
    ksum[k6] = qsum;
  }
}

// encode_query_fp6_slices, returning the lane's sum of the rounded channels.
template <int HALF, int BITS>
__device__ KVQ_INLINE float encode_query_fp6(const float (&qv)[HALF], i32x8 (&q6)[HALF / 32][3], uint32_t (&sc)[2]) {
  float ks[HALF / 32];
  encode_query_fp6_slices<HALF, BITS>(qv, q6, sc, ks);
  float t = 0.f;
#pragma unroll
  for (int k6 = 0; k6 < HALF / 32; k6++) t += ks[k6];
  return t;
}

// S = sum_c q~_c code_c of one 32x32 block in fp32: six scaled MFMAs (three query passes
// x two 64-channel K-steps; D = 64: three), the key operands ka (code c as the value
// c / 2: fp4 e2m1 for 2-bit codes, FA = 4, fp6 e2m3 for 4-bit codes, FA = 2; key scale
// 2^1 = E8M0 128) against encode_query_fp6's operands.
template <int FA, int KS6>  // KS6 deduced from the operand arrays
__device__ KVQ_INLINE f32x16 qk_fp6(const i32x8 (&ka)[KS6], const i32x8 (&q6)[KS6][3], const uint32_t (&sc)[2]) {
  f32x16 acc = {};
  acc = mfma_kq<FA, 0>(ka[0], q6[0][0], acc, sc[0]);
  if constexpr (KS6 > 1) acc = mfma_kq<FA, 2>(ka[1], q6[1][0], acc, sc[0]);
  acc = mfma_kq<FA, 1>(ka[0], q6[0][1], acc, sc[0]);
  if constexpr (KS6 > 1) acc = mfma_kq<FA, 3>(ka[1], q6[1][1], acc, sc[0]);
  acc = mfma_kq<FA, 0>(ka[0], q6[0][2], acc, sc[1]);
  if constexpr (KS6 > 1) acc = mfma_kq<FA, 1>(ka[1], q6[1][2], acc, sc[1]);
  return acc;
}

// 32 INT4 codes (four packed words, channel k at bits 4k of word k / 8) as 32 fp6 e2m3
// values c / 2, exact, in channel order: six words. The conversion is written out with
// its result marked early-clobber: it writes part of its result before it has read all
// of its sources, and these sources die at it.
__device__ inline i32x6 fp6_key_slice(uint4 w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  f32x16 s0, s1;  // element 2j: channel 2j, 2j + 1: channel 2j + 1
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const uint32_t lo = ws[m] & 0x0F0F0F0Fu, hi = (ws[m] >> 4) & 0x0F0F0F0Fu;  // channels 8m + 2b, + 1
#pragma unroll
    for (int b = 0; b < 4; b++) {
      s0[4 * m + b] = (float)((lo >> (8 * b)) & 0xFFu);
      s1[4 * m + b] = (float)((hi >> (8 * b)) & 0xFFu);
    }
  }
  i32x6 r;
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(s0), "v"(s1), "v"(2.0f));
  return r;
}

// fp4 key operand of 32 channels from two packed INT2 words (16 channels each, channel
// k at bits 2k): nibble n of the four dwords is channel 2n, 2n + 1 of the first word, then
// of the second (the kperm6 order).
__device__ inline i32x8 fp4_key_operand(uint32_t w0, uint32_t w1) {
  return i32x8{(int)(w0 & 0x33333333u), (int)((w0 >> 2) & 0x33333333u), (int)(w1 & 0x33333333u),
               (int)((w1 >> 2) & 0x33333333u), 0, 0, 0, 0};
}

enum : int { kNone = 0, kCached = 1, kCurrent = 2 };
template <int K>
using Kind = std::integral_constant<int, K>;

// One workgroup's work: workgroup wg of the n_wg a call launches (n_qblk * B * H *
// n_split; the linear ids are dealt to the XCDs round-robin, wg % 8 being the XCD). The
// LDS is declared here rather than passed in: the kernels address it as before.
template <int D, int BITS, bool MASS_ONLY, bool PERCH, bool EXACT, int TG = 0>
__device__ KVQ_INLINE void attn_body(const Params p, const int wg, const int n_wg) {
  __shared__ Smem<D, PERCH, TG> sm;
  using SM = Smem<D, PERCH, TG>;
  // Group-wise keys and values (TG channels per group): NG (step, zero point) pairs per
  // token. Cached keys are dequantized to fp16 Delta_jg (code - z_jg) in the staging (each
  // 16-channel unit lies in one group) and QK^T runs on fp16 MFMA against the rotated query
  // split into fp16 hi + lo parts (two MFMAs per K-step, one fp32 accumulator); the bias
  // MFMA carries the per-group correction (3 fp16 slots per group), -m and the mask.
  constexpr int NG = TG > 0 ? D / TG : 1;
  static_assert(TG == 0 || (!PERCH && TG % 32 == 0 && TG < D && NG <= kNS), "group-wise options");
  constexpr int HALF = D / 2;
  constexpr int KSTEPS = D / 32;  // int8 K-steps of 32 channels
  // Per-token keys: QK^T on the scaled MFMA (32x32x64, twice the K of the int8 MFMA per
  // instruction at its rate): the codes as the values code / 2 (2-bit: fp4 e2m1, 4-bit:
  // fp6 e2m3; key scale 2), the rotated query as three fp6 e2m3 passes (a rounding, the
  // rounding of its residual, the rounding of what is left), each with a power-of-two
  // scale per lane and 32 channels, summed in one fp32 accumulator.
  constexpr bool kF6 = !PERCH && TG == 0;
  constexpr int kFA = BITS == 2 ? 4 : 2;  // key operand format: fp4 e2m1, fp6 e2m3
  // Group-wise keys in two 64-channel groups (Taylor or no correction): the same QK^T
  // with one accumulator per group, a 64-channel K-step being one group (the lane halves
  // swap query channels so that K-step g holds group g), the codes as fp4 / fp6 rows, and
  // the logit sum_g (Delta_jg A) S_g + c with the groups' zero points in the bias.
  constexpr bool kF6G = TG == 64 && NG == 2 && !EXACT && !PERCH;
  // 2-bit per-token keys (Taylor or no correction) issue each phase's first tile loads
  // before the query build and before the switch to the current chunk (the other forms
  // keep them in the pipeline start: measured slower, or their registers there spill)
  constexpr bool kPre = kF6 && BITS == 2 && !EXACT;
  constexpr int KS6 = D / 64;  // fp6 K-steps of 64 channels (a lane holds 32 of each)
  constexpr int CBLK = D / 32;    // 32-channel output blocks
  constexpr int CPW = 32 / BITS;
  constexpr int KW = D * BITS / 32;  // key words per token
  constexpr int VWPC = kBN / CPW;    // value words per channel per 64-token block
  constexpr int VWT = D * VWPC;      // value words per tile
  constexpr int KU = BITS / 2;       // key words per 16-channel unit
  constexpr int KUNITS = kBN * D / 16;
  constexpr int WPG = BITS / 2;             // value words per 16-token group
  constexpr int VGROUPS = D * (kBN / 16);   // 16-token value groups per tile
  constexpr int SEGS = D / 8;               // 16-byte segments of a bf16 row
  constexpr int RITEMS = kBN * SEGS;        // current-key (token, segment) items per tile
  constexpr int VITEMS = (kBN / 2) * SEGS;  // current-value (token pair, segment) items per tile
  // items per thread (work counts below kThreads leave whole waves idle)
  constexpr int KUPT = (KUNITS + kThreads - 1) / kThreads;
  // 4-bit keys on the fp6 path are staged 32 channels (two units) per thread by the first
  // KPAIRS threads (the first wave of each SIMD finishes its block work first)
  constexpr int KPAIRS = KUNITS / 2;
  // Cached values are staged by the first wave of each SIMD only (waves 0..3): the second
  // wave of a SIMD issues after the first and is the one that ends each step last.
  constexpr int kVST = kThreads / 2;
  constexpr int VGPT = (VGROUPS + kVST - 1) / kVST;
  constexpr int RIPT = (RITEMS + kThreads - 1) / kThreads;
  constexpr int VRPT = (VITEMS + kThreads - 1) / kThreads;
  static_assert(kStreams == 1, "one 32-query stream per wave");
  static_assert(KUNITS % 64 == 0 && VGROUPS % 64 == 0 && RITEMS % 64 == 0 && VITEMS % 64 == 0, "wave-uniform split");
  static_assert(KUPT <= RIPT && VGPT <= 2 * VRPT && RIPT <= 4 && VRPT <= 2, "staging registers");
  static_assert(KPAIRS % 64 == 0 && KPAIRS <= kThreads / 2, "4-bit key pairs: whole waves");
  static_assert(kVST % 64 == 0 && kVST % 4 == 0, "value staging by whole waves, one token group per lane");

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  int qbs, bh;
  xcd_map(wg, n_wg, p.n_qblk * p.n_split, qbs, bh);
  const int qb = qbs / p.n_split, sp = qbs % p.n_split;  // query block, share of the tiles
  const int qi = qb * kBM + wave * 32 + col;  // this lane's query
  const bool q_ok = qi < p.n_q;
  // A wave whose 32 queries all lie past n_q (in the ragged last query block) stages tiles
  // and takes the barriers with the others but computes nothing.
  const bool computes = __builtin_amdgcn_readfirstlane(__ballot(q_ok) != 0ull ? 1 : 0) != 0;
  const float scale_l2 = p.s * kLog2e;  // softmax scale in log2 units

  // ---------------- query operands ----------------
  i32x4 qhi[KSTEPS], qlo[KSTEPS];  // int8 hi/lo of q_f (per-channel keys), or the bf16 query
  // group-wise keys: the rotated query as fp16 hi + lo, in the staged key rows' channel order
  f16x8 q16h[TG > 0 && !kF6G ? D / 16 : 1], q16l[TG > 0 && !kF6G ? D / 16 : 1];
  f16x8 qbias;                     // query operand of the bias MFMA
  i32x8 q6[kF6 || kF6G ? KS6 : 1][3];  // fp6 query operands: K-step, pass
  uint32_t q6sc[2] = {0u, 0u};     // their E8M0 scale bytes
  float m_run = -INFINITY;         // reference max (log2 units); -inf until the first block
  float a_st = 0.f;                // A of this wave's stream
  // Rotated query q' = H q / sqrt(d) (or q) of this lane's half: channels HALF h + i.
  auto rotated_query = [&](float* qv) KVQ_INLINE {
    const uint16_t* qrow = p.q + ((size_t)bh * p.n_q + (q_ok ? qi : 0)) * D + HALF * h;
    uint32_t sgw[HALF / 32];  // key-rotation signs of this lane's channels HALF h ..
#pragma unroll
    for (int k = 0; k < HALF / 32; k++) {
      sgw[k] = h ? p.k_sg[HALF / 32 + k] : p.k_sg[k];
      asm volatile("" : "+v"(sgw[k]));  // keeps the per-pair masks here, not hoisted out of the tile loop
    }
#pragma unroll
    for (int u = 0; u < HALF / 8; u++) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (q_ok) w = reinterpret_cast<const uint4*>(qrow)[u];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int j = 8 * u + 2 * e;
        const uint32_t we = ww[e] ^ pair_sign_xor(sgw[j >> 5], j & 31);
        qv[j] = __uint_as_float(we << 16);
        qv[j + 1] = __uint_as_float(we & 0xFFFF0000u);
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
  };
  // -m, plus the key group's constant c_grp (per-channel keys), into query slots 8, 9.
  float c_grp = 0.f;
  float ex2 = 0.f, ex3 = 0.f, ex4 = 0.f;  // exact correction, per-token keys (log2 units)
  float exg[3][NG];                        // the same per channel group (group-wise keys)
  auto write_mslot = [&]() KVQ_INLINE {
    _Float16 mh = (_Float16)0.f, ml = (_Float16)0.f;
    split16(c_grp - (m_run == -INFINITY ? 0.f : m_run), mh, ml);
    qbias[0] = h ? mh : qbias[0];
    qbias[1] = h ? ml : qbias[1];
  };
  auto build_query = [&]() KVQ_INLINE {
    float qv[HALF];
    rotated_query(qv);
    float qgrp[2] = {0.f, 0.f};  // kF6G: the rounded query's sum over each group
    if constexpr (kF6G) {
      // K-step g holds group g: lane half h takes channels 64 g + 32 h + e, swapping half
      // of its channels with the partner lane
      float qx[HALF];
#pragma unroll
      for (int i = 0; i < 32; i++) {
        const float r = xor32(h ? qv[i] : qv[32 + i]);
        qx[i] = h ? r : qv[i];
        qx[32 + i] = h ? qv[32 + i] : r;
      }
      float ks[2];
      encode_query_fp6_slices<HALF, BITS>(qx, q6, q6sc, ks);
      qgrp[0] = ks[0] + xor32(ks[0]);
      qgrp[1] = ks[1] + xor32(ks[1]);
    } else if constexpr (TG > 0) {
      // position 16u + 2k + b of a staged key row holds channel 16u + k + 8b (the pair
      // order of the code unpack); lane half h, K-step t reads positions HALF h + 8t ..
#pragma unroll
      for (int t = 0; t < D / 16; t++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int pp = 8 * t + e, c = 16 * (pp >> 4) + ((pp & 15) >> 1) + 8 * (pp & 1);
          _Float16 hi_, lo_;
          split16(qv[c], hi_, lo_);
          q16h[t][e] = hi_;
          q16l[t][e] = lo_;
        }
    }
    float ss = 0.f, mxa = 0.f;
#pragma unroll
    for (int i = 0; i < HALF; i++) {
      ss += qv[i] * qv[i];
      mxa = fmaxf(mxa, fabsf(qv[i]));
    }
    ss += xor32(ss);
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) mxa = fmaxf(mxa, __shfl_xor(mxa, sh));  // stream-wide max
    const float inv = mxa > 0.f ? kQFix / mxa : 0.f;
    const float A = kF6 || kF6G ? scale_l2 : mxa > 0.f ? scale_l2 * (mxa / kQFix) : 0.f;
    int qs = 0;
    float qs6 = 0.f;  // fp6 path: the sum of the rounded query's channels
    if constexpr (!kF6) {
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
    }
    qs += __shfl_xor(qs, 32);
    const float G = p.correction ? p.s * p.s * ss * (1.f / 24.f) * kLog2e : 0.f;
    if constexpr (EXACT && TG > 0) {
      // group-wise keys: the same series per channel group g, with the group's step
      // Delta_jg and moments M_n^g = sum over g's channels of (s q'_c / 2)^2n (this lane
      // holds channels HALF h + i, the partner lane the other half)
#pragma unroll
      for (int g = 0; g < NG; g++) {
        float m2 = 0.f, m3 = 0.f, m4 = 0.f;
#pragma unroll
        for (int i = 0; i < HALF; i++) {
          if ((HALF * h + i) / TG != g) continue;
          const float y = 0.5f * p.s * qv[i], u = y * y, u2 = u * u;
          m2 += u2;
          m3 = fmaf(u2, u, m3);
          m4 = fmaf(u2, u2, m4);
        }
        exg[0][g] = (m2 + xor32(m2)) * (1.f / 180.f) * kLog2e;
        exg[1][g] = (m3 + xor32(m3)) * (1.f / 2835.f) * kLog2e;
        exg[2][g] = (m4 + xor32(m4)) * (1.f / 37800.f) * kLog2e;
      }
    } else if constexpr (EXACT && !PERCH) {
      // b(Delta) = sum_c log_sinhc(s q'_c Delta / 2) = sum_n c_n M_n Delta^2n with
      // M_n = sum_c (s q'_c / 2)^2n: the n = 1 term is G's, n = 2..4 enter the logits
      float m2 = 0.f, m3 = 0.f, m4 = 0.f;
#pragma unroll
      for (int i = 0; i < HALF; i++) {
        const float y = 0.5f * p.s * qv[i], u = y * y, u2 = u * u;
        m2 += u2;
        m3 = fmaf(u2, u, m3);
        m4 = fmaf(u2, u2, m4);
      }
      m2 += xor32(m2);
      m3 += xor32(m3);
      m4 += xor32(m4);
      ex2 = m2 * (1.f / 180.f) * kLog2e;
      ex3 = m3 * (1.f / 2835.f) * kLog2e;
      ex4 = m4 * (1.f / 37800.f) * kLog2e;
    }
    // query-side factors of the bias MFMA (key side in the tile parameters):
    //   (Delta_j z_j) * w + (Delta_j^2 / 64) * g - m - 65504 * mask_j
    if constexpr (kF6) {
      const float lsum = encode_query_fp6<HALF, BITS>(qv, q6, q6sc);
      qs6 = lsum + xor32(lsum);
    }
    const float w = -A * (kF6 ? qs6 : (float)qs);
    const float g = -G * kD2Scale;
    _Float16 wh, wl, gh, gl;
    split16(w, wh, wl);
    split16(g, gh, gl);
    if (h == 0) {
      qbias[0] = wh;
      qbias[1] = wl;
      qbias[2] = wh;
      qbias[3] = gh;
      qbias[4] = gl;
      qbias[5] = gh;
      qbias[6] = (_Float16)0.f;
      qbias[7] = (_Float16)0.f;
    } else {
      qbias[2] = (_Float16)(-kMaskLogit);
#pragma unroll
      for (int e = 3; e < 8; e++) qbias[e] = (_Float16)0.f;
    }
    if constexpr (EXACT && !PERCH && TG == 0) {
      // the exact correction's terms past the second order, e2 D^4 - e3 D^6 + e4 D^8, ride
      // on the free bias slots against the key powers u^2, u^3, u^4 of u = D^2 / 64:
      // D^4 as (hi, lo, hi) in slots 6, 7, 11, D^6 likewise in 12, 13, 14, D^8 in 15
      _Float16 a4h, a4l, a6h, a6l;
      split16(fminf(ex2 * 4096.f, 65504.f), a4h, a4l);
      split16(fmaxf(-ex3 * 262144.f, -65504.f), a6h, a6l);
      const _Float16 a8 = (_Float16)fminf(ex4 * 16777216.f, 65504.f);
      if (h == 0) {
        qbias[6] = a4h;
        qbias[7] = a4l;
      } else {
        qbias[3] = a4h;
        qbias[4] = a6h;
        qbias[5] = a6l;
        qbias[6] = a6h;
        qbias[7] = a8;
      }
    }
    if constexpr (TG > 0) {
      // term t: the correction of group t, -s^2 |q'_t|^2 / 24 (times 64, log2 units); its
      // three slots are k = 3t .. 3t+2 at bias slot k + 3 (k >= 8): 8, 9, 10 carry -m and
      // the mask
      _Float16 qsl[16];
#pragma unroll
      for (int k = 0; k < 16; k++) qsl[k] = (_Float16)0.f;
#pragma unroll
      for (int t = 0; t < NG; t++) {
        float sg = 0.f;
#pragma unroll
        for (int i = 0; i < HALF; i++)
          if ((HALF * h + i) / TG == t) sg += qv[i] * qv[i];
        sg += xor32(sg);
        const float y = p.correction ? -(p.s * p.s * sg * (1.f / 24.f) * kLog2e) * kD2Scale : 0.f;
        _Float16 yh, yl;
        split16(y, yh, yl);
        const int k0 = 3 * t;
        qsl[k0 + (k0 >= 8 ? 3 : 0)] = yh;
        qsl[k0 + 1 + (k0 + 1 >= 8 ? 3 : 0)] = yl;
        qsl[k0 + 2 + (k0 + 2 >= 8 ? 3 : 0)] = yh;
      }
      if constexpr (kF6G) {
        // the zero points of groups 0 and 1, -A Q_g against Delta_jg z_jg: slots 6, 7, 11
        // and 12, 13, 14 as (hi, lo, hi)
        _Float16 zh, zl;
        split16(-A * qgrp[0], zh, zl);
        qsl[6] = zh;
        qsl[7] = zl;
        qsl[11] = zh;
        split16(-A * qgrp[1], zh, zl);
        qsl[12] = zh;
        qsl[13] = zl;
        qsl[14] = zh;
      }
#pragma unroll
      for (int e = 0; e < 8; e++) qbias[e] = h ? qsl[8 + e] : qsl[e];
      if (h) qbias[2] = (_Float16)(-kMaskLogit);
    }
    write_mslot();  // -m (hi, lo); 0 while m is unset
    if (lane == 0) sm.a_stream[wave] = A;
    __syncthreads();
    a_st = sm.a_stream[wave];
  };
  // From the first current-chunk tile on, the cached keys' query operands are no longer needed;
  // their registers take the bf16 query (half h: channels HALF h .. HALF h + HALF - 1).
  auto load_query_bf16 = [&]() KVQ_INLINE {
    const uint4* qrow16 = reinterpret_cast<const uint4*>(p.q + ((size_t)bh * p.n_q + (q_ok ? qi : 0)) * D + HALF * h);
#pragma unroll
    for (int t = 0; t < D / 16; t++) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (q_ok) w = qrow16[t];
      if (t < KSTEPS)
        qhi[t] = __builtin_bit_cast(i32x4, w);
      else
        qlo[t - KSTEPS] = __builtin_bit_cast(i32x4, w);
    }
  };
  // Sets the reference max to mx; with per-token keys m is rounded to what the bias
  // operand carries (-m as an fp16 hi + lo pair), so that every block sees the same m.
  auto set_m = [&](float mx) KVQ_INLINE {
    if constexpr (PERCH) {
      m_run = mx;
    } else {
      _Float16 mh, ml;
      split16(-mx, mh, ml);
      m_run = -((float)mh + (float)ml);
    }
    write_mslot();
  };
  if constexpr (!kPre) build_query();

  // ---------------- tile geometry ----------------
  const int tiles_per_chunk = p.cp / kBN;
  const int n_ct = p.n_chunks * tiles_per_chunk;  // cached tiles
  const int n_rt = (p.n_r + kBN - 1) / kBN;       // current-chunk tiles
  const size_t n_tot = (size_t)p.n_chunks * p.cp;     // cached tokens attended (padded)
  const size_t n_str = (size_t)p.n_wchunks * p.cp;    // per-head stride of the window arrays
  const uint32_t* kc_base = p.k_codes + (size_t)bh * n_str * KW;
  const uint32_t* vc_base = p.v_codes + (size_t)bh * (n_str / kBN) * VWT;
  constexpr int PPT = TG > 0 ? NG : 1;  // (step, zero point) pairs per token
  const uint16_t* ks_base = p.k_scale + (size_t)bh * n_str * PPT;
  const uint16_t* kz_base = p.k_zero + (size_t)bh * n_str * PPT;
  const uint16_t* vs_base = p.v_scale + (size_t)bh * n_str * PPT;
  const uint16_t* vz_base = p.v_zero + (size_t)bh * n_str * PPT;
  const uint16_t* kr_base = p.k_cur + (size_t)bh * p.n_r * D;
  const uint16_t* vr_base = p.v_cur + (size_t)bh * p.n_r * D;
  // descriptors of this head's cached window (the byte sizes fit 31 bits: checked on the host)
  const __amdgpu_buffer_rsrc_t rs_kc = buffer_rsrc(kc_base, (uint32_t)(n_tot * KW * 4));
  const __amdgpu_buffer_rsrc_t rs_vc = buffer_rsrc(vc_base, (uint32_t)(n_tot * VWT / kBN * 4));
  const __amdgpu_buffer_rsrc_t rs_ks = buffer_rsrc(ks_base, (uint32_t)(n_tot * 2 * PPT));
  const __amdgpu_buffer_rsrc_t rs_kz = buffer_rsrc(kz_base, (uint32_t)(n_tot * 2 * PPT));
  const __amdgpu_buffer_rsrc_t rs_vs = buffer_rsrc(vs_base, (uint32_t)(n_tot * 2 * PPT));
  const __amdgpu_buffer_rsrc_t rs_vz = buffer_rsrc(vz_base, (uint32_t)(n_tot * 2 * PPT));
  auto n_valid = [&](int U) KVQ_INLINE {
    return U < n_ct ? min(kBN, p.chunk_len - (U % tiles_per_chunk) * kBN) : min(kBN, p.n_r - (U - n_ct) * kBN);
  };

  // Per-channel keys: a key of channel group g (of its chunk) dequantizes as
  // Delta_gc (code_c - z_gc), so its logit is s q~.code - s q~.z_g - b - m with
  // q~_c = q'_c Delta_gc and b = s^2 |q~|^2 / 24 (the per-channel Taylor correction).
  // At each group's first tile the wave rebuilds the int8 operands from q~ (own scale
  // a_ch) and folds the group constant c_grp = -a_ch sum(q~_f z_g) - G into the bias.
  const int k_tpg = PERCH ? p.k_group / kBN : 1;                       // tiles per key group
  const int k_gpc = PERCH ? (p.chunk_len + p.k_group - 1) / p.k_group : 1;  // groups per chunk
  float a_ch = 0.f;
  // The group's step and zero-point rows come from the tile's parameter slot (staged with
  // the tile's keys): D fp16 steps, then D fp16 zero points.
  // The rotated query rows stay in LDS for the cached tiles as q'_f = rint(q' / sq0) in
  // 16 bits (sq0 = max |q'| / 32767 per query); a refresh starts from q'_f, so the group
  // terms below carry sq0 where they need q~ itself.
  float sq0 = 0.f;
  auto qf_chunk = [&](int u) KVQ_INLINE -> uint4* {  // 16-byte chunk u of this lane's half row
    if constexpr (PERCH)
      return reinterpret_cast<uint4*>(&sm.pc.qf[(wave * 32 + col) * D]) + (((HALF / 8) * h + u) ^ (col & 7));
    else
      return nullptr;
  };
  auto fill_qf = [&]() KVQ_INLINE {
    float qv[HALF];
    rotated_query(qv);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < HALF; i++) mx = fmaxf(mx, fabsf(qv[i]));
    mx = fmaxf(mx, xor32(mx));
    sq0 = mx * (1.f / 32767.f);
    const float inv = mx > 0.f ? 32767.f / mx : 0.f;
#pragma unroll
    for (int u = 0; u < HALF / 8; u++) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int a = (int)rintf(qv[8 * u + 2 * e] * inv), b = (int)rintf(qv[8 * u + 2 * e + 1] * inv);
        w[e] = ((uint32_t)a & 0xFFFFu) | ((uint32_t)b << 16);
      }
      *qf_chunk(u) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  auto refresh_group = [&](int slot) KVQ_INLINE {
    const uint4* drow = reinterpret_cast<const uint4*>(&sm.prm[slot].dka[0][0]) + HALF * h / 8;
    const uint4* zrow = drow + D / 8;
    float qv[HALF];
    if constexpr (PERCH) {
#pragma unroll
      for (int u = 0; u < HALF / 8; u++) {
        const uint4 w = *qf_chunk(u);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          qv[8 * u + 2 * e] = (float)(int)(int16_t)(ww[e] & 0xFFFFu);
          qv[8 * u + 2 * e + 1] = (float)((int)ww[e] >> 16);
        }
      }
    } else {
      // never called for per-token keys; the reference keeps their kernels' code unchanged
      // (the per-token loop measured 1.5% slower when this lambda did not use it)
      rotated_query(qv);
    }
    float ss = 0.f, mxa = 0.f;
#pragma unroll
    for (int u = 0; u < HALF / 8; u++) {
      const uint4 w = drow[u];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; e++) {
        // the fp16 step enters a mixed-precision fma (no separate conversion)
        const f16x2 d2 = __builtin_bit_cast(f16x2, ww[e >> 1]);
        const float qt = fmaf(qv[8 * u + e], (float)d2[e & 1], 0.f);
        qv[8 * u + e] = qt;
        ss = fmaf(qt, qt, ss);
        mxa = fmaxf(mxa, fabsf(qt));
      }
    }
    ss += xor32(ss);
    float bx = 0.f;  // exact correction: sum_c log_sinhc(s q~_c / 2)
    if constexpr (EXACT) {
#pragma unroll
      for (int i = 0; i < HALF; i++) bx += log_sinhc((0.5f * p.s * sq0) * qv[i]);
      bx += xor32(bx);
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) mxa = fmaxf(mxa, __shfl_xor(mxa, sh));  // stream-wide max
    const float inv = mxa > 0.f ? kQFix / mxa : 0.f;
    a_ch = mxa > 0.f ? scale_l2 * (mxa * sq0 / kQFix) : 0.f;
    // zero-point sum sum_c q~_c z_gc from the unrounded q~ (one mixed fma per channel; the
    // rounding of q_f it leaves out shifts all of the group's logits alike, by ~1e-5 of
    // s max|q~|)
    float zs = 0.f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; kk++) {
      _Float16 zt[16];
#pragma unroll
      for (int u2 = 0; u2 < 2; u2++) {
        const uint4 w = zrow[2 * kk + u2];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 8; e++) zt[8 * u2 + e] = __builtin_bit_cast(f16x2, ww[e >> 1])[e & 1];
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        // four codes of this word: q_f = rint(q~ / sigma), split into hi = (q_f + 128) >> 8
        // and lo = q_f - 256 hi. fma(x, inv, 1.5 2^23) rounds x inv to an integer in the
        // low mantissa bits (|x inv| < 2^22), so the low 16 bits of the float are q_f as
        // int16; lo is q_f's low byte and hi is byte 1 of q_f + 128
        uint32_t fb[4];
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int c = kperm<BITS>(j, b);
          const float f = fmaf(qv[16 * kk + c], inv, kRoundMagic);
          fb[b] = __float_as_uint(f);
          zs = fmaf(qv[16 * kk + c], (float)zt[c], zs);
        }
        const uint32_t p0 = __builtin_amdgcn_perm(fb[1], fb[0], 0x05040100u);  // int16 pairs
        const uint32_t p1 = __builtin_amdgcn_perm(fb[3], fb[2], 0x05040100u);
        const u16x2 off = {(unsigned short)128, (unsigned short)128};
        const uint32_t h0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, p0) + off);
        const uint32_t h1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, p1) + off);
        qhi[kk][j] = (int)__builtin_amdgcn_perm(h1, h0, 0x07050301u);
        qlo[kk][j] = (int)__builtin_amdgcn_perm(p1, p0, 0x06040200u);
      }
    }
    zs += xor32(zs);
    const float G = EXACT ? bx * kLog2e : p.correction ? p.s * p.s * (sq0 * sq0) * ss * (1.f / 24.f) * kLog2e : 0.f;
    c_grp = -a_ch * inv * zs - G;
    write_mslot();
  };

  // ---------------- staging (all threads) ----------------
  // Step T stages the keys, per-key parameters and value zero-point / step pairs of
  // tile T+2, and the values of tile T+1. Global loads are issued at the start of the
  // step (per-channel keys: in the step before), unconditional, with indices clamped into
  // the arrays (positions past the end are replaced when stored); the LDS stores come
  // later in the step, before its barrier.
  uint4 kpre[RIPT];          // keys (code units, or current rows)
  uint4 vpre[2 * VRPT];      // values (code groups, or current row pairs)
  uint32_t pk_dk = 0, pk_zk = 0;                 // key step / zero point of key tid & 63
  uint4 gpre = make_uint4(0, 0, 0, 0);           // per-channel keys: 16 bytes of the group rows
  uint32_t pz0 = 0, pz1 = 0, pd0 = 0, pd1 = 0;   // value zero points / steps of a token pair
  // group-wise: the NG fp16 steps of key tid & 63 (groups 0, 1 in .x, groups 2, 3 in .y),
  // and the step and zero point of this thread's 16-channel key unit
  uint2 gk_d = make_uint2(0, 0);
  uint2 gk_z = make_uint2(0, 0);  // kF6G: the NG zero points of key tid & 63
  uint32_t uk_d = 0, uk_z = 0;
  uint2 gv_z0 = make_uint2(0, 0), gv_z1 = make_uint2(0, 0), gv_d0 = make_uint2(0, 0), gv_d1 = make_uint2(0, 0);
  auto load_pairs = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t tok, uint32_t tok0) KVQ_INLINE -> uint2 {
    if constexpr (NG == 4) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs, tok * 8u, tok0 * 8u, 0);
      return make_uint2(w[0], w[1]);
    } else {
      return make_uint2(__builtin_amdgcn_raw_buffer_load_b32(rs, tok * 4u, tok0 * 4u, 0), 0u);
    }
  };
  auto pair_bits = [&](const uint2& w, int g) KVQ_INLINE -> uint32_t {
    return ((g < 2 ? w.x : w.y) >> (16 * (g & 1))) & 0xFFFFu;
  };

  auto load_k = [&](int U, auto k_c) KVQ_INLINE {
    if constexpr (decltype(k_c)::value == kCached) {
      // buffer loads: per-lane offsets are loop-invariant, the tile offset is uniform
      const uint32_t tok0 = (uint32_t)U * kBN;
      if constexpr ((kF6 || kF6G) && BITS == 4) {
        const int kp = tid;  // unit pair: 32 channels of token kp / (D / 32)
        if (kp < KPAIRS) {
          const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs_kc, (uint32_t)kp * 16u, tok0 * KW * 4u, 0);
          kpre[0] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      } else
#pragma unroll
      for (int i = 0; i < KUPT; i++) {
        const uint32_t un = (uint32_t)min(tid + i * kThreads, KUNITS - 1);
        if constexpr (KU == 2) {
          const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs_kc, un * 8u, tok0 * KW * 4u, 0);
          kpre[i].x = w[0];
          kpre[i].y = w[1];
        } else {
          kpre[i].x = __builtin_amdgcn_raw_buffer_load_b32(rs_kc, un * 4u, tok0 * KW * 4u, 0);
        }
      }
      if constexpr (kF6G) {
        const uint32_t j = (uint32_t)(tid & (kBN - 1));
        gk_d = load_pairs(rs_ks, j, tok0);
        gk_z = load_pairs(rs_kz, j, tok0);
      } else if constexpr (TG > 0) {
        const uint32_t j = (uint32_t)(tid & (kBN - 1));
        gk_d = load_pairs(rs_ks, j, tok0);
        const uint32_t un = (uint32_t)min(tid, KUNITS - 1);
        const uint32_t pi = (un / (D / 16)) * NG + (un % (D / 16)) * 16 / TG;  // (token, group) pair
        uk_d = __builtin_amdgcn_raw_buffer_load_b16(rs_ks, pi * 2u, tok0 * 2u * NG, 0);
        uk_z = __builtin_amdgcn_raw_buffer_load_b16(rs_kz, pi * 2u, tok0 * 2u * NG, 0);
      } else if constexpr (!PERCH) {
        const uint32_t j = (uint32_t)(tid & (kBN - 1));
        pk_dk = __builtin_amdgcn_raw_buffer_load_b16(rs_ks, j * 2u, tok0 * 2u, 0);
        pk_zk = __builtin_amdgcn_raw_buffer_load_b16(rs_kz, j * 2u, tok0 * 2u, 0);
      } else if (tid < D / 4) {
        // per-channel keys: the step row (lanes 0 .. D/8-1) and zero-point row of the
        // tile's key group, 16 bytes per lane
        const int ci = U / tiles_per_chunk, tt = U % tiles_per_chunk;
        const size_t row = ((size_t)bh * p.n_wchunks * k_gpc + (size_t)ci * k_gpc + tt / k_tpg) * D;
        const uint16_t* src = tid < D / 8 ? p.k_scale : p.k_zero;
        gpre = reinterpret_cast<const uint4*>(src + row)[tid % (D / 8)];
      }
      if constexpr (!MASS_ONLY && TG > 0) {
        const uint32_t j = (uint32_t)(16 * ((tid >> 3) & 3) + (tid & 7));
        gv_z0 = load_pairs(rs_vz, j, tok0);
        gv_z1 = load_pairs(rs_vz, j + 8u, tok0);
        gv_d0 = load_pairs(rs_vs, j, tok0);
        gv_d1 = load_pairs(rs_vs, j + 8u, tok0);
      } else if constexpr (!MASS_ONLY) {
        const uint32_t j = (uint32_t)(16 * ((tid >> 3) & 3) + (tid & 7));
        pz0 = __builtin_amdgcn_raw_buffer_load_b16(rs_vz, j * 2u, tok0 * 2u, 0);
        pz1 = __builtin_amdgcn_raw_buffer_load_b16(rs_vz, j * 2u + 16u, tok0 * 2u, 0);
        pd0 = __builtin_amdgcn_raw_buffer_load_b16(rs_vs, j * 2u, tok0 * 2u, 0);
        pd1 = __builtin_amdgcn_raw_buffer_load_b16(rs_vs, j * 2u + 16u, tok0 * 2u, 0);
      }
    } else {
      const int t0 = (U - n_ct) * kBN;
#pragma unroll
      for (int i = 0; i < RIPT; i++) {
        const int it = min(tid + i * kThreads, RITEMS - 1);
        const int tok = min(t0 + it / SEGS, p.n_r - 1), seg = it % SEGS;
        kpre[i] = reinterpret_cast<const uint4*>(kr_base + (size_t)tok * D)[seg];
      }
    }
  };
  auto store_k = [&](int U, int slot, auto k_c) KVQ_INLINE {
    typename SM::KSlot& ks = sm.k[slot];
    auto& ps = sm.prm[slot];
    const int nv = n_valid(U);
    if constexpr (decltype(k_c)::value == kCached) {
      if constexpr ((kF6 || kF6G) && BITS == 4) {
        // fp6 rows: 32 channels (a unit pair) in 24 bytes
        const int kp = tid;
        if (kp < KPAIRS) {
          const int tok = kp / (D / 32), pi = kp % (D / 32);
          const i32x6 c = fp6_key_slice(kpre[0]);
          uint2* dst = reinterpret_cast<uint2*>(&ks.c[tok][24 * pi]);
          dst[0] = make_uint2((uint32_t)c[0], (uint32_t)c[1]);
          dst[1] = make_uint2((uint32_t)c[2], (uint32_t)c[3]);
          dst[2] = make_uint2((uint32_t)c[4], (uint32_t)c[5]);
        }
      } else
#pragma unroll
      for (int i = 0; i < KUPT; i++) {
        const int un = tid + i * kThreads;
        if (KUNITS % kThreads != 0 && un >= KUNITS) break;
        const int tok = un / (D / 16), ui = un % (D / 16);
        uint4 lo;
        if constexpr (BITS == 2) {
          const uint32_t w = kpre[i].x;
          lo = make_uint4(w & 0x03030303u, (w >> 2) & 0x03030303u, (w >> 4) & 0x03030303u, (w >> 6) & 0x03030303u);
        } else {
          const uint32_t w0 = kpre[i].x, w1 = kpre[i].y;
          lo = make_uint4(w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu);
        }
        if constexpr (TG > 0 && !kF6G) {
          // fp16 Delta (code - z) of channels 16 ui + k (low half) and 16 ui + k + 8 (high)
          // at positions 16 ui + 2k, + 1: (1024 + code) - (1024 + z) is exact in fp16
          uint32_t a[8];
          if constexpr (BITS == 2) {
            const uint32_t w = kpre[i].x;
#pragma unroll
            for (int j = 0; j < 8; j++) a[j] = ((w >> (2 * j)) & 0x00030003u) | 0x64006400u;
          } else {
            const uint32_t w0 = kpre[i].x, w1 = kpre[i].y;
            const uint32_t t0 = (w0 & 0xFFFFu) | (w1 << 16);
            const uint32_t t1 = (w0 >> 16) | (w1 & 0xFFFF0000u);
#pragma unroll
            for (int j = 0; j < 4; j++) {
              a[j] = ((t0 >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
              a[4 + j] = ((t1 >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
            }
          }
          const float zf = half_bits_to_f32(uk_z);
          const uint32_t zz = pack_f16x2(-1024.f - zf, -1024.f - zf);
          const uint32_t dd = (uk_d & 0xFFFFu) | (uk_d << 16);
          uint32_t res[8];
#pragma unroll
          for (int j = 0; j < 8; j++) {
            const f16x2 cz = __builtin_bit_cast(f16x2, a[j]) + __builtin_bit_cast(f16x2, zz);
            res[j] = __builtin_bit_cast(uint32_t, cz * __builtin_bit_cast(f16x2, dd));
          }
          uint4* dst = reinterpret_cast<uint4*>(&ks.kr[tok][16 * ui]);
          dst[0] = make_uint4(res[0], res[1], res[2], res[3]);
          dst[1] = make_uint4(res[4], res[5], res[6], res[7]);
        } else if constexpr (PERCH) {  // packed code slots
          *reinterpret_cast<uint4*>(&sm.kc(slot)[tok][16 * ui]) = lo;
        } else if constexpr (kF6 || kF6G) {  // 2-bit keys (4-bit ones are staged above)
          // fp4 nibbles of channels 16 ui + 2 n (first word) and 16 ui + 2 n + 1 (second)
          const uint32_t w = kpre[i].x;
          *reinterpret_cast<uint2*>(&ks.c[tok][8 * ui]) = make_uint2(w & 0x33333333u, (w >> 2) & 0x33333333u);
        } else {
          *reinterpret_cast<uint4*>(&ks.c[tok][16 * ui]) = lo;
        }
      }
      // Delta_j A of each wave's stream; 0 for padding keys (their logit is set by the mask)
      if constexpr (PERCH) {
        if (tid < D / 4) reinterpret_cast<uint4*>(&ps.dka[0][0])[tid] = gpre;
      }
      if constexpr (kF6G) {
        // Delta_jg A of each group (0 for padding keys), one row per group, M-row order
        if (wave < NG) {
          const int r = 32 * (lane >> 5) + key_mrow(lane & 31);
          ps.dka[wave][r] = lane < nv ? half_bits_to_f32(pair_bits(gk_d, wave)) * scale_l2 : 0.f;
        }
      } else if constexpr (TG > 0) {
        // per-group steps Delta_jg as fp16 bits (0 for padding keys), one row per group,
        // M-row order, in the per-key table's storage
        if (wave < NG) {
          const int r = 32 * (lane >> 5) + key_mrow(lane & 31);
          reinterpret_cast<uint16_t*>(&ps.dka[0][0])[wave * kBN + r] = lane < nv ? (uint16_t)pair_bits(gk_d, wave) : 0;
        }
      } else if constexpr (!PERCH) {
        const int key = tid & (kBN - 1);
        const int r = 32 * (key >> 5) + key_mrow(key & 31);
        const float dk = key < nv ? half_bits_to_f32(pk_dk) : 0.f;
        ps.dka[wave][r] = dk * a_st;
      }
      if constexpr (TG > 0) {
        if (wave == 0) {
          // bias key operand: term t (Delta^2 / 64 of group t) as (hi, hi, lo) at slots
          // k = 3t.., slot k + 3 from k = 8 on; slots 8, 9 = 1 (the -m pair), 10 = the mask
          const int r = 32 * (lane >> 5) + key_mrow(lane & 31);
          uint32_t ksl[8];
#pragma unroll
          for (int k = 0; k < 8; k++) ksl[k] = 0u;
          const uint32_t one = 0x3C00u;
          ksl[4] = one | (one << 16);
          if (lane < nv) {
#pragma unroll
            for (int t = 0; t < NG; t++) {
              const float dk = half_bits_to_f32(pair_bits(gk_d, t));
              const float x = dk * dk * (1.f / kD2Scale);
              _Float16 xh, xl;
              split16(x, xh, xl);
              const uint32_t hb = __builtin_bit_cast(uint16_t, xh), lb = __builtin_bit_cast(uint16_t, xl);
              const uint32_t v3[3] = {hb, hb, lb};
#pragma unroll
              for (int e = 0; e < 3; e++) {
                const int k = 3 * t + e, sl = k + (k >= 8 ? 3 : 0);
                ksl[sl >> 1] |= v3[e] << (16 * (sl & 1));
              }
              if constexpr (kF6G) {
                // the zero point Delta_jg z_jg of group t as (hi, hi, lo) at slots 6, 7, 11
                // (t = 0) or 12, 13, 14 (t = 1)
                _Float16 zh, zl;
                split16(dk * half_bits_to_f32(pair_bits(gk_z, t)), zh, zl);
                const uint32_t zhb = __builtin_bit_cast(uint16_t, zh), zlb = __builtin_bit_cast(uint16_t, zl);
                const int sz[3] = {t == 0 ? 6 : 12, t == 0 ? 7 : 13, t == 0 ? 11 : 14};
                const uint32_t z3[3] = {zhb, zhb, zlb};
#pragma unroll
                for (int e = 0; e < 3; e++) ksl[sz[e] >> 1] |= z3[e] << (16 * (sz[e] & 1));
              }
            }
          } else {
            ksl[5] = one;  // the mask slot: padding keys get -65504
          }
          ps.kb[r][0] = make_uint4(ksl[0], ksl[1], ksl[2], ksl[3]);
          ps.kb[r][1] = make_uint4(ksl[4], ksl[5], ksl[6], ksl[7]);
        }
      } else if (PERCH && wave == 0) {
        // per-channel keys: the group terms ride on the query side (slots 8, 9)
        const int r = 32 * (lane >> 5) + key_mrow(lane & 31);
        ps.kb[r][0] = make_uint4(0, 0, 0, 0);
      } else if (wave == 0) {
        // bias key operand, slots 0..7: dz_hi, dz_hi, dz_lo, d2_hi, d2_hi, d2_lo, 0, 0
        const int r = 32 * (lane >> 5) + key_mrow(lane & 31);
        uint4 row = make_uint4(0, 0, 0, 0);
        if (lane < nv) {
          const float dk = half_bits_to_f32(pk_dk), zk = half_bits_to_f32(pk_zk);
          _Float16 dzh, dzl, d2h, d2l;
          split16(dk * zk, dzh, dzl);
          split16(dk * dk * (1.f / kD2Scale), d2h, d2l);
          const uint32_t dzh_b = __builtin_bit_cast(uint16_t, dzh), dzl_b = __builtin_bit_cast(uint16_t, dzl);
          const uint32_t d2h_b = __builtin_bit_cast(uint16_t, d2h), d2l_b = __builtin_bit_cast(uint16_t, d2l);
          row.x = dzh_b | (dzh_b << 16);
          row.y = dzl_b | (d2h_b << 16);
          row.z = d2h_b | (d2l_b << 16);
          if constexpr (EXACT) {
            const float u = dk * dk * (1.f / kD2Scale);
            _Float16 u4h, u4l;
            split16(fminf(u * u, 65504.f), u4h, u4l);
            const uint32_t u4h_b = __builtin_bit_cast(uint16_t, u4h);
            row.w = u4h_b | (u4h_b << 16);
          }
        }
        ps.kb[r][0] = row;
      }
      if constexpr (EXACT && TG == 0 && !PERCH) {
        if (wave == 1) {
          // slots 8..15: 1, 1, the mask, then the D^4 lo part, D^6 (hi, hi, lo), D^8
          const int r = 32 * (lane >> 5) + key_mrow(lane & 31);
          const uint32_t one = 0x3C00u;
          uint4 row = make_uint4(one | (one << 16), one, 0u, 0u);
          if (lane < nv) {
            const float dk = half_bits_to_f32(pk_dk);
            const float u = dk * dk * (1.f / kD2Scale), u2 = u * u;
            _Float16 u4h, u4l, u6h, u6l;
            split16(fminf(u2, 65504.f), u4h, u4l);
            split16(fminf(u2 * u, 65504.f), u6h, u6l);
            const _Float16 u8 = (_Float16)fminf(u2 * u2, 65504.f);
            const uint32_t u4l_b = __builtin_bit_cast(uint16_t, u4l), u6h_b = __builtin_bit_cast(uint16_t, u6h);
            const uint32_t u6l_b = __builtin_bit_cast(uint16_t, u6l), u8_b = __builtin_bit_cast(uint16_t, u8);
            row.y = u4l_b << 16;
            row.z = u6h_b | (u6h_b << 16);
            row.w = u6l_b | (u8_b << 16);
          }
          ps.kb[r][1] = row;
        }
      }
      if constexpr (!MASS_ONLY && TG > 0) {
        if (wave == 2 && lane < kBN / 2) {
          auto& zs = sm.z[slot];
          const int g = lane >> 3, j = lane & 7;
          const bool ok0 = 16 * g + j < nv, ok1 = 16 * g + j + 8 < nv;
#pragma unroll
          for (int gg = 0; gg < NG; gg++) {
            zs.zv[gg][lane] = pack_f16x2(ok0 ? -1024.f - half_bits_to_f32(pair_bits(gv_z0, gg)) : -1024.f,
                                         ok1 ? -1024.f - half_bits_to_f32(pair_bits(gv_z1, gg)) : -1024.f);
            zs.dvp[gg][lane] = (ok0 ? pair_bits(gv_d0, gg) : 0u) | ((ok1 ? pair_bits(gv_d1, gg) : 0u) << 16);
          }
        }
      } else if constexpr (!MASS_ONLY) {
        if (wave == 2 && lane < kBN / 2) {
          auto& zs = sm.z[slot];
          const int g = lane >> 3, j = lane & 7;
          const bool ok0 = 16 * g + j < nv, ok1 = 16 * g + j + 8 < nv;
          zs.zv[lane] = pack_f16x2(ok0 ? -1024.f - half_bits_to_f32(pz0) : -1024.f,
                                   ok1 ? -1024.f - half_bits_to_f32(pz1) : -1024.f);
          zs.dvp[lane] = (ok0 ? (pd0 & 0xFFFFu) : 0u) | ((ok1 ? (pd1 & 0xFFFFu) : 0u) << 16);
        }
      }
    } else {
      const int t0 = (U - n_ct) * kBN;
#pragma unroll
      for (int i = 0; i < RIPT; i++) {
        const int it = tid + i * kThreads;
        if (RITEMS % kThreads != 0 && it >= RITEMS) break;
        const int tok = it / SEGS, seg = it % SEGS;
        *reinterpret_cast<uint4*>(&ks.kr[tok][8 * seg]) = t0 + tok < p.n_r ? kpre[i] : make_uint4(0, 0, 0, 0);
      }
      if (wave == 0) {
        const int r = 32 * (lane >> 5) + key_mrow(lane & 31);
        ps.kb[r][0] = make_uint4(0, 0, 0, 0);
      }
    }
    if (wave == 1 && !(TG > 0 && decltype(k_c)::value == kCached) &&
        !(EXACT && TG == 0 && !PERCH && decltype(k_c)::value == kCached)) {
      // bias key operand, slots 8..15: 1, 1, mask, 0...
      const int r = 32 * (lane >> 5) + key_mrow(lane & 31);
      const uint32_t one = 0x3C00u;
      ps.kb[r][1] = make_uint4(one | (one << 16), lane < nv ? 0u : one, 0u, 0u);
    }
  };
  auto load_v = [&](int U, auto k_c) KVQ_INLINE {
    if constexpr (MASS_ONLY) return;
    if constexpr (decltype(k_c)::value == kCached) {
      if (tid >= kVST) return;
#pragma unroll
      for (int i = 0; i < VGPT; i++) {
        const uint32_t vg = (uint32_t)min(tid + i * kVST, VGROUPS - 1);
        if constexpr (WPG == 2) {
          const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs_vc, vg * 8u, (uint32_t)U * VWT * 4u, 0);
          vpre[i].x = w[0];
          vpre[i].y = w[1];
        } else {
          vpre[i].x = __builtin_amdgcn_raw_buffer_load_b32(rs_vc, vg * 4u, (uint32_t)U * VWT * 4u, 0);
        }
      }
    } else {
      // item (token pair pr, segment seg): tokens 16(pr>>3) + (pr&7) and that + 8
      const int t0 = (U - n_ct) * kBN;
#pragma unroll
      for (int i = 0; i < VRPT; i++) {
        const int it = min(tid + i * kThreads, VITEMS - 1);
        const int seg = it % SEGS, pr = it / SEGS;
        const int tokA = 16 * (pr >> 3) + (pr & 7);
        vpre[2 * i] = reinterpret_cast<const uint4*>(vr_base + (size_t)min(t0 + tokA, p.n_r - 1) * D)[seg];
        vpre[2 * i + 1] = reinterpret_cast<const uint4*>(vr_base + (size_t)min(t0 + tokA + 8, p.n_r - 1) * D)[seg];
      }
    }
  };
  // the 2-bit field mask in a vector register lets the unpack use one and-or per pair
  uint32_t vmask2 = 0x00030003u;
  asm volatile("" : "+v"(vmask2));
  auto store_v = [&](int U, int slot, auto k_c) KVQ_INLINE {  // the pairs of tile U must be visible in sm.z[slot]
    if constexpr (MASS_ONLY) return;
    _Float16(*vrows)[SM::VROW] = sm.v[slot];
    if constexpr (decltype(k_c)::value == kCached) {
      if (tid >= kVST) return;
      const auto& zs = sm.z[slot];
      // every group of this lane has the same token group g = tid mod 4 (kVST % 4 == 0)
      const int g = tid & 3;
      auto zd_rows = [&](const uint32_t* zrow, const uint32_t* drow, uint32_t* zz, uint32_t* dd) KVQ_INLINE {
        const uint4 z0 = *reinterpret_cast<const uint4*>(&zrow[8 * g]);
        const uint4 z1 = *reinterpret_cast<const uint4*>(&zrow[8 * g + 4]);
        const uint4 d0 = *reinterpret_cast<const uint4*>(&drow[8 * g]);
        const uint4 d1 = *reinterpret_cast<const uint4*>(&drow[8 * g + 4]);
        zz[0] = z0.x, zz[1] = z0.y, zz[2] = z0.z, zz[3] = z0.w, zz[4] = z1.x, zz[5] = z1.y, zz[6] = z1.z, zz[7] = z1.w;
        dd[0] = d0.x, dd[1] = d0.y, dd[2] = d0.z, dd[3] = d0.w, dd[4] = d1.x, dd[5] = d1.y, dd[6] = d1.z, dd[7] = d1.w;
      };
      uint32_t zz[8], dd[8];
      if constexpr (TG == 0) zd_rows(zs.zv, zs.dvp, zz, dd);
#pragma unroll
      for (int i = 0; i < VGPT; i++) {
        const int vg = tid + i * kVST;
        if (VGROUPS % kVST != 0 && vg >= VGROUPS) break;
        const int ch = vg >> 2;  // 16-token group g of channel ch
        if constexpr (TG > 0) zd_rows(zs.zv[ch / TG], zs.dvp[ch / TG], zz, dd);
        uint32_t a[8];
        if constexpr (BITS == 2) {
          const uint32_t w = vpre[i].x;
#pragma unroll
          for (int j = 0; j < 8; j++) a[j] = ((w >> (2 * j)) & vmask2) | 0x64006400u;
        } else {
          // t0 = [w0.b0 w0.b1 w1.b0 w1.b1], t1 = [w0.b2 w0.b3 w1.b2 w1.b3]
          const uint32_t w0 = vpre[i].x, w1 = vpre[i].y;
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
        for (int j = 0; j < 8; j++) {
          const f16x2 cz = __builtin_bit_cast(f16x2, a[j]) + __builtin_bit_cast(f16x2, zz[j]);  // code - z, exact
          res[j] = __builtin_bit_cast(uint32_t, cz * __builtin_bit_cast(f16x2, dd[j]));
        }
        uint4* dst = reinterpret_cast<uint4*>(&vrows[ch][16 * g]);
        dst[0] = make_uint4(res[0], res[1], res[2], res[3]);
        dst[1] = make_uint4(res[4], res[5], res[6], res[7]);
      }
    } else {
      const int t0 = (U - n_ct) * kBN;
#pragma unroll
      for (int i = 0; i < VRPT; i++) {
        const int it = tid + i * kThreads;
        if (VITEMS % kThreads != 0 && it >= VITEMS) break;
        const int seg = it % SEGS, pr = it / SEGS;
        const int pos = 16 * (pr >> 3) + 2 * (pr & 7);  // positions of the pair's tokens: pos, pos+1
        const int tokA = 16 * (pr >> 3) + (pr & 7);
        const uint4 zero4 = make_uint4(0, 0, 0, 0);
        const uint4 va = t0 + tokA < p.n_r ? vpre[2 * i] : zero4;
        const uint4 vb = t0 + tokA + 8 < p.n_r ? vpre[2 * i + 1] : zero4;
        const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float a0 = __uint_as_float(wa[e] << 16), a1 = __uint_as_float(wa[e] & 0xFFFF0000u);
          const float b0 = __uint_as_float(wb[e] << 16), b1 = __uint_as_float(wb[e] & 0xFFFF0000u);
          *reinterpret_cast<uint32_t*>(&vrows[8 * seg + 2 * e][pos]) = pack_f16x2(a0, b0);
          *reinterpret_cast<uint32_t*>(&vrows[8 * seg + 2 * e + 1][pos]) = pack_f16x2(a1, b1);
        }
      }
    }
  };

  // ---------------- stream state ----------------
  // A block's scores sit in sqh (int32 sums for cached keys, fp32 bits for current
  // ones) and cb (bias MFMA output) between its QK^T and its softmax; its fp16 P pairs
  // sit in pb until its PV.
  float l_s = 0.f, l_r = 0.f;

  f32x16 acc[CBLK];
  i32x16 sqh[1];
  i32x16 sqg1[1];  // kF6G: group 1's sums (group 0's in sqh)
  f32x16 cb[1];
  uint32_t pb[2][4];
#pragma unroll
  for (int c = 0; c < CBLK; c++) acc[c] = f32x16{};

  // Key-side operands of block mb of tile U: the bias row and the key codes (cached) or
  // bf16 key rows (current), read from LDS ahead of their MFMAs.
  uint4 kbop;
  i32x4 kop[D / 16];
  i32x8 kop6[kF6 || kF6G ? KS6 : 1];  // key operands (fp4: 4 of 8 words used, fp6: 6)
  int rk_slot = 0, rk_mb = 0;  // group-wise keys: the block whose key rows qk reads
  auto read_k = [&](int slot, int mb, auto k_c) KVQ_INLINE {
    const typename SM::KSlot& ks = sm.k[slot];
    const int krow = 32 * mb + mrow_key(col);
    kbop = sm.prm[slot].kb[32 * mb + col][h];
    if constexpr (decltype(k_c)::value == kCached && kF6G) {
      // K-step g is group g: this lane half's 32 channels 64 g + 32 h .. (fp4 rows: 16
      // bytes; fp6 rows: 24)
#pragma unroll
      for (int g = 0; g < 2; g++) {
        if constexpr (BITS == 2) {
          const uint4 w4 = *reinterpret_cast<const uint4*>(&ks.c[krow][32 * g + 16 * h]);
          kop6[g] = i32x8{(int)w4.x, (int)w4.y, (int)w4.z, (int)w4.w, 0, 0, 0, 0};
        } else {
          const uint2* r = reinterpret_cast<const uint2*>(&ks.c[krow][48 * g + 24 * h]);
          const uint2 a = r[0], b = r[1], c = r[2];
          kop6[g] = i32x8{(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, 0, 0};
        }
      }
    } else if constexpr (decltype(k_c)::value == kCached && TG > 0) {
      // group-wise keys: qk reads the fp16 key rows one K-step ahead of their MFMAs
      rk_slot = slot;
      rk_mb = mb;
      kop[0] = *reinterpret_cast<const i32x4*>(&ks.kr[krow][HALF * h]);
    } else if constexpr (decltype(k_c)::value == kCached) {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; kk++) {
        if constexpr (PERCH)
          kop[kk] = *reinterpret_cast<const i32x4*>(&sm.kc(slot)[krow][HALF * h + 16 * kk]);
        else if constexpr (!kF6)
          kop[kk] = *reinterpret_cast<const i32x4*>(&ks.c[krow][HALF * h + 16 * kk]);
      }
      if constexpr (kF6 && BITS == 2) {
        // fp4 rows: channel c at nibble c of the row (in kperm6 order per 32 channels)
#pragma unroll
        for (int k6 = 0; k6 < KS6; k6++) {
          const uint4 w4 = *reinterpret_cast<const uint4*>(&ks.c[krow][(HALF * h + 32 * k6) / 2]);
          kop6[k6] = i32x8{(int)w4.x, (int)w4.y, (int)w4.z, (int)w4.w, 0, 0, 0, 0};
        }
      } else if constexpr (kF6) {
        // fp6 rows: 32 channels in 24 bytes, channel order
#pragma unroll
        for (int k6 = 0; k6 < KS6; k6++) {
          const uint2* r = reinterpret_cast<const uint2*>(&ks.c[krow][3 * (HALF * h + 32 * k6) / 4]);
          const uint2 a = r[0], b = r[1], c = r[2];
          kop6[k6] = i32x8{(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, 0, 0};
        }
      }
    } else {  // fp16 rows: current-chunk keys (bf16)
#pragma unroll
      for (int t = 0; t < D / 16; t++) kop[t] = *reinterpret_cast<const i32x4*>(&ks.kr[krow][HALF * h + 8 * t]);
    }
  };
  // QK^T and bias of the block whose operands read_k loaded, into score set SET.
  auto qk = [&](auto set_c, auto k_c) KVQ_INLINE {
    constexpr int SET = decltype(set_c)::value;
    {
      const f32x16 zf = {};
      cb[SET] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kbop), qbias, zf, 0, 0, 0);
    }
    if constexpr (decltype(k_c)::value == kCached && kF6G) {
      // S_g = sum over group g of q~_c code_c: one three-pass chain per group
      f32x16 s0 = {}, s1 = {};
      s0 = mfma_kq<kFA, 0>(kop6[0], q6[0][0], s0, q6sc[0]);
      s1 = mfma_kq<kFA, 2>(kop6[1], q6[1][0], s1, q6sc[0]);
      s0 = mfma_kq<kFA, 1>(kop6[0], q6[0][1], s0, q6sc[0]);
      s1 = mfma_kq<kFA, 3>(kop6[1], q6[1][1], s1, q6sc[0]);
      s0 = mfma_kq<kFA, 0>(kop6[0], q6[0][2], s0, q6sc[1]);
      s1 = mfma_kq<kFA, 1>(kop6[1], q6[1][2], s1, q6sc[1]);
      sqh[SET] = __builtin_bit_cast(i32x16, s0);
      sqg1[SET] = __builtin_bit_cast(i32x16, s1);
    } else if constexpr (decltype(k_c)::value == kCached && TG > 0) {
      // S = k_hat' . (q'_hi + q'_lo) on fp16 MFMA, fp32 accumulation, K-step by K-step
      // (each key operand is read one K-step ahead and used by the hi and the lo MFMA)
      const uint16_t* krow = &sm.k[rk_slot].kr[32 * rk_mb + mrow_key(col)][HALF * h];
      f32x16 sc = {};
      i32x4 kcur = kop[0];
#pragma unroll
      for (int t = 0; t < D / 16; t++) {
        i32x4 knext = kcur;
        if (t + 1 < D / 16) knext = *reinterpret_cast<const i32x4*>(krow + 8 * (t + 1));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kcur), q16h[t], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kcur), q16l[t], sc, 0, 0, 0);
        kcur = knext;
      }
      sqh[SET] = __builtin_bit_cast(i32x16, sc);
    } else if constexpr (decltype(k_c)::value == kCached && kF6) {
      // S = sum_c q'_c code_c in fp32, pass by pass; the key scale 2^1 (E8M0 128) turns the
      // fp4 values code / 2 into the codes
      sqh[SET] = __builtin_bit_cast(i32x16, qk_fp6<kFA>(kop6, q6, q6sc));
    } else if constexpr (decltype(k_c)::value == kCached) {
      // S = 256 S_hi + S_lo in one accumulator: the hi sums, a shift, then the lo sums
      i32x16 acc_s = {};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; kk++) acc_s = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[kk], qhi[kk], acc_s, 0, 0, 0);
      acc_s = acc_s << 8;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; kk++) acc_s = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[kk], qlo[kk], acc_s, 0, 0, 0);
      sqh[SET] = acc_s;
    } else {
      f32x16 sc;
#pragma unroll
      for (int t = 0; t < D / 16; t++) {
        const bf16x8 qop = __builtin_bit_cast(bf16x8, t < KSTEPS ? qhi[t] : qlo[t - KSTEPS]);
        const bf16x8 aop = __builtin_bit_cast(bf16x8, kop[t]);
        if (t == 0) {
          const f32x16 z = {};
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qop, z, 0, 0, 0);
        } else {
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qop, sc, 0, 0, 0);
        }
      }
      sqh[SET] = __builtin_bit_cast(i32x16, sc);
    }
  };
  // Value operands of block mb of tile U, read from LDS ahead of the PV MFMAs.
  f16x8 vop[2][CBLK];
  auto read_v = [&](int slot, int mb) KVQ_INLINE {
    if constexpr (!MASS_ONLY) {
      const _Float16(*vrows)[SM::VROW] = sm.v[slot];
#pragma unroll
      for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int c = 0; c < CBLK; c++)
          vop[ks][c] = *reinterpret_cast<const f16x8*>(&vrows[32 * c + col][32 * mb + 16 * ks + 8 * h]);
    }
  };
  // PV of the block whose values read_v loaded, with the pairs in pb.
  auto pv = [&]() KVQ_INLINE {
    if constexpr (!MASS_ONLY) {
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(pb[ks][0], pb[ks][1], pb[ks][2], pb[ks][3]));
#pragma unroll
        for (int c = 0; c < CBLK; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop[ks][c], bop, acc[c], 0, 0, 0);
      }
    }
  };
  // Logits (log2 units; they carry -m through the bias) of block mb of tile U from SET.
  auto logits = [&](int slot, int mb, auto set_c, auto k_c, float* x) KVQ_INLINE {
    constexpr int SET = decltype(set_c)::value;
    if constexpr (decltype(k_c)::value == kCached && kF6G) {
      const float* d0 = sm.prm[slot].dka[0];
      const float* d1 = sm.prm[slot].dka[1];
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const float4 a4 = *reinterpret_cast<const float4*>(&d0[32 * mb + 8 * v4 + 4 * h]);
        const float4 b4 = *reinterpret_cast<const float4*>(&d1[32 * mb + 8 * v4 + 4 * h]);
        const float da[4] = {a4.x, a4.y, a4.z, a4.w}, db[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int v = 4 * v4 + b;
          x[v] = fmaf(da[b], __int_as_float(sqh[SET][v]), fmaf(db[b], __int_as_float(sqg1[SET][v]), cb[SET][v]));
        }
      }
    } else if constexpr (decltype(k_c)::value == kCached && TG > 0) {
#pragma unroll
      for (int v = 0; v < 16; v++) x[v] = fmaf(scale_l2, __int_as_float(sqh[SET][v]), cb[SET][v]);
      if constexpr (EXACT) {
        // the exact correction's terms past the second order, per channel group:
        // -b gains Delta_g^4 (c2 M2^g - Delta_g^2 (c3 M3^g - Delta_g^2 c4 M4^g))
        const _Float16* dkg = reinterpret_cast<const _Float16*>(&sm.prm[slot].dka[0][0]);
#pragma unroll
        for (int g = 0; g < NG; g++)
#pragma unroll
          for (int v4 = 0; v4 < 4; v4++) {
            const f16x4 d4 = *reinterpret_cast<const f16x4*>(&dkg[g * kBN + 32 * mb + 8 * v4 + 4 * h]);
#pragma unroll
            for (int b = 0; b < 4; b++) {
              const float dd = (float)d4[b], u = dd * dd;
              const float t = fmaf(-u, fmaf(-u, exg[2][g], exg[1][g]), exg[0][g]);
              x[4 * v4 + b] = fmaf(u * u, t, x[4 * v4 + b]);
            }
          }
      }
    } else if constexpr (decltype(k_c)::value == kCached && PERCH) {
#pragma unroll
      for (int v = 0; v < 16; v++) x[v] = fmaf(a_ch, (float)sqh[SET][v], cb[SET][v]);
    } else if constexpr (decltype(k_c)::value == kCached) {
      const float* dka = sm.prm[slot].dka[wave];
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const float4 d4 = *reinterpret_cast<const float4*>(&dka[32 * mb + 8 * v4 + 4 * h]);
        const float d[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int v = 4 * v4 + b;
          x[v] = fmaf(d[b], kF6 ? __int_as_float(sqh[SET][v]) : (float)sqh[SET][v], cb[SET][v]);
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; v++) x[v] = fmaf(scale_l2, __int_as_float(sqh[SET][v]), cb[SET][v]);
    }
  };
  // fp16 P pairs with p = exp2(x - off) into pb; returns this lane's fp16 sum.
  auto pairs = [&](const float* x, float off) KVQ_INLINE {
    float ls2[2] = {0.f, 0.f};  // two dependency chains of four dot2 each
    const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int v2 = 0; v2 < 8; v2++) {
      const uint32_t pr = pack_f16x2(exp2_(x[2 * v2] - off), exp2_(x[2 * v2 + 1] - off));
      pb[v2 >> 2][v2 & 3] = pr;
      ls2[v2 & 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pr), ones, ls2[v2 & 1], false);
    }
    return ls2[0] + ls2[1];
  };
  // Softmax numerators of block mb of tile U (scores in SET). The reference m starts at
  // the maximum of the stream's first block plus a headroom of 2^2 (FIRST) and is raised
  // only when a block's fp16 row sum passes 2^15 (some p may have left the fp16 range):
  // then m becomes that block's maximum, the sums and the accumulator are rescaled and
  // the block's p recomputed (a rare, wave-uniform branch).
  auto softmax = [&](int slot, int mb, auto set_c, auto k_c, auto first_c) KVQ_INLINE {
    float x[16];
    logits(slot, mb, set_c, k_c, x);
    float lsum = 0.f;
    bool done = false;
    if constexpr (decltype(first_c)::value) {
      if (__builtin_amdgcn_readfirstlane(m_run == -INFINITY ? 1 : 0)) {
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; v++) mx = fmaxf(mx, x[v]);
        mx = fmaxf(mx, xor32(mx));
        set_m(mx + kHeadroom);
        lsum = pairs(x, m_run);
        done = true;
      }
    }
    if (!done) {
      lsum = pairs(x, 0.f);
      const bool raise = !(lsum <= kPmax);
      if (__ballot(raise) != 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; v++) mx = fmaxf(mx, x[v]);
        mx = fmaxf(mx, xor32(mx));
        // either half of the query (the shuffle runs on every lane, outside any ||)
        const float partner_raise = xor32(raise ? 1.f : 0.f);
        const bool up = raise || partner_raise != 0.f;
        const float m_old = m_run;
        set_m(up ? m_old + mx : m_old);
        const float sc = exp2_(m_old - m_run);
        l_s *= sc;
        l_r *= sc;
        if constexpr (!MASS_ONLY) {
#pragma unroll
          for (int c = 0; c < CBLK; c++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[c][v] *= sc;
        }
        lsum = pairs(x, m_run - m_old);
      }
    }
    if constexpr (decltype(k_c)::value == kCached)
      l_s += lsum;
    else
      l_r += lsum;
  };

  auto unrotate = [&]() KVQ_INLINE {
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
        const float pvv = xor32(acc[c][v]);
        acc[c][v] = h ? (pvv - acc[c][v]) : (acc[c][v] + pvv);
      }
#pragma unroll
    for (int cbk = 1; cbk < CBLK; cbk <<= 1)  // channel bits 5, 6: the 32-channel block
#pragma unroll
      for (int c = 0; c < CBLK; c++)
        if ((c & cbk) == 0)
#pragma unroll
          for (int v = 0; v < 16; v++) {
            const float a = acc[c][v], b = acc[c | cbk][v];
            acc[c][v] = a + b;
            acc[c | cbk][v] = a - b;
          }
    const float cn = rsqrtf((float)D);
#pragma unroll
    for (int c = 0; c < CBLK; c++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[c][v] *= cn;
    if (p.v_sg[0] | p.v_sg[1] | p.v_sg[2] | p.v_sg[3]) {  // randomized rotation: diag(t) H
#pragma unroll
      for (int c = 0; c < CBLK; c++) {
        const uint32_t wv = p.v_sg[c] >> (4 * h);
#pragma unroll
        for (int v = 0; v < 16; v++)
          acc[c][v] = __uint_as_float(__float_as_uint(acc[c][v]) ^ (((wv >> ((v & 3) + 8 * (v >> 2))) & 1u) << 31));
      }
    }
  };

  // Per-channel keys issue a tile's global loads a step earlier: its keys right after the
  // previous tile's keys are stored, its values right after the previous values are
  // stored (before the barrier), so the loads have a whole step to arrive; per-token keys
  // issue both at the step start (measured faster there).
  constexpr bool kEarlyK = PERCH;
  // Step T of a run of n_t tiles of one kind (tile index U = U0 + T in LDS slot slot0;
  // the next two tiles in slots slot1, slot2): QK^T, softmax and PV of the tile's two 32-key
  // blocks, while the keys of tile U+2 and the values of tile U+1 are staged. FIRST:
  // block (U,0) may be the stream's first.
  auto step = [&](int U0, int n_t, int T, int slot0, int slot1, int slot2, auto k_c, auto first_c) KVQ_INLINE {
    const Kind<0> set0;
    const std::false_type no;
    const int U = U0 + T;
    const bool stage_k = T + 2 < n_t, stage_v = T + 1 < n_t;
    if (!kEarlyK && stage_k) load_k(U + 2, k_c);
    if (!kEarlyK && stage_v) load_v(U + 1, k_c);
    if (computes) {
      if constexpr (PERCH && decltype(k_c)::value == kCached) {
        if (T == 0 || (U % tiles_per_chunk) % k_tpg == 0) refresh_group(slot0);
      }
      // operand reads are issued one phase ahead of their MFMAs (the sched barriers keep
      // the compiler from sinking them): values under the softmax, keys under the PV
      // (group-wise keys read a block's values after its softmax: their fp16 query halves
      // take the registers)
      constexpr bool kLateV = TG > 0 && !kF6G && decltype(k_c)::value == kCached;
      read_k(slot0, 0, k_c);
      qk(set0, k_c);
      if (!kLateV) read_v(slot0, 0);
      __builtin_amdgcn_sched_barrier(0);
      softmax(slot0, 0, set0, k_c, first_c);
      if (kLateV) read_v(slot0, 0);
      read_k(slot0, 1, k_c);
      __builtin_amdgcn_sched_barrier(0);
      pv();
      qk(set0, k_c);
      if (!kLateV) read_v(slot0, 1);
      __builtin_amdgcn_sched_barrier(0);
      // the key staging (VALU and LDS writes) runs in the shadow of block 1's QK^T MFMAs
      // (4-bit keys on the fp6 path: at the end of the step, where their conversion's 32
      // floats do not meet the live scores)
      constexpr bool kLateK = (kF6 || kF6G) && BITS == 4 && decltype(k_c)::value == kCached;
      if (!kLateK && stage_k) store_k(U + 2, slot2, k_c);
      if (kEarlyK && T + 3 < n_t) load_k(U + 3, k_c);
      __builtin_amdgcn_sched_barrier(0);
      softmax(slot0, 1, set0, k_c, no);
      if (kLateV) read_v(slot0, 1);
      pv();
      if (kLateK && stage_k) store_k(U + 2, slot2, k_c);
    } else {
      if (stage_k) store_k(U + 2, slot2, k_c);
      if (kEarlyK && T + 3 < n_t) load_k(U + 3, k_c);
    }
    if (stage_v) store_v(U + 1, slot1, k_c);
    if (kEarlyK && T + 2 < n_t) load_v(U + 2, k_c);
    __syncthreads();
  };
  // All tiles of one kind (tile U0 + T in slot T mod 3, the slots rotating with T): stage
  // the first two tiles' keys and the first values, then run the steps.
  // (with kPre the caller has issued tile U0's key and value loads)
  auto run = [&](int U0, int n_t, auto k_c) KVQ_INLINE {
    const std::false_type no;
    if constexpr (!kPre) load_k(U0, k_c);
    store_k(U0, 0, k_c);
    if (n_t > 1) {
      load_k(U0 + 1, k_c);
      store_k(U0 + 1, 1, k_c);
    }
    __syncthreads();
    if constexpr (!kPre) load_v(U0, k_c);
    store_v(U0, 0, k_c);
    if (kEarlyK && n_t > 2) load_k(U0 + 2, k_c);
    if (kEarlyK && n_t > 1) load_v(U0 + 1, k_c);
    __syncthreads();
    step(U0, n_t, 0, 0, 1, 2, k_c, std::true_type());
    int s0 = 1, s1 = 2, s2 = 0;
    for (int T = 1; T < n_t; T++) {
      step(U0, n_t, T, s0, s1, s2, k_c, no);
      const int t = s0;
      s0 = s1;
      s1 = s2;
      s2 = t;
    }
  };

  // ---------------- this workgroup's tiles: cached ones, then current ones ----------------
  // Share sp of the tile sequence (cached tiles 0..n_ct-1, then the current chunk's), the
  // shares cut at equal cost: a current tile (bf16 keys and values read from memory, bf16
  // QK^T on eight MFMAs per block) takes about 4/3 of a cached tile's time.
  const long long cost_all = 3LL * n_ct + 4LL * n_rt;
  auto cut = [&](int s) KVQ_INLINE -> int {
    const long long x = (long long)s * cost_all / p.n_split;
    return x <= 3LL * n_ct ? (int)(x / 3) : n_ct + (int)((x - 3LL * n_ct) / 4);
  };
  const int t_beg = cut(sp), t_end = cut(sp + 1);
  const int c_beg = min(t_beg, n_ct), c_end = min(t_end, n_ct);
  const int r_beg = max(t_beg, n_ct) - n_ct, r_end = max(t_end, n_ct) - n_ct;
  // With kPre each phase's first tile is loaded before the work that precedes the phase
  // (the query build, the un-rotation), whose instructions then cover the loads' latency.
  if constexpr (kPre) {
    if (c_end > c_beg) {
      load_k(c_beg, Kind<kCached>());
      load_v(c_beg, Kind<kCached>());
    } else if (r_end > r_beg) {
      load_k(n_ct + r_beg, Kind<kCurrent>());
      load_v(n_ct + r_beg, Kind<kCurrent>());
    }
    build_query();
  }
  if (c_end > c_beg) {
    if constexpr (PERCH) {
      if (computes) fill_qf();
    }
    run(c_beg, c_end - c_beg, Kind<kCached>());
    if constexpr (kPre) {
      if (r_end > r_beg) {
        load_k(n_ct + r_beg, Kind<kCurrent>());
        load_v(n_ct + r_beg, Kind<kCurrent>());
      }
    }
    if constexpr (!MASS_ONLY) {
      if (p.v_had && computes) unrotate();
    }
  }
  if (r_end > r_beg) {
    load_query_bf16();
    if constexpr (PERCH) {
      c_grp = 0.f;
      write_mslot();
    }
    run(n_ct + r_beg, r_end - r_beg, Kind<kCurrent>());
  }

  // ---------------- epilogue ----------------
  const float ls = l_s + xor32(l_s);
  const float lr = l_r + xor32(l_r);
  const float tot = ls + lr;
  if (!q_ok) return;
  if (p.part) {
    // partial record of this share: the unnormalized sum, its reference max and the sums
    float* rec = p.part + (((size_t)sp * p.B * p.H + bh) * p.n_q + qi) * (D + 4);
    if constexpr (!MASS_ONLY) {
#pragma unroll
      for (int c = 0; c < CBLK; c++)
#pragma unroll
        for (int v4 = 0; v4 < 4; v4++)
          *reinterpret_cast<float4*>(rec + 32 * c + 8 * v4 + 4 * h) =
              make_float4(acc[c][4 * v4], acc[c][4 * v4 + 1], acc[c][4 * v4 + 2], acc[c][4 * v4 + 3]);
    }
    if (h == 0) *reinterpret_cast<float4*>(rec + D) = make_float4(m_run, ls, lr, 0.f);
    return;
  }
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
    p.mass_s[(size_t)bh * p.n_q + qi] = ls * inv;
    p.mass_r[(size_t)bh * p.n_q + qi] = lr * inv;
  }
}

template <int D, int BITS, bool MASS_ONLY, bool PERCH, bool EXACT, int TG = 0>
__global__ __launch_bounds__(kThreads) void jb_attn_kernel(const Params p) {
  attn_body<D, BITS, MASS_ONLY, PERCH, EXACT, TG>(p, blockIdx.x, gridDim.x);
}

// Several calls in one launch: call c owns workgroups start[c] .. start[c] + grid[c] - 1.
// Every start is a multiple of 8, so a call's workgroup wg runs on XCD wg % 8 as it would
// alone; the few workgroups between one call's end and the next start exit at once.
constexpr int kMaxBatch = KVQ_BATCH_MAX;
struct BatchParams {
  Params p[kMaxBatch];
  int start[kMaxBatch];
  int grid[kMaxBatch];
  int n;
};

template <int D, int BITS, bool MASS_ONLY, bool PERCH, bool EXACT, int TG = 0>
__global__ __launch_bounds__(kThreads) void jb_attn_batch_kernel(const BatchParams bp) {
  int c = 0;
  while (c + 1 < bp.n && (int)blockIdx.x >= bp.start[c + 1]) c++;
  const int wg = (int)blockIdx.x - bp.start[c];
  if (wg >= bp.grid[c]) return;
  attn_body<D, BITS, MASS_ONLY, PERCH, EXACT, TG>(bp.p[c], wg, bp.grid[c]);
}

// ---------------- few queries: one wave per share of a head's cached tiles ----------------
// With at most 32 queries (one 32-query stream) the main kernel would keep one of its eight
// waves busy per workgroup while the cache stream is the real cost. Here a workgroup is a
// single wave that owns a contiguous share of one head's cached tiles and reads its
// operands straight from global memory in MFMA order: each lane loads its own key's code
// row half and step / zero point (the key of its M row), and the 64 cached tokens of its
// value channels, dequantized in registers. Small per-wave LDS tables broadcast the per-key
// factors of the logits and the value zero-point / step pairs. Queries, bias MFMA, softmax
// and PV follow the main kernel. A share ends with its partial record (un-rotated sum,
// reference max, l_S); the current chunk is one more share, and jb_combine_kernel merges.
struct SmemDec {
  float dka[kBN];        // Delta_j A, M-row order
  uint32_t zv[kBN / 2];  // value (-1024 - z) fp16 pairs, token pair (j, j+8) order
  uint32_t dv[kBN / 2];  // value step pairs
};

// n 32-bit words from a raw buffer at byte offset off (n = 2, 4 or 8)
template <int N>
__device__ inline void load_words(const __amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff, uint32_t* w) {
  if constexpr (N == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, soff, 0);
    w[0] = v[0];
    w[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < N / 4; i++) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u * i, soff, 0);
      w[4 * i] = v[0];
      w[4 * i + 1] = v[1];
      w[4 * i + 2] = v[2];
      w[4 * i + 3] = v[3];
    }
  }
}

// The current chunk of a few-query call as one more share of the decode grid (one wave):
// bf16 QK^T (exact products, no correction), the bias MFMA for -m and the padding mask, fp16
// P and values, written as a partial record (l_R, natural basis) for the merge. Key rows
// are read straight into MFMA operands: lane (h, col) holds channels HALF h .. of the
// block's key in M row col, as the main kernel's current tiles do from LDS.
template <int D, bool MASS_ONLY>
__device__ KVQ_INLINE void decode_current(const Params& p, const int bh, const int rec) {
  constexpr int HALF = D / 2;
  constexpr int CBLK = D / 32;
  const int lane = threadIdx.x;
  const int h = lane >> 5, col = lane & 31;
  const bool q_ok = col < p.n_q;
  const int qi = q_ok ? col : 0;
  const float scale_l2 = p.s * kLog2e;
  const uint16_t* kr = p.k_cur + (size_t)bh * p.n_r * D;
  const uint16_t* vr = p.v_cur + (size_t)bh * p.n_r * D;
  bf16x8 qop[D / 16];
  {
    const uint4* qrow = reinterpret_cast<const uint4*>(p.q + ((size_t)bh * p.n_q + qi) * D + HALF * h);
#pragma unroll
    for (int t = 0; t < D / 16; t++) qop[t] = __builtin_bit_cast(bf16x8, q_ok ? qrow[t] : make_uint4(0, 0, 0, 0));
  }
  f16x8 qbias;
#pragma unroll
  for (int e = 0; e < 8; e++) qbias[e] = (_Float16)0.f;
  if (h) qbias[2] = (_Float16)(-kMaskLogit);
  float m_run = -INFINITY;
  auto set_m = [&](float mx) KVQ_INLINE {
    _Float16 mh, ml;
    split16(-mx, mh, ml);
    m_run = -((float)mh + (float)ml);
    qbias[0] = h ? mh : qbias[0];
    qbias[1] = h ? ml : qbias[1];
  };
  float l_r = 0.f;
  f32x16 acc[CBLK];
#pragma unroll
  for (int c = 0; c < CBLK; c++) acc[c] = f32x16{};
  uint32_t pb[2][4];
  const int n_rt = (p.n_r + kBN - 1) / kBN;
  for (int U = 0; U < n_rt; U++) {
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      const int t0 = U * kBN + 32 * mb;
      const int tok = t0 + mrow_key(col);
      const bool kv = tok < p.n_r;
      const uint4* krow = reinterpret_cast<const uint4*>(kr + (size_t)min(tok, p.n_r - 1) * D + HALF * h);
      bf16x8 kop[D / 16];
#pragma unroll
      for (int t = 0; t < D / 16; t++) kop[t] = __builtin_bit_cast(bf16x8, kv ? krow[t] : make_uint4(0, 0, 0, 0));
      const uint32_t one = 0x3C00u;
      const uint4 kbop = h ? make_uint4(one | (one << 16), kv ? 0u : one, 0u, 0u) : make_uint4(0, 0, 0, 0);
      const f32x16 zf = {};
      const f32x16 cbv = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kbop), qbias, zf, 0, 0, 0);
      f32x16 sc = {};
#pragma unroll
      for (int t = 0; t < D / 16; t++) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[t], qop[t], sc, 0, 0, 0);
      float x[16];
#pragma unroll
      for (int v = 0; v < 16; v++) x[v] = fmaf(scale_l2, sc[v], cbv[v]);
      auto pairs = [&](float off) KVQ_INLINE {
        float ls2[2] = {0.f, 0.f};
        const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
        for (int v2 = 0; v2 < 8; v2++) {
          const uint32_t pr = pack_f16x2(exp2_(x[2 * v2] - off), exp2_(x[2 * v2 + 1] - off));
          pb[v2 >> 2][v2 & 3] = pr;
          ls2[v2 & 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pr), ones, ls2[v2 & 1], false);
        }
        return ls2[0] + ls2[1];
      };
      float lsum;
      if (__builtin_amdgcn_readfirstlane(m_run == -INFINITY ? 1 : 0)) {
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; v++) mx = fmaxf(mx, x[v]);
        mx = fmaxf(mx, xor32(mx));
        set_m(mx + kHeadroom);
        lsum = pairs(m_run);
      } else {
        lsum = pairs(0.f);
        const bool raise = !(lsum <= kPmax);
        if (__ballot(raise) != 0) {
          float mx = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; v++) mx = fmaxf(mx, x[v]);
          mx = fmaxf(mx, xor32(mx));
          const float partner_raise = xor32(raise ? 1.f : 0.f);
          const bool up = raise || partner_raise != 0.f;
          const float m_old = m_run;
          set_m(up ? m_old + mx : m_old);
          const float scl = exp2_(m_old - m_run);
          l_r *= scl;
          if constexpr (!MASS_ONLY) {
#pragma unroll
            for (int c = 0; c < CBLK; c++)
#pragma unroll
              for (int v = 0; v < 16; v++) acc[c][v] *= scl;
          }
          lsum = pairs(m_run - m_old);
        }
      }
      l_r += lsum;
      if constexpr (!MASS_ONLY) {
        // value operands: element i of lane (h, col) is token 4 h + (i >> 1) + 8 (i & 1) of
        // 16-key group ks, channel 32 c + col (the P operand's key order)
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          f16x8 vop[CBLK];
#pragma unroll
          for (int c = 0; c < CBLK; c++) {
            uint32_t w[4];
#pragma unroll
            for (int i2 = 0; i2 < 4; i2++) {
              float f[2];
#pragma unroll
              for (int e = 0; e < 2; e++) {
                const int tv = t0 + 16 * ks + 4 * h + i2 + 8 * e;
                const uint16_t b = vr[(size_t)min(tv, p.n_r - 1) * D + 32 * c + col];
                f[e] = tv < p.n_r ? __uint_as_float((uint32_t)b << 16) : 0.f;
              }
              w[i2] = pack_f16x2(f[0], f[1]);
            }
            vop[c] = __builtin_bit_cast(f16x8, make_uint4(w[0], w[1], w[2], w[3]));
          }
          const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(pb[ks][0], pb[ks][1], pb[ks][2], pb[ks][3]));
#pragma unroll
          for (int c = 0; c < CBLK; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop[c], bop, acc[c], 0, 0, 0);
        }
      }
    }
  }
  const float lr = l_r + xor32(l_r);
  if (!q_ok) return;
  float* out = p.part + (((size_t)rec * p.B * p.H + bh) * p.n_q + qi) * (D + 4);
  if constexpr (!MASS_ONLY) {
#pragma unroll
    for (int c = 0; c < CBLK; c++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++)
        *reinterpret_cast<float4*>(out + 32 * c + 8 * v4 + 4 * h) =
            make_float4(acc[c][4 * v4], acc[c][4 * v4 + 1], acc[c][4 * v4 + 2], acc[c][4 * v4 + 3]);
  }
  if (h == 0) *reinterpret_cast<float4*>(out + D) = make_float4(m_run, 0.f, lr, 0.f);
}

template <int D, int BITS, bool MASS_ONLY>
__global__ __launch_bounds__(64, 2) void jb_decode_kernel(const Params p, const int shares) {
  constexpr int HALF = D / 2;
  constexpr int KSTEPS = D / 32;
  constexpr int CBLK = D / 32;
  constexpr int KW = D * BITS / 32;     // key words per token
  constexpr int KWH = KW / 2;           // key words of one half row (a lane's operand)
  constexpr int CPW = 32 / BITS;
  constexpr int VWPC = kBN / CPW;       // value words per channel per tile
  constexpr int VWT = D * VWPC;         // value words per tile
  __shared__ SmemDec sm;
  const int lane = threadIdx.x;
  const int h = lane >> 5, col = lane & 31;
  const int per = shares + (p.n_r > 0 ? 1 : 0);  // the last share of a head: its current chunk
  const int bh = blockIdx.x / per, sp = blockIdx.x % per;
  if (sp == shares) {
    decode_current<D, MASS_ONLY>(p, bh, shares);
    return;
  }
  const bool q_ok = col < p.n_q;
  const int qi = q_ok ? col : 0;
  const float scale_l2 = p.s * kLog2e;

  // ---- query operands: 2-bit keys, the rotated query as three fp6 passes (scaled fp4 x fp6
  // QK^T); 4-bit keys, as 16-bit fixed point split into int8 hi/lo (the main kernel's builds)
  constexpr bool kF6 = BITS == 2;
  constexpr int KS6 = D / 64;
  i32x4 qhi[kF6 ? 1 : KSTEPS], qlo[kF6 ? 1 : KSTEPS];
  i32x8 q6[kF6 ? KS6 : 1][3];
  uint32_t q6sc[2] = {0u, 0u};
  f16x8 qbias;
  float A;
  {
    float qv[HALF];
    const uint16_t* qrow = p.q + ((size_t)bh * p.n_q + qi) * D + HALF * h;
    uint32_t sgw[HALF / 32];
#pragma unroll
    for (int k = 0; k < HALF / 32; k++) sgw[k] = h ? p.k_sg[HALF / 32 + k] : p.k_sg[k];
#pragma unroll
    for (int u = 0; u < HALF / 8; u++) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (q_ok) w = reinterpret_cast<const uint4*>(qrow)[u];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int j = 8 * u + 2 * e;
        const uint32_t we = ww[e] ^ pair_sign_xor(sgw[j >> 5], j & 31);
        qv[j] = __uint_as_float(we << 16);
        qv[j + 1] = __uint_as_float(we & 0xFFFF0000u);
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
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) mxa = fmaxf(mxa, __shfl_xor(mxa, sh));
    float qsum;  // the sum of the query channels as the QK^T operands hold them
    if constexpr (kF6) {
      A = scale_l2;
      const float lsum = encode_query_fp6<HALF, 2>(qv, q6, q6sc);
      qsum = lsum + xor32(lsum);
    } else {
      const float inv = mxa > 0.f ? kQFix / mxa : 0.f;
      A = mxa > 0.f ? scale_l2 * (mxa / kQFix) : 0.f;
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
      qsum = (float)qs;
    }
    const float G = p.correction ? p.s * p.s * ss * (1.f / 24.f) * kLog2e : 0.f;
    _Float16 wh, wl, gh, gl;
    split16(-A * qsum, wh, wl);
    split16(-G * kD2Scale, gh, gl);
    if (h == 0) {
      qbias[0] = wh;
      qbias[1] = wl;
      qbias[2] = wh;
      qbias[3] = gh;
      qbias[4] = gl;
      qbias[5] = gh;
      qbias[6] = (_Float16)0.f;
      qbias[7] = (_Float16)0.f;
    } else {
      qbias[0] = (_Float16)0.f;  // -m (hi, lo) once m is set
      qbias[1] = (_Float16)0.f;
      qbias[2] = (_Float16)(-kMaskLogit);
#pragma unroll
      for (int e = 3; e < 8; e++) qbias[e] = (_Float16)0.f;
    }
  }
  float m_run = -INFINITY;
  auto set_m = [&](float mx) KVQ_INLINE {
    _Float16 mh, ml;
    split16(-mx, mh, ml);
    m_run = -((float)mh + (float)ml);
    qbias[0] = h ? mh : qbias[0];
    qbias[1] = h ? ml : qbias[1];
  };

  // ---- this share's cached tiles
  const int tpc = p.cp / kBN;
  const int n_ct = p.n_chunks * tpc;
  const int t_beg = (int)((long long)sp * n_ct / shares), t_end = (int)((long long)(sp + 1) * n_ct / shares);
  const size_t n_tot = (size_t)p.n_chunks * p.cp;
  const size_t n_str = (size_t)p.n_wchunks * p.cp;
  const __amdgpu_buffer_rsrc_t rs_kc = buffer_rsrc(p.k_codes + (size_t)bh * n_str * KW, (uint32_t)(n_tot * KW * 4));
  const __amdgpu_buffer_rsrc_t rs_vc =
      buffer_rsrc(p.v_codes + (size_t)bh * (n_str / kBN) * VWT, (uint32_t)(n_tot / kBN * VWT * 4));
  const __amdgpu_buffer_rsrc_t rs_ks = buffer_rsrc(p.k_scale + (size_t)bh * n_str, (uint32_t)(n_tot * 2));
  const __amdgpu_buffer_rsrc_t rs_kz = buffer_rsrc(p.k_zero + (size_t)bh * n_str, (uint32_t)(n_tot * 2));
  const __amdgpu_buffer_rsrc_t rs_vs = buffer_rsrc(p.v_scale + (size_t)bh * n_str, (uint32_t)(n_tot * 2));
  const __amdgpu_buffer_rsrc_t rs_vz = buffer_rsrc(p.v_zero + (size_t)bh * n_str, (uint32_t)(n_tot * 2));

  // raw operands of one tile: this lane's key (M row col) of both blocks, its step and
  // zero point, the value zero-point / step pair of token pair (lane), and the value
  // words of channels 32c + col
  struct Raw {
    uint32_t k[2][KWH];
    uint32_t kd[2], kz[2];
    uint32_t vz0, vz1, vd0, vd1;
    uint32_t v[CBLK][VWPC];
  };
  const int krow[2] = {mrow_key(col), 32 + mrow_key(col)};
  const int vg = (lane >> 3) & 3, vj = lane & 7;  // value token pair (16 vg + vj, + 8)
  auto load_raw = [&](int U, Raw& r) KVQ_INLINE {
    const uint32_t tok0 = (uint32_t)U * kBN;
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      load_words<KWH>(rs_kc, ((uint32_t)krow[mb] * KW + (uint32_t)h * KWH) * 4u, tok0 * KW * 4u, r.k[mb]);
      r.kd[mb] = __builtin_amdgcn_raw_buffer_load_b16(rs_ks, (uint32_t)krow[mb] * 2u, tok0 * 2u, 0);
      r.kz[mb] = __builtin_amdgcn_raw_buffer_load_b16(rs_kz, (uint32_t)krow[mb] * 2u, tok0 * 2u, 0);
    }
    if constexpr (!MASS_ONLY) {
      const uint32_t t = (uint32_t)(16 * vg + vj);
      r.vz0 = __builtin_amdgcn_raw_buffer_load_b16(rs_vz, t * 2u, tok0 * 2u, 0);
      r.vz1 = __builtin_amdgcn_raw_buffer_load_b16(rs_vz, t * 2u + 16u, tok0 * 2u, 0);
      r.vd0 = __builtin_amdgcn_raw_buffer_load_b16(rs_vs, t * 2u, tok0 * 2u, 0);
      r.vd1 = __builtin_amdgcn_raw_buffer_load_b16(rs_vs, t * 2u + 16u, tok0 * 2u, 0);
#pragma unroll
      for (int c = 0; c < CBLK; c++)
        load_words<VWPC>(rs_vc, (uint32_t)(32 * c + col) * VWPC * 4u, (uint32_t)U * VWT * 4u, r.v[c]);
    }
  };

  float l_s = 0.f;
  f32x16 acc[CBLK];
#pragma unroll
  for (int c = 0; c < CBLK; c++) acc[c] = f32x16{};
  uint32_t pb[2][4];
  // the value code field mask in a vector register, so that the unpack takes one and-or
  // per pair (with two literals it would take an and and an or); 2-bit pair i of a value
  // word sits at bit 8 h + 2 i for this lane half
  uint32_t vmask = BITS == 2 ? 0x00030003u : 0x000F000Fu;
  asm volatile("" : "+v"(vmask));
  uint32_t vsh[4];
#pragma unroll
  for (int i = 0; i < 4; i++) vsh[i] = (uint32_t)(8 * h + 2 * i);

  // two waves per SIMD (at most 256 registers) hide each other's load latency; holding a
  // second tile's operands in registers would cost that occupancy
  for (int U = t_beg; U < t_end; U++) {
    Raw cur;
    load_raw(U, cur);
    const int nv = min(kBN, p.chunk_len - (U % tpc) * kBN);
    // per-key factors of both blocks into the wave's tables
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      if (h == 0) sm.dka[32 * mb + col] = krow[mb] < nv ? half_bits_to_f32(cur.kd[mb]) * A : 0.f;
    }
    if constexpr (!MASS_ONLY) {
      if (lane < kBN / 2) {
        const bool ok0 = 16 * vg + vj < nv, ok1 = 16 * vg + vj + 8 < nv;
        sm.zv[lane] = pack_f16x2(ok0 ? -1024.f - half_bits_to_f32(cur.vz0) : -1024.f,
                                 ok1 ? -1024.f - half_bits_to_f32(cur.vz1) : -1024.f);
        sm.dv[lane] = (ok0 ? (cur.vd0 & 0xFFFFu) : 0u) | ((ok1 ? (cur.vd1 & 0xFFFFu) : 0u) << 16);
      }
    }
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      // bias operand of this lane's M row: slots 0..7 (h = 0) or 8..15 (h = 1)
      uint4 kbop = make_uint4(0, 0, 0, 0);
      const bool kv = krow[mb] < nv;
      if (h == 0) {
        if (kv) {
          const float dk = half_bits_to_f32(cur.kd[mb]), zk = half_bits_to_f32(cur.kz[mb]);
          _Float16 dzh, dzl, d2h, d2l;
          split16(dk * zk, dzh, dzl);
          split16(dk * dk * (1.f / kD2Scale), d2h, d2l);
          const uint32_t dzh_b = __builtin_bit_cast(uint16_t, dzh), dzl_b = __builtin_bit_cast(uint16_t, dzl);
          const uint32_t d2h_b = __builtin_bit_cast(uint16_t, d2h), d2l_b = __builtin_bit_cast(uint16_t, d2l);
          kbop = make_uint4(dzh_b | (dzh_b << 16), dzl_b | (d2h_b << 16), d2h_b | (d2l_b << 16), 0u);
        }
      } else {
        const uint32_t one = 0x3C00u;
        kbop = make_uint4(one | (one << 16), kv ? 0u : one, 0u, 0u);
      }
      const f32x16 zf = {};
      const f32x16 cbv = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kbop), qbias, zf, 0, 0, 0);
      float sqf[16];  // S = sum_c q_c code_c of this lane's 16 scores
      if constexpr (kF6) {
        i32x8 ka[KS6];
#pragma unroll
        for (int k6 = 0; k6 < KS6; k6++) ka[k6] = fp4_key_operand(cur.k[mb][2 * k6], cur.k[mb][2 * k6 + 1]);
        const f32x16 sf = qk_fp6<4>(ka, q6, q6sc);
#pragma unroll
        for (int v = 0; v < 16; v++) sqf[v] = sf[v];
      } else {
        // key codes as int8 (kperm order in each 16-channel unit)
        i32x4 kop[KSTEPS];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) {
          const uint32_t w0 = cur.k[mb][2 * kk], w1 = cur.k[mb][2 * kk + 1];
          kop[kk] = i32x4{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu),
                          (int)((w1 >> 4) & 0x0F0F0F0Fu)};
        }
        i32x16 sq = {};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) sq = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[kk], qhi[kk], sq, 0, 0, 0);
        sq = sq << 8;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) sq = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[kk], qlo[kk], sq, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; v++) sqf[v] = (float)sq[v];
      }
      // logits (log2 units, -m through the bias) and softmax numerators
      float x[16];
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dka[32 * mb + 8 * v4 + 4 * h]);
        const float d[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int b = 0; b < 4; b++) x[4 * v4 + b] = fmaf(d[b], sqf[4 * v4 + b], cbv[4 * v4 + b]);
      }
      auto pairs = [&](float off) KVQ_INLINE {
        float ls2[2] = {0.f, 0.f};
        const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
        for (int v2 = 0; v2 < 8; v2++) {
          const uint32_t pr = pack_f16x2(exp2_(x[2 * v2] - off), exp2_(x[2 * v2 + 1] - off));
          pb[v2 >> 2][v2 & 3] = pr;
          ls2[v2 & 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pr), ones, ls2[v2 & 1], false);
        }
        return ls2[0] + ls2[1];
      };
      float lsum;
      if (__builtin_amdgcn_readfirstlane(m_run == -INFINITY ? 1 : 0)) {
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; v++) mx = fmaxf(mx, x[v]);
        mx = fmaxf(mx, xor32(mx));
        set_m(mx + kHeadroom);
        lsum = pairs(m_run);
      } else {
        lsum = pairs(0.f);
        const bool raise = !(lsum <= kPmax);
        if (__ballot(raise) != 0) {
          float mx = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; v++) mx = fmaxf(mx, x[v]);
          mx = fmaxf(mx, xor32(mx));
          const float partner_raise = xor32(raise ? 1.f : 0.f);
          const bool up = raise || partner_raise != 0.f;
          const float m_old = m_run;
          set_m(up ? m_old + mx : m_old);
          const float sc = exp2_(m_old - m_run);
          l_s *= sc;
          if constexpr (!MASS_ONLY) {
#pragma unroll
            for (int c = 0; c < CBLK; c++)
#pragma unroll
              for (int v = 0; v < 16; v++) acc[c][v] *= sc;
          }
          lsum = pairs(m_run - m_old);
        }
      }
      l_s += lsum;
      if constexpr (!MASS_ONLY) {
        // value operands: fp16((code - z) Delta) of positions 16 ks + 8 h .. + 7 (token
        // pairs (j, j + 8), j = 4 h .. 4 h + 3, of 16-token group 2 mb + ks)
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          const int g = 2 * mb + ks;
          const uint4 z4 = *reinterpret_cast<const uint4*>(&sm.zv[8 * g + 4 * h]);
          const uint4 d4 = *reinterpret_cast<const uint4*>(&sm.dv[8 * g + 4 * h]);
          const uint32_t zz[4] = {z4.x, z4.y, z4.z, z4.w}, dd[4] = {d4.x, d4.y, d4.z, d4.w};
          f16x8 vop[CBLK];
#pragma unroll
          for (int c = 0; c < CBLK; c++) {
            uint32_t t;
            if constexpr (BITS == 2) {
              t = cur.v[c][g];  // pair i: bits 8 h + 2 i (one shift, one and-or per pair)
            } else {
              const uint32_t w0 = cur.v[c][2 * g], w1 = cur.v[c][2 * g + 1];
              t = h ? ((w0 >> 16) | (w1 & 0xFFFF0000u)) : ((w0 & 0xFFFFu) | (w1 << 16));
            }
            uint32_t res[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const uint32_t a = BITS == 2 ? (((t >> vsh[i]) & vmask) | 0x64006400u)
                                           : (((t >> (4 * i)) & vmask) | 0x64006400u);
              const f16x2 cz = __builtin_bit_cast(f16x2, a) + __builtin_bit_cast(f16x2, zz[i]);
              res[i] = __builtin_bit_cast(uint32_t, cz * __builtin_bit_cast(f16x2, dd[i]));
            }
            vop[c] = __builtin_bit_cast(f16x8, make_uint4(res[0], res[1], res[2], res[3]));
          }
          const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(pb[ks][0], pb[ks][1], pb[ks][2], pb[ks][3]));
#pragma unroll
          for (int c = 0; c < CBLK; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop[c], bop, acc[c], 0, 0, 0);
        }
      }
    }
  }

  // ---- un-rotate the value sum (as the main kernel) and write the share's partial record
  if constexpr (!MASS_ONLY) {
    if (p.v_had) {
#pragma unroll
      for (int bit = 0; bit < 4; bit++)
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
      for (int c = 0; c < CBLK; c++)
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const float pvv = xor32(acc[c][v]);
          acc[c][v] = h ? (pvv - acc[c][v]) : (acc[c][v] + pvv);
        }
#pragma unroll
      for (int cbk = 1; cbk < CBLK; cbk <<= 1)
#pragma unroll
        for (int c = 0; c < CBLK; c++)
          if ((c & cbk) == 0)
#pragma unroll
            for (int v = 0; v < 16; v++) {
              const float a = acc[c][v], b = acc[c | cbk][v];
              acc[c][v] = a + b;
              acc[c | cbk][v] = a - b;
            }
      const float cn = rsqrtf((float)D);
#pragma unroll
      for (int c = 0; c < CBLK; c++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[c][v] *= cn;
      if (p.v_sg[0] | p.v_sg[1] | p.v_sg[2] | p.v_sg[3]) {
#pragma unroll
        for (int c = 0; c < CBLK; c++) {
          const uint32_t wv = p.v_sg[c] >> (4 * h);
#pragma unroll
          for (int v = 0; v < 16; v++)
            acc[c][v] = __uint_as_float(__float_as_uint(acc[c][v]) ^ (((wv >> ((v & 3) + 8 * (v >> 2))) & 1u) << 31));
        }
      }
    }
  }
  const float ls = l_s + xor32(l_s);
  if (!q_ok) return;
  float* rec = p.part + (((size_t)sp * p.B * p.H + bh) * p.n_q + qi) * (D + 4);
  if constexpr (!MASS_ONLY) {
#pragma unroll
    for (int c = 0; c < CBLK; c++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++)
        *reinterpret_cast<float4*>(rec + 32 * c + 8 * v4 + 4 * h) =
            make_float4(acc[c][4 * v4], acc[c][4 * v4 + 1], acc[c][4 * v4 + 2], acc[c][4 * v4 + 3]);
  }
  if (h == 0) *reinterpret_cast<float4*>(rec + D) = make_float4(m_run, ls, 0.f, 0.f);
}

// Combines the partial records of the n_split shares of each query: with M the largest
// reference max, weights w = 2^(m - M); O = sum w acc / sum w (l_S + l_R), and the
// masses from the weighted sums. One thread per (query, 4 output channels); G threads
// per query (G = 1 for masses only).
template <int D, int G, bool MASS_ONLY>
__global__ __launch_bounds__(256) void jb_combine_kernel(const float* __restrict__ part, int n_split, size_t rows,
                                                         float* __restrict__ o, float* __restrict__ mass_s,
                                                         float* __restrict__ mass_r) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = t / G;
  const int cg = (int)(t % G);
  if (row >= rows) return;
  const size_t stride = rows * (D + 4);
  const float* rec0 = part + row * (D + 4);
  float M = -INFINITY;
  for (int sp = 0; sp < n_split; sp++) M = fmaxf(M, rec0[sp * stride + D]);
  float ls = 0.f, lr = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = 0; sp < n_split; sp++) {
    const float* rec = rec0 + sp * stride;
    const float4 st = *reinterpret_cast<const float4*>(rec + D);
    const float w = exp2f(st.x - M);
    ls = fmaf(w, st.y, ls);
    lr = fmaf(w, st.z, lr);
    if constexpr (!MASS_ONLY) {
      const float4 v = *reinterpret_cast<const float4*>(rec + 4 * cg);
      a.x = fmaf(w, v.x, a.x);
      a.y = fmaf(w, v.y, a.y);
      a.z = fmaf(w, v.z, a.z);
      a.w = fmaf(w, v.w, a.w);
    }
  }
  const float inv = 1.f / (ls + lr);
  if constexpr (!MASS_ONLY)
    *reinterpret_cast<float4*>(o + row * D + 4 * cg) = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
  if (cg == 0 && mass_s) {
    mass_s[row] = ls * inv;
    mass_r[row] = lr * inv;
  }
}

// The same merge for many records per query (the few-query path: one record per share of
// the window, tens of shares): one workgroup per query, its threads split over channel
// groups (G of 4 channels) and record slices (R = 256 / G, records r, r + R, ...). Each
// thread merges its slice against the slice's own largest reference max; the slices are
// then combined through LDS against the largest of all.
template <int D, bool MASS_ONLY>
__global__ __launch_bounds__(256) void jb_merge_records_kernel(const float* __restrict__ part, int n_rec, size_t rows,
                                                               float* __restrict__ o, float* __restrict__ mass_s,
                                                               float* __restrict__ mass_r) {
  constexpr int G = D / 4, R = 256 / G;
  __shared__ float4 sa[R][G];
  __shared__ float sm_m[R], sm_s[R], sm_r[R];
  const size_t row = blockIdx.x;
  const int cg = threadIdx.x % G, r = threadIdx.x / G;
  const size_t stride = rows * (D + 4);
  const float* rec0 = part + row * (D + 4);
  float M = -INFINITY;
  for (int sp = r; sp < n_rec; sp += R) M = fmaxf(M, rec0[sp * stride + D]);
  float ls = 0.f, lr = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = r; sp < n_rec; sp += R) {
    const float* rec = rec0 + sp * stride;
    const float4 st = *reinterpret_cast<const float4*>(rec + D);
    const float w = exp2f(st.x - M);
    ls = fmaf(w, st.y, ls);
    lr = fmaf(w, st.z, lr);
    if constexpr (!MASS_ONLY) {
      const float4 v = *reinterpret_cast<const float4*>(rec + 4 * cg);
      a.x = fmaf(w, v.x, a.x);
      a.y = fmaf(w, v.y, a.y);
      a.z = fmaf(w, v.z, a.z);
      a.w = fmaf(w, v.w, a.w);
    }
  }
  sa[r][cg] = a;
  if (cg == 0) {
    sm_m[r] = M;
    sm_s[r] = ls;
    sm_r[r] = lr;
  }
  __syncthreads();
  if (r != 0) return;
  float Mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < R; i++) Mx = fmaxf(Mx, sm_m[i]);
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
  float ts = 0.f, tr = 0.f;
#pragma unroll
  for (int i = 0; i < R; i++) {
    if (sm_m[i] == -INFINITY) continue;  // a slice without records
    const float f = exp2f(sm_m[i] - Mx);
    ts = fmaf(f, sm_s[i], ts);
    tr = fmaf(f, sm_r[i], tr);
    const float4 v = sa[i][cg];
    t.x = fmaf(f, v.x, t.x);
    t.y = fmaf(f, v.y, t.y);
    t.z = fmaf(f, v.z, t.z);
    t.w = fmaf(f, v.w, t.w);
  }
  const float inv = 1.f / (ts + tr);
  if constexpr (!MASS_ONLY)
    *reinterpret_cast<float4*>(o + row * D + 4 * cg) = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  if (cg == 0 && mass_s) {
    mass_s[row] = ts * inv;
    mass_r[row] = tr * inv;
  }
}

// Compute units of the current device (0 if it cannot be queried: no split, no decode path).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1) {
    (void)hipGetLastError();
    return 0;
  }
  return cus;
}

// Kernel parameters of one call under plan pl (split partials in the call's workspace).
template <int D, bool MASS_ONLY, bool PERCH>
Params fill_params(const jb_attn_args* a, const AttnPlan& pl) {
  Params p;
  p.B = a->B;
  p.H = a->H;
  p.n_q = a->n_q;
  p.n_r = a->n_r;
  p.chunk_len = a->chunk_len;
  p.n_chunks = a->n_chunks;
  p.n_wchunks = a->window_chunks > 0 ? a->window_chunks : a->n_chunks;
  p.cp = chunk_pad(a->chunk_len);
  p.n_qblk = pl.n_qblk;
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
  for (int i = 0; i < 4; i++) {
    p.k_sg[i] = a->k_fmt.signs[i];
    p.v_sg[i] = a->v_fmt.signs[i];
  }
  p.k_group = PERCH ? a->k_fmt.group : 0;
  // workspace: the split partials (16-byte aligned)
  p.n_split = pl.n_split;
  p.part = pl.n_split > 1 ? static_cast<float*>(a->workspace) : nullptr;
  p.o = MASS_ONLY ? nullptr : a->o;
  p.mass_s = a->mass_s;
  p.mass_r = a->mass_r;
  return p;
}

template <int D, int BITS, bool MASS_ONLY, bool PERCH, bool EXACT = false, int TG = 0>
int launch_attn(const jb_attn_args* a, const AttnPlan& pl, hipStream_t st) {
  const Params p = fill_params<D, MASS_ONLY, PERCH>(a, pl);
  const unsigned grid = (unsigned)(pl.n_qblk * a->B * a->H * pl.n_split);
  jb_attn_kernel<D, BITS, MASS_ONLY, PERCH, EXACT, TG><<<grid, kThreads, 0, st>>>(p);
  if (pl.n_split > 1) {
    const size_t rows = (size_t)a->B * a->H * a->n_q;
    constexpr int G = MASS_ONLY ? 1 : D / 4;
    const unsigned cgrid = (unsigned)((rows * G + 255) / 256);
    jb_combine_kernel<D, G, MASS_ONLY><<<cgrid, 256, 0, st>>>(p.part, pl.n_split, rows, p.o, p.mass_s, p.mass_r);
  }
  return launch_status();
}

// Few queries: the decode kernel over the cached window (one partial record per share)
// and, in the same grid, over the current chunk (one more record per query), then the merge.
template <int D, int BITS, bool MASS_ONLY>
int launch_decode(const jb_attn_args* a, const AttnPlan& pl0, hipStream_t st) {
  AttnPlan pl = pl0;
  pl.n_split = 1;
  pl.part_bytes = 0;
  Params p = fill_params<D, MASS_ONLY, false>(a, pl);
  const int S = pl.dec_shares;
  const size_t rows = (size_t)a->B * a->H * a->n_q;
  float* part = static_cast<float*>(a->workspace);
  p.part = part;
  const int n_rec = S + (a->n_r > 0 ? 1 : 0);  // the window's shares, then the current chunk
  jb_decode_kernel<D, BITS, MASS_ONLY><<<(unsigned)(n_rec * a->B * a->H), 64, 0, st>>>(p, S);
  jb_merge_records_kernel<D, MASS_ONLY><<<(unsigned)rows, 256, 0, st>>>(part, n_rec, rows, p.o, p.mass_s, p.mass_r);
  return launch_status();
}

// A call with a workspace runs the plan (decode path, or split when the grid is small for
// the device); one without runs the main kernel unsplit. A workspace smaller than the plan
// needs is an error.
template <bool MASS_ONLY>
int dispatch(const jb_attn_args* a, void* stream) {
  const int st = validate_attn(a, MASS_ONLY);
  if (st) return st;
  AttnPlan pl = plan_attn(a, device_cus());
  const size_t need = plan_workspace(pl);
  if (a->workspace) {
    if (a->workspace_bytes < need) return KVQ_ERR_WORKSPACE;
    if (need && !aligned16(a->workspace)) return KVQ_ERR_ALIGN;
  } else {
    pl.dec_shares = 0;
    pl.n_split = 1;
    pl.part_bytes = 0;
  }
  if (pl.dec_shares) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (a->d == 128)
      return a->k_fmt.bits == 2 ? launch_decode<128, 2, MASS_ONLY>(a, pl, s) : launch_decode<128, 4, MASS_ONLY>(a, pl, s);
    return a->k_fmt.bits == 2 ? launch_decode<64, 2, MASS_ONLY>(a, pl, s) : launch_decode<64, 4, MASS_ONLY>(a, pl, s);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool perch = a->k_fmt.granularity == KVQ_PER_CHANNEL;
  if (a->k_fmt.granularity == KVQ_PER_TOKEN_GROUP && a->correction == JB_CORR_EXACT && a->n_chunks > 0) {
    const bool i2 = a->k_fmt.bits == 2;
    if (a->d == 64)
      return i2 ? launch_attn<64, 2, MASS_ONLY, false, true, 32>(a, pl, s)
                : launch_attn<64, 4, MASS_ONLY, false, true, 32>(a, pl, s);
    if (a->k_fmt.group == 32)
      return i2 ? launch_attn<128, 2, MASS_ONLY, false, true, 32>(a, pl, s)
                : launch_attn<128, 4, MASS_ONLY, false, true, 32>(a, pl, s);
    return i2 ? launch_attn<128, 2, MASS_ONLY, false, true, 64>(a, pl, s)
              : launch_attn<128, 4, MASS_ONLY, false, true, 64>(a, pl, s);
  }
  if (a->k_fmt.granularity == KVQ_PER_TOKEN_GROUP) {
    const bool i2 = a->k_fmt.bits == 2;
    if (a->d == 64)
      return i2 ? launch_attn<64, 2, MASS_ONLY, false, false, 32>(a, pl, s)
                : launch_attn<64, 4, MASS_ONLY, false, false, 32>(a, pl, s);
    if (a->k_fmt.group == 32)
      return i2 ? launch_attn<128, 2, MASS_ONLY, false, false, 32>(a, pl, s)
                : launch_attn<128, 4, MASS_ONLY, false, false, 32>(a, pl, s);
    return i2 ? launch_attn<128, 2, MASS_ONLY, false, false, 64>(a, pl, s)
              : launch_attn<128, 4, MASS_ONLY, false, false, 64>(a, pl, s);
  }
  if (a->correction == JB_CORR_EXACT && a->n_chunks > 0) {
    if (a->d == 128) {
      if (a->k_fmt.bits == 2)
        return perch ? launch_attn<128, 2, MASS_ONLY, true, true>(a, pl, s)
                     : launch_attn<128, 2, MASS_ONLY, false, true>(a, pl, s);
      return perch ? launch_attn<128, 4, MASS_ONLY, true, true>(a, pl, s)
                   : launch_attn<128, 4, MASS_ONLY, false, true>(a, pl, s);
    }
    if (a->k_fmt.bits == 2)
      return perch ? launch_attn<64, 2, MASS_ONLY, true, true>(a, pl, s) : launch_attn<64, 2, MASS_ONLY, false, true>(a, pl, s);
    return perch ? launch_attn<64, 4, MASS_ONLY, true, true>(a, pl, s) : launch_attn<64, 4, MASS_ONLY, false, true>(a, pl, s);
  }
  if (a->d == 128) {
    if (a->k_fmt.bits == 2)
      return perch ? launch_attn<128, 2, MASS_ONLY, true>(a, pl, s) : launch_attn<128, 2, MASS_ONLY, false>(a, pl, s);
    return perch ? launch_attn<128, 4, MASS_ONLY, true>(a, pl, s) : launch_attn<128, 4, MASS_ONLY, false>(a, pl, s);
  }
  if (a->k_fmt.bits == 2)
    return perch ? launch_attn<64, 2, MASS_ONLY, true>(a, pl, s) : launch_attn<64, 2, MASS_ONLY, false>(a, pl, s);
  return perch ? launch_attn<64, 4, MASS_ONLY, true>(a, pl, s) : launch_attn<64, 4, MASS_ONLY, false>(a, pl, s);
}

template <int D, int BITS, bool MASS_ONLY, bool PERCH, bool EXACT, int TG = 0>
int launch_batch(const jb_attn_args* calls, int n, hipStream_t st) {
  // One split count S for the whole batch, chosen as for a single call but over the
  // workgroups of all calls: rounds of the device times the longest share. It is used
  // only when every call's workspace holds its S partials.
  const int S = batch_split(calls, n, device_cus());
  AttnPlan pl[kMaxBatch];
  BatchParams bp;
  bp.n = n;
  long long next = 0;
  for (int c = 0; c < n; c++) {
    const jb_attn_args* a = &calls[c];
    pl[c] = plan_attn(a, 0);
    pl[c].n_split = S;
    pl[c].part_bytes = S > 1 ? partial_bytes(a, S) : 0;
    bp.p[c] = fill_params<D, MASS_ONLY, PERCH>(a, pl[c]);
    bp.grid[c] = (int)(pl[c].n_qblk * a->B * a->H * S);
    bp.start[c] = (int)next;
    next += ((long long)bp.grid[c] + 7) / 8 * 8;
    if (next > 0x7FFFFFFFLL) return KVQ_ERR_SHAPE;
  }
  jb_attn_batch_kernel<D, BITS, MASS_ONLY, PERCH, EXACT, TG><<<(unsigned)next, kThreads, 0, st>>>(bp);
  if (S > 1) {
    constexpr int G = MASS_ONLY ? 1 : D / 4;
    for (int c = 0; c < n; c++) {
      const size_t rows = (size_t)calls[c].B * calls[c].H * calls[c].n_q;
      jb_combine_kernel<D, G, MASS_ONLY><<<(unsigned)((rows * G + 255) / 256), 256, 0, st>>>(
          bp.p[c].part, S, rows, bp.p[c].o, bp.p[c].mass_s, bp.p[c].mass_r);
    }
  }
  return launch_status();
}

template <bool MASS_ONLY>
int dispatch_batch(const jb_attn_args* calls, int n, void* stream) {
  const int st = validate_batch(calls, n, MASS_ONLY);
  if (st) return st;
  const jb_attn_args& a0 = calls[0];
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool perch = a0.k_fmt.granularity == KVQ_PER_CHANNEL;
  const bool exact = a0.correction == JB_CORR_EXACT;
  if (a0.k_fmt.granularity == KVQ_PER_TOKEN_GROUP) {
    // group-wise keys and values: one group size for the batch (checked by validate_batch)
    const bool i2 = a0.k_fmt.bits == 2;
#define KVQ_TG_BATCH(EX)                                                                                  \
  if (a0.d == 64)                                                                                         \
    return i2 ? launch_batch<64, 2, MASS_ONLY, false, EX, 32>(calls, n, s)                                \
              : launch_batch<64, 4, MASS_ONLY, false, EX, 32>(calls, n, s);                               \
  if (a0.k_fmt.group == 32)                                                                               \
    return i2 ? launch_batch<128, 2, MASS_ONLY, false, EX, 32>(calls, n, s)                               \
              : launch_batch<128, 4, MASS_ONLY, false, EX, 32>(calls, n, s);                              \
  return i2 ? launch_batch<128, 2, MASS_ONLY, false, EX, 64>(calls, n, s)                                 \
            : launch_batch<128, 4, MASS_ONLY, false, EX, 64>(calls, n, s);
    if (exact) {
      KVQ_TG_BATCH(true)
    }
    KVQ_TG_BATCH(false)
#undef KVQ_TG_BATCH
  }
#define KVQ_BATCH_CASE(D_, B_)                                                                             \
  if (a0.d == D_ && a0.k_fmt.bits == B_) {                                                                 \
    if (perch)                                                                                             \
      return exact ? launch_batch<D_, B_, MASS_ONLY, true, true>(calls, n, s)                              \
                   : launch_batch<D_, B_, MASS_ONLY, true, false>(calls, n, s);                            \
    return exact ? launch_batch<D_, B_, MASS_ONLY, false, true>(calls, n, s)                               \
                 : launch_batch<D_, B_, MASS_ONLY, false, false>(calls, n, s);                             \
  }
  KVQ_BATCH_CASE(128, 2)
  KVQ_BATCH_CASE(128, 4)
  KVQ_BATCH_CASE(64, 2)
  KVQ_BATCH_CASE(64, 4)
#undef KVQ_BATCH_CASE
  return KVQ_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace kvq

extern "C" int jb_attn_fwd_batch(const jb_attn_args* calls, int32_t n_calls, void* stream) {
  return kvq::dispatch_batch<false>(calls, n_calls, stream);
}

extern "C" int jb_attn_mass_batch(const jb_attn_args* calls, int32_t n_calls, void* stream) {
  return kvq::dispatch_batch<true>(calls, n_calls, stream);
}

extern "C" int jb_attn_fwd(const jb_attn_args* a, void* stream) { return kvq::dispatch<false>(a, stream); }

extern "C" int jb_attn_mass(const jb_attn_args* a, void* stream) { return kvq::dispatch<true>(a, stream); }

extern "C" size_t jb_attn_workspace_bytes(const jb_attn_args* a) {
  if (kvq::validate_attn(a, false) != KVQ_OK && kvq::validate_attn(a, true) != KVQ_OK) return SIZE_MAX;
  return kvq::plan_workspace(kvq::plan_attn(a, kvq::device_cus()));
}

// ---------------- the forward pass without allocation ----------------
// For callers that cannot allocate device memory (code under graph capture, serving loops
// that forbid it): the split partials or few-query records go to a fixed array in device
// memory, one copy per device, which the library holds until the process ends.
static __device__ __align__(256) unsigned char scratch[JB_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch` (looked up on the first call on that device;
// the array's name is a host-side stand-in, never passed to a kernel).
int scratch_on_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return KVQ_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return KVQ_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}
}  // namespace

extern "C" int jb_attn_fwd_noalloc(const jb_attn_args* a, void* stream) {
  const int st = kvq::validate_attn(a, false);
  if (st) return st;
  const size_t need = kvq::plan_workspace(kvq::plan_attn(a, kvq::device_cus()));
  if (need > (size_t)JB_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
  jb_attn_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (need > 0) {
    void* ptr = nullptr;
    const int s2 = scratch_on_device(&ptr);
    if (s2) return s2;
    b.workspace = ptr;
    b.workspace_bytes = JB_NOALLOC_SCRATCH_BYTES;
  }
  return kvq::dispatch<false>(&b, stream);
}
