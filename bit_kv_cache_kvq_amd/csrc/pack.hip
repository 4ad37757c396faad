// kvq_pack: compress one chunk of keys or values into the cache format.
//
// Paper: "Quantized Keys Steal Attention" (arXiv 2605.26266), §3 -- Hadamard rotation,
// asymmetric round-to-nearest integer quantization (Eq. (1)) and its granularities
// (per token; per group of channels of a token; per channel over a group of tokens for
// keys). The exact float32 operation
// order is the one stated in include/kvq.h at kvq_format; it makes codes, steps and zero
// points reproducible bit for bit. This translation unit is built with -ffp-contract=off
// and correctly rounded float32 division.
//
// Work mapping (HBM-bound streaming kernel): one workgroup per 64-token block of the
// padded chunk (per token) or per channel group (per channel). Each token is held by
// D/16 consecutive lanes, 16 channels per lane: four butterfly stages run inside a lane,
// the remaining log2(D/16) across lanes with xor shuffles, in the contract's order.
#include "common.h"

namespace kvq {
namespace {

// Channel signs of a randomized rotation (bit c of w[c / 32] set: channel c negated).
struct SignBits {
  uint32_t w[4];
};

template <int D>
__device__ inline void load_token16(const uint16_t* __restrict__ row, int lt, bool valid, const SignBits& sg,
                                    float (&y)[16]) {
  if (valid) {
    const uint4* p = reinterpret_cast<const uint4*>(row + 16 * lt);
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    // this lane's 16 sign bits, moved onto the bf16 sign bits (15, 31) of each channel pair
    const uint32_t m16 = (sg.w[lt >> 1] >> (16 * (lt & 1))) & 0xFFFFu;
#pragma unroll
    for (int i = 0; i < 8; i++) w[i] ^= (((m16 >> (2 * i)) & 1u) << 15) | (((m16 >> (2 * i + 1)) & 1u) << 31);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      y[2 * i] = __uint_as_float(w[i] << 16);
      y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) y[i] = 0.f;
  }
}

// y = H_D x over channels 16*lt + i held by the D/16 lanes of one token.
template <int D>
__device__ inline void fwht_rows(float (&y)[16], int lt) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if ((i & h) == 0) {
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int hl = 1; hl < D / 16; hl <<= 1) {
    const bool upper = (lt & hl) != 0;  // this lane holds the "i + h" side of each pair
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const float p = __shfl_xor(y[i], hl);
      y[i] = upper ? (p - y[i]) : (y[i] + p);
    }
  }
  const float c = (D == 64) ? 0.125f : 0.08838834764831845f;  // float32 nearest 1/sqrt(D)
#pragma unroll
  for (int i = 0; i < 16; i++) y[i] = y[i] * c;
}

struct QParams {
  float delta;  // 0 for a degenerate group
  float z;
  uint16_t scale_bits, zero_bits;
};

template <int BITS>
__device__ inline QParams make_params(float mn, float mx) {
  constexpr float qmax = float((1 << BITS) - 1);
  QParams p;
  const float d32 = (mx - mn) / qmax;
  const _Float16 dh = (_Float16)d32;
  p.delta = (float)dh;
  if (p.delta == 0.f) {
    p.z = 0.f;
    p.scale_bits = 0;
    p.zero_bits = 0;
  } else {
    p.z = __builtin_rintf(-mn / p.delta) + 0.0f;
    p.scale_bits = __builtin_bit_cast(uint16_t, dh);
    p.zero_bits = __builtin_bit_cast(uint16_t, (_Float16)p.z);
  }
  return p;
}

template <int BITS>
__device__ inline uint32_t code_of(float y, float delta, float z) {
  constexpr float qmax = float((1 << BITS) - 1);
  if (delta == 0.f) return 0u;
  const float c = __builtin_rintf(y / delta) + z;
  return (uint32_t)fminf(fmaxf(c, 0.f), qmax);
}

template <int D, int BITS>
__device__ inline void store_key_words(uint32_t* __restrict__ dst_token, int lt, const uint32_t (&c)[16]) {
  if (BITS == 2) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) w |= c[i] << (2 * i);
    dst_token[lt] = w;
  } else {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      w0 |= c[i] << (4 * i);
      w1 |= c[8 + i] << (4 * i);
    }
    reinterpret_cast<uint2*>(dst_token)[lt] = make_uint2(w0, w1);
  }
}

// Per-token quantization of one 64-token block of the padded chunk; with CG < D, each
// token's channels form groups of CG (group-wise per token), one (Delta, z) pair each.
template <int D, int BITS, int ROLE, int CG = D>
__global__ __launch_bounds__(64 * D / 16) void pack_token_kernel(
    const uint16_t* __restrict__ x, int n, int n_chunks, int chunk_idx, int hadamard, const SignBits sg,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale, uint16_t* __restrict__ zero) {
  constexpr int LPT = D / 16;            // lanes per token
  constexpr int LPG = CG / 16;           // lanes per channel group
  constexpr int NG = D / CG;             // (Delta, z) pairs per token
  constexpr int CPW = 32 / BITS;         // codes per word
  const int tid = threadIdx.x;
  const int tl = tid / LPT, lt = tid % LPT;
  const int blk = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int cp = chunk_pad(n);
  const int t = blk * kTokenBlock + tl;  // token within the chunk
  const bool valid = t < n;
  const size_t n_tot = (size_t)n_chunks * cp;

  float y[16];
  load_token16<D>(x + (bh * n + (valid ? t : 0)) * D, lt, valid, sg, y);
  if (hadamard) fwht_rows<D>(y, lt);

  float mn = y[0], mx = y[0];
#pragma unroll
  for (int i = 1; i < 16; i++) {
    mn = fminf(mn, y[i]);
    mx = fmaxf(mx, y[i]);
  }
#pragma unroll
  for (int hl = 1; hl < LPG; hl <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, hl));
    mx = fmaxf(mx, __shfl_xor(mx, hl));
  }
  const QParams qp = make_params<BITS>(mn, mx);
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 16; i++) c[i] = valid ? code_of<BITS>(y[i], qp.delta, qp.z) : 0u;

  const size_t tok_w = (size_t)chunk_idx * cp + t;
  if (lt % LPG == 0) {
    const size_t at = (bh * n_tot + tok_w) * NG + lt / LPG;
    scale[at] = valid ? qp.scale_bits : (uint16_t)0;
    zero[at] = valid ? qp.zero_bits : (uint16_t)0;
  }
  if (ROLE == KVQ_ROLE_KEY) {
    store_key_words<D, BITS>(codes + (bh * n_tot + tok_w) * (D / CPW), lt, c);
  } else {
    __shared__ uint8_t s_codes[kTokenBlock][D];
#pragma unroll
    for (int i = 0; i < 16; i++) s_codes[tl][16 * lt + i] = (uint8_t)c[i];
    __syncthreads();
    constexpr int WPC = kTokenBlock / CPW;  // words per channel per block
    constexpr int NW = D * WPC;
    const size_t blk_w = (size_t)chunk_idx * (cp / kTokenBlock) + blk;
    uint32_t* dst = codes + (bh * (n_tot / kTokenBlock) + blk_w) * NW;
    for (int widx = tid; widx < NW; widx += blockDim.x) {
      const int ch = widx / WPC, u = widx % WPC;
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < CPW; i++) w |= (uint32_t)s_codes[CPW * u + i][ch] << (BITS * i);
      dst[widx] = w;
    }
  }
}

// Per-channel key quantization: one workgroup per group of GROUP tokens of the chunk.
template <int D, int BITS, int GROUP>
__global__ __launch_bounds__(GROUP * D / 16) void pack_channel_kernel(
    const uint16_t* __restrict__ x, int n, int n_chunks, int chunk_idx, int hadamard, const SignBits sg,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale, uint16_t* __restrict__ zero) {
  constexpr int LPT = D / 16;
  constexpr int CPW = 32 / BITS;
  __shared__ float s_y[GROUP][D];
  __shared__ float s_delta[D], s_z[D];
  const int tid = threadIdx.x;
  const int tl = tid / LPT, lt = tid % LPT;
  const int g = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int cp = chunk_pad(n);
  const int G = (n + GROUP - 1) / GROUP;
  const int t0 = g * GROUP;
  const int t = t0 + tl;
  const bool valid = t < n;
  const int n_valid = min(GROUP, n - t0);

  float y[16];
  load_token16<D>(x + (bh * n + (valid ? t : 0)) * D, lt, valid, sg, y);
  if (hadamard) fwht_rows<D>(y, lt);
#pragma unroll
  for (int i = 0; i < 16; i++) s_y[tl][16 * lt + i] = y[i];
  __syncthreads();
  if (tid < D) {
    float mn = s_y[0][tid], mx = s_y[0][tid];
    for (int k = 1; k < n_valid; k++) {
      mn = fminf(mn, s_y[k][tid]);
      mx = fmaxf(mx, s_y[k][tid]);
    }
    const QParams qp = make_params<BITS>(mn, mx);
    s_delta[tid] = qp.delta;
    s_z[tid] = qp.z;
    const size_t row = bh * ((size_t)n_chunks * G) + (size_t)chunk_idx * G + g;
    scale[row * D + tid] = qp.scale_bits;
    zero[row * D + tid] = qp.zero_bits;
  }
  __syncthreads();
  if (t < cp) {
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int ch = 16 * lt + i;
      c[i] = valid ? code_of<BITS>(y[i], s_delta[ch], s_z[ch]) : 0u;
    }
    const size_t n_tot = (size_t)n_chunks * cp;
    const size_t tok_w = (size_t)chunk_idx * cp + t;
    store_key_words<D, BITS>(codes + (bh * n_tot + tok_w) * (D / CPW), lt, c);
  }
}

template <int D, int BITS>
int launch_pack(const uint16_t* x, int B, int H, int n, const kvq_format* f, int n_chunks, int chunk_idx,
                uint32_t* codes, uint16_t* scale, uint16_t* zero, hipStream_t st) {
  const dim3 bh(1, (unsigned)(B * H));
  const SignBits sg = {{f->signs[0], f->signs[1], f->signs[2], f->signs[3]}};
  if (f->granularity == KVQ_PER_TOKEN_GROUP) {
    const dim3 grid((unsigned)(chunk_pad(n) / kTokenBlock), (unsigned)(B * H));
    constexpr int T = 64 * D / 16;
    if (f->role == KVQ_ROLE_KEY) {
      if (f->group == 32)
        pack_token_kernel<D, BITS, KVQ_ROLE_KEY, 32><<<grid, T, 0, st>>>(x, n, n_chunks, chunk_idx, f->hadamard, sg,
                                                                         codes, scale, zero);
      else
        pack_token_kernel<D, BITS, KVQ_ROLE_KEY, 64><<<grid, T, 0, st>>>(x, n, n_chunks, chunk_idx, f->hadamard, sg,
                                                                         codes, scale, zero);
    } else {
      if (f->group == 32)
        pack_token_kernel<D, BITS, KVQ_ROLE_VALUE, 32><<<grid, T, 0, st>>>(x, n, n_chunks, chunk_idx, f->hadamard,
                                                                           sg, codes, scale, zero);
      else
        pack_token_kernel<D, BITS, KVQ_ROLE_VALUE, 64><<<grid, T, 0, st>>>(x, n, n_chunks, chunk_idx, f->hadamard,
                                                                           sg, codes, scale, zero);
    }
  } else if (f->granularity == KVQ_PER_TOKEN) {
    const dim3 grid((unsigned)(chunk_pad(n) / kTokenBlock), (unsigned)(B * H));
    if (f->role == KVQ_ROLE_KEY)
      pack_token_kernel<D, BITS, KVQ_ROLE_KEY><<<grid, 64 * D / 16, 0, st>>>(x, n, n_chunks, chunk_idx, f->hadamard,
                                                                             sg, codes, scale, zero);
    else
      pack_token_kernel<D, BITS, KVQ_ROLE_VALUE><<<grid, 64 * D / 16, 0, st>>>(x, n, n_chunks, chunk_idx,
                                                                               f->hadamard, sg, codes, scale, zero);
  } else {
    const dim3 grid((unsigned)((n + f->group - 1) / f->group), (unsigned)(B * H));
    if (f->group == 64)
      pack_channel_kernel<D, BITS, 64><<<grid, 64 * D / 16, 0, st>>>(x, n, n_chunks, chunk_idx, f->hadamard, sg,
                                                                     codes, scale, zero);
    else
      pack_channel_kernel<D, BITS, 128><<<grid, 128 * D / 16, 0, st>>>(x, n, n_chunks, chunk_idx, f->hadamard,
                                                                       sg, codes, scale, zero);
  }
  (void)bh;
  return launch_status();
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" int kvq_pack(const uint16_t* x, int32_t B, int32_t H, int32_t n, int32_t d, const kvq_format* fmt,
                        int32_t n_chunks, int32_t chunk_idx, uint32_t* codes, uint16_t* scale, uint16_t* zero,
                        void* stream) {
  const int st = validate_pack(x, B, H, n, d, fmt, n_chunks, chunk_idx, codes, scale, zero);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d == 128)
    return fmt->bits == 2 ? launch_pack<128, 2>(x, B, H, n, fmt, n_chunks, chunk_idx, codes, scale, zero, s)
                          : launch_pack<128, 4>(x, B, H, n, fmt, n_chunks, chunk_idx, codes, scale, zero, s);
  return fmt->bits == 2 ? launch_pack<64, 2>(x, B, H, n, fmt, n_chunks, chunk_idx, codes, scale, zero, s)
                        : launch_pack<64, 4>(x, B, H, n, fmt, n_chunks, chunk_idx, codes, scale, zero, s);
}
