/* kvq.h -- C ABI of libkvq: Jensen-bias-corrected chunk attention over an INT2/INT4
 * quantized KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow "Quantized Keys Steal Attention: Bias Correction for KV-Cache
 * Compression in Video Diffusion" (Tuncer, Becker, Pfeil; arXiv 2605.26266):
 *   - kvq_pack: the cache compression of §3 -- Hadamard rotation ("Hadamard rotation"),
 *     asymmetric round-to-nearest integer quantization (Eq. (1)) per token or, for keys,
 *     per channel over a group of tokens, or per group of channels of a token
 *     ("Quantization granularity");
 *   - jb_attn_fwd: chunk-wise attention of the current chunk's queries over the cached
 *     window and the unquantized current chunk (abstract; §1), with the per-score
 *     correction b subtracted from cached-key scores before the softmax (abstract; Fig. 3
 *     caption), computed on the fly from the cached keys' step sizes and the query, with
 *     no extra memory; optionally the cached/current attention masses P_S, P_R (Fig. 2);
 *   - jb_attn_mass: the masses alone.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library never
 *     allocates, frees or keeps them. Layouts are dense row-major; every pointer must be
 *     16-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream) and is asynchronous to the host.
 *   - Arguments are validated on the host first. On a negative status nothing was
 *     launched and no output was written. KVQ_ERR_HIP reports a failed launch.
 *   - No global mutable state: calls are reentrant; calls on different streams may run
 *     concurrently if their outputs do not overlap.
 *   - Preconditions that are NOT checked: inputs are finite; inputs and outputs do not
 *     alias; per group, (max - min)/(2^bits - 1) fits in fp16 (< 65504).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = -1,        /* a required pointer is NULL */
  KVQ_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  KVQ_ERR_UNSUPPORTED = -3, /* a format/option combination this library does not implement */
  KVQ_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  KVQ_ERR_WORKSPACE = -5,   /* a workspace smaller than the call needs (jb_attn_workspace_bytes) */
  KVQ_ERR_HIP = -6          /* the HIP launch failed */
};

enum { KVQ_PER_TOKEN = 0, KVQ_PER_CHANNEL = 1, KVQ_PER_TOKEN_GROUP = 2 };
enum { KVQ_ROLE_KEY = 0, KVQ_ROLE_VALUE = 1 };
enum { JB_CORR_NONE = 0, JB_CORR_TAYLOR = 1, JB_CORR_EXACT = 2 };

/* Storage format of one cached tensor.
 *
 * Window geometry: a window holds n_chunks chunks of chunk_len tokens. Each chunk's
 * token axis is padded to chunk_pad = kvq_chunk_pad(chunk_len) (a multiple of 64);
 * pad tokens hold code 0 and, per token, scale = zero = 0.
 *
 * Codes (c = 32/bits codes per 32-bit word):
 *   KVQ_ROLE_KEY   uint32 [B, H, n_chunks*chunk_pad, d/c]: token-major; channel c*w + i of
 *                  a token is in bits [bits*i, bits*i + bits) of its word w.
 *   KVQ_ROLE_VALUE uint32 [B, H, n_chunks*chunk_pad/64, d, 64/c]: 64-token blocks, channel-
 *                  major inside a block; word u of channel ch holds tokens c*u .. c*u+c-1 of
 *                  the block, token c*u + i in bits [bits*i, bits*i + bits).
 * Step size and zero point (fp16 bit patterns):
 *   KVQ_PER_TOKEN   [B, H, n_chunks*chunk_pad]
 *   KVQ_PER_TOKEN_GROUP [B, H, n_chunks*chunk_pad, d/group]: §3's group-wise per-token
 *                   granularity; pair j of a token covers channels [j*group, (j+1)*group)
 *                   of the stored (rotated) basis; pad tokens hold 0.
 *   KVQ_PER_CHANNEL [B, H, n_chunks*ceil(chunk_len/group), d]; groups restart at each
 *                   chunk's first token, the last group of a chunk may be short. Groups that
 *                   span the boundaries of the chunks a stream produced are had by packing
 *                   those chunks as one (chunk_len = their total, n_chunks = 1).
 *
 * Quantizer (paper §3, Eq. (1)), one fixed float32 operation order, so results are
 * reproducible bit for bit: y = H x in float32 (butterfly stages h = 1, 2, ..., d/2,
 * pair (i, i+h) -> (a+b, a-b), then one multiply by float32(1/sqrt(d))) when hadamard
 * is set, else y = x; per group mn = min y, mx = max y; d32 = (mx - mn)/(2^bits - 1)
 * (correctly rounded); Delta = fp16(d32) (nearest even); if Delta == 0 then scale =
 * zero = +0 and codes 0; else z = rint(-mn/Delta) + 0 (half-even, -0 -> +0, not
 * clamped); code = clamp(rint(y/Delta) + z, 0, 2^bits - 1); scale = Delta, zero = fp16(z)
 * (exact for |z| <= 2048). Reconstruction: x_hat' = (code - zero) * scale, x_hat = H x_hat'.
 *
 * Randomized rotation (§3 names QuaRot's randomized Hadamard rotation): with signs set,
 * the rotation is R = H diag(s), s_c = -1 where bit c % 32 of signs[c / 32] is set: those
 * channels are negated (exactly) before the butterflies, and x_hat = diag(s) H x_hat'.
 * Attention rotates the queries with the key format's R and un-rotates its output with
 * the value format's. All-zero signs give R = H. */
typedef struct {
  int32_t bits;        /* 2 or 4 */
  int32_t granularity; /* KVQ_PER_TOKEN, KVQ_PER_TOKEN_GROUP, or KVQ_PER_CHANNEL (role KEY only) */
  int32_t group;       /* KVQ_PER_CHANNEL: tokens per channel group, 64 or 128;
                          KVQ_PER_TOKEN_GROUP: channels per group, 32 or 64 (< d);
                          ignored for KVQ_PER_TOKEN */
  int32_t hadamard;    /* 1: rotate by the normalized Sylvester-Hadamard matrix first */
  int32_t role;        /* KVQ_ROLE_KEY or KVQ_ROLE_VALUE: selects the code layout */
  uint32_t signs[4];   /* channel sign mask of a randomized rotation (hadamard = 1 only;
                          bits at channels >= d must be 0); all zero: none */
} kvq_format;

/* Tokens per chunk after padding to a multiple of 64. */
int32_t kvq_chunk_pad(int32_t chunk_len);

/* Element counts of a window's arrays: *code_words (uint32) and *param_elems (fp16,
 * for scale and for zero each). Returns KVQ_OK or a negative status for a bad format. */
int kvq_window_elems(const kvq_format* fmt, int32_t B, int32_t H, int32_t d, int32_t chunk_len,
                     int32_t n_chunks, size_t* code_words, size_t* param_elems);

/* Quantize ONE chunk (paper §3: Hadamard rotation, Eq. (1), quantization granularity)
 * and write it as chunk `chunk_idx` of a window of `n_chunks` chunks of n tokens.
 *   x      bf16 [B, H, n, d], d in {64, 128}, n >= 1 (the chunk; chunk_len = n)
 *   codes, scale, zero  the window arrays described at kvq_format; only chunk
 *          chunk_idx's slice (its padded tokens, or its channel groups) is written.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE (B,H,n < 1; d not 64/128; chunk_idx outside
 * [0, n_chunks)), KVQ_ERR_UNSUPPORTED (bits, granularity/role/group combination, signs
 * without hadamard or past channel d),
 * KVQ_ERR_ALIGN, KVQ_ERR_HIP. */
int kvq_pack(const uint16_t* x, int32_t B, int32_t H, int32_t n, int32_t d, const kvq_format* fmt,
             int32_t n_chunks, int32_t chunk_idx, uint32_t* codes, uint16_t* scale, uint16_t* zero,
             void* stream);

/* Arguments of one attention call (abstract; §1; Fig. 2 and Fig. 3 captions).
 * Query i of the current chunk attends, with no mask, to every valid cached token j of
 * the window and every current-chunk token r:
 *   l_ij = s * q_i . k_hat_j - b_ij     b_ij = s^2 * sum_c q'_ic^2 Delta_jc^2 / 24
 *   l_ir = s * q_i . k_r                (current chunk: not quantized, no correction)
 *   O_i  = (sum_j e^l_ij v_hat_j + sum_r e^l_ir v_r) / sum e^l
 *   P_S,i = sum_j e^l_ij / sum e^l,  P_R,i = sum_r e^l_ir / sum e^l
 * where q' = H q if the keys were rotated (else q), Delta_jc is the key's step size
 * (per token: the same for every c, giving b_ij = s^2 |q_i|^2 Delta_j^2 / 24; group-wise
 * per token: the step of c's channel group, giving s^2 sum_groups |q'_i,grp|^2 Delta_j,grp^2 / 24), and
 * b is the second-order Taylor form of the expected inflation of e^l under uniform
 * rounding noise on the cached keys. b_ij = 0 when correction == JB_CORR_NONE.
 * JB_CORR_EXACT replaces b by the logarithm of that inflation itself (Fig. 3 caption's
 * model, an ablation of the second-order form):
 *   b_ij = sum_c log(sinh(x) / x),  x = s q'_ic Delta_jc / 2.
 * Per-channel keys evaluate it once per query and key group (relative error of each
 * channel's term below 1e-6). Per-token keys evaluate its power series in Delta_j through
 * Delta_j^8 (the omitted terms are below (max_c x)^8 sum_c x^2 / 467775 nats: 2e-6 per
 * channel at x = 1; the series does not converge past x = pi; its terms past the second
 * order are fp16 products (hi/lo pairs for the Delta^4 and Delta^6 terms) whose key-side
 * powers of Delta_j saturate from Delta_j = 32 on, where x passes pi for every channel
 * with s |q'_ic| > 0.2); group-wise
 * per-token keys the same series per channel group, in that group's step Delta_j,grp. */
typedef struct {
  int32_t B, H, d;            /* d in {64, 128}; the same H for queries and keys */
  int32_t n_q;                /* current-chunk queries, >= 1 */
  int32_t n_r;                /* current-chunk keys/values, >= 0 */
  int32_t chunk_len;          /* tokens per cached chunk, >= 1 */
  int32_t n_chunks;           /* cached chunks in the window, >= 0 */
  const uint16_t* q;          /* bf16 [B, H, n_q, d], not rotated */
  const uint16_t* k_cur;      /* bf16 [B, H, n_r, d] */
  const uint16_t* v_cur;      /* bf16 [B, H, n_r, d] */
  const uint32_t* k_codes;    /* window layout of k_fmt (role KEY) */
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint32_t* v_codes;    /* window layout of v_fmt (role VALUE) */
  const uint16_t* v_scale;
  const uint16_t* v_zero;
  kvq_format k_fmt, v_fmt;    /* same bits; k: KEY per token or per channel with v: VALUE per
                                 token; or both KVQ_PER_TOKEN_GROUP with one group (32 or
                                 64 < d) */
  float softmax_scale;        /* s; 0 selects 1/sqrt(d) */
  int32_t correction;         /* JB_CORR_NONE, JB_CORR_TAYLOR or JB_CORR_EXACT */
  float* o;                   /* fp32 [B, H, n_q, d]: required by fwd, ignored by mass */
  float* mass_s;              /* fp32 [B, H, n_q]: optional in fwd (NULL), required in mass */
  float* mass_r;              /* fp32 [B, H, n_q]: as mass_s */
  void* workspace;            /* device, 16-byte aligned, caller-owned; may be NULL (see below) */
  size_t workspace_bytes;     /* its size in bytes */
  int32_t window_chunks;      /* chunks per head the window arrays are laid out for (their
                                 stride), >= n_chunks; 0 means n_chunks. A sliding window
                                 kept as a ring of window_chunks slots (kvq_pack's n_chunks
                                 and chunk_idx) passes the slots in use as chunks 0 ..
                                 n_chunks - 1 in any order: the attention does not depend on
                                 the order of the cached tokens. */
} jb_attn_args;

/* Corrected attention forward: writes o and, if given, mass_s/mass_r.
 * Numerics: with per-token keys, and with group-wise keys of 64 channels under the
 * Taylor or no correction, cached-key scores take the rotated query as the sum of three
 * fp6 (e2m3) roundings (the query, then twice what is left), each with a power-of-two
 * scale per query and 32 channels, against the exact codes, summed in fp32 (4-bit keys
 * with at most 32 queries: the rotated query as a 16-bit fixed-point integer, one scale
 * per 32 queries, against the exact codes); with per-channel keys, the rotated query
 * times the key group's steps as a 16-bit fixed-point integer (one scale per 32 queries
 * and key group) against the exact codes; with group-wise keys of 32 channels, or
 * group-wise keys under the exact correction, fp16 keys fp16((code - z) Delta) against
 * the rotated query as fp16 hi + lo parts; softmax numerators are
 * fp16 (relative to a per-query reference max that is raised whenever a numerator could
 * leave the fp16 range), values fp16((code - z) Delta); sums and outputs fp32.
 * Preconditions on the data (not checked): key steps Delta < 2048 and |Delta z| < 65504
 * (per token); value zero points -2032 <= z <= 1024 (code - z is then formed exactly in
 * fp16) and |(code - z) Delta| < 65504; scaled logits |s q.k| and the correction below
 * 2^15 nats.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE (also when one head's cached codes exceed 2^31 - 1
 * bytes), KVQ_ERR_UNSUPPORTED (mixed bits, value per-channel, wrong roles, group not
 * 64/128, signs without hadamard or past channel d), KVQ_ERR_ALIGN (also a misaligned
 * workspace that a split would use), KVQ_ERR_WORKSPACE (a workspace was given but is
 * smaller than jb_attn_workspace_bytes reports), KVQ_ERR_HIP. */
int jb_attn_fwd(const jb_attn_args* a, void* stream);

/* Attention masses only (Fig. 2): writes mass_s and mass_r; o and values are not read. */
int jb_attn_mass(const jb_attn_args* a, void* stream);

/* Several attention calls in one launch (for example the same chunk step of several
 * layers, §1's chunk-wise generation, whose calls are independent): the workgroups of all
 * calls share the device, so calls that would each leave compute units idle fill it
 * together. The split over window shares (see jb_attn_workspace_bytes) is planned for
 * the batch as a whole, with one share count for every call, and taken only when each
 * call's workspace holds its partials for that count; otherwise
 * no call is split, and each computes exactly what jb_attn_fwd (jb_attn_mass) would for
 * it unsplit. Calls must agree on d, bits, key
 * granularity (and group, for per-channel and group-wise formats),
 * and on whether correction is JB_CORR_EXACT; shapes, windows,
 * rotation flags and signs, softmax scale and the other correction modes may differ.
 * calls points to n_calls host structs, 1 <= n_calls <= KVQ_BATCH_MAX.
 * Errors: the first failing call's jb_attn_fwd (jb_attn_mass) status, KVQ_ERR_NULL
 * (calls NULL), KVQ_ERR_SHAPE (n_calls out of range, too many workgroups in total),
 * KVQ_ERR_UNSUPPORTED (calls that disagree as above). */
#define KVQ_BATCH_MAX 8
int jb_attn_fwd_batch(const jb_attn_args* calls, int32_t n_calls, void* stream);
int jb_attn_mass_batch(const jb_attn_args* calls, int32_t n_calls, void* stream);

/* Few queries (n_q <= 32, per-token keys, correction other than exact): with a workspace of
 * the size jb_attn_workspace_bytes reports, the call streams each head's cached window in
 * one-wave shares (a decode-like regime: the window is read once per call rather than
 * once per 256-query block), computes the current chunk as one more share and merges the
 * shares' partial records; without a workspace (NULL), the main kernel runs unsplit. */

/* Workspace bytes a call with these arguments uses on the current device (0: none).
 * When the grid of query blocks is small for the device (fewer workgroups than its compute
 * units can take in whole rounds), the call splits each query block's tiles (cached
 * window, then current chunk) into up to 8 contiguous shares, one workgroup each, writes
 * one partial record per share and query (unnormalized sum, reference max, l_S, l_R:
 * fp32 [shares][B*H][n_q][d + 4]) into the workspace and combines them in a second kernel
 * on the same stream. A call given no workspace (NULL) runs unsplit on the main kernel;
 * the two differ by rounding only (each share takes its fp16 numerators relative to its
 * own reference max). A call given a workspace smaller than this size fails with
 * KVQ_ERR_WORKSPACE before anything is launched. The workspace must not be shared by calls
 * that may run concurrently. Returns 0 when the call needs no workspace on this device and
 * SIZE_MAX when the arguments are invalid (jb_attn_fwd would return a negative status). */
size_t jb_attn_workspace_bytes(const jb_attn_args* a);

/* The forward pass of jb_attn_fwd for callers that cannot allocate device memory (code under
 * graph capture, serving loops or harnesses that forbid allocation): it calls no allocator.
 * The split partials or few-query records that jb_attn_fwd keeps in the caller's workspace
 * go to a fixed array of JB_NOALLOC_SCRATCH_BYTES bytes in device memory instead, one per
 * device the library runs on, held until the process ends; a->workspace and
 * a->workspace_bytes are ignored. Results equal jb_attn_fwd's with a workspace of
 * jb_attn_workspace_bytes. Errors: those of jb_attn_fwd, and KVQ_ERR_WORKSPACE when the
 * call would need more than JB_NOALLOC_SCRATCH_BYTES (jb_attn_workspace_bytes reports the
 * need; nothing is launched). Every call on one device shares that device's array, and
 * nothing in it needs to start at zero (each call writes every record it reads): calls
 * that may overlap in time on one device (other streams or host threads) race on it and
 * must be serialized by the caller. */
#define JB_NOALLOC_SCRATCH_BYTES (64u << 20)
int jb_attn_fwd_noalloc(const jb_attn_args* a, void* stream);

/* Static description of a status code. */
const char* kvq_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
