// Host-side argument validation and launch planning of libkvq (plain C++, no HIP).
// The checks follow the contracts stated in include/kvq.h.
#include "host.h"

#include <math.h>

#include <algorithm>

namespace kvq {

int validate_format(const kvq_format* f) {
  if (!f) return KVQ_ERR_NULL;
  if (f->bits != 2 && f->bits != 4) return KVQ_ERR_UNSUPPORTED;
  if (f->hadamard != 0 && f->hadamard != 1) return KVQ_ERR_UNSUPPORTED;
  if (!f->hadamard && (f->signs[0] | f->signs[1] | f->signs[2] | f->signs[3])) return KVQ_ERR_UNSUPPORTED;
  if (f->role != KVQ_ROLE_KEY && f->role != KVQ_ROLE_VALUE) return KVQ_ERR_UNSUPPORTED;
  if (f->granularity == KVQ_PER_TOKEN) return KVQ_OK;
  if (f->granularity == KVQ_PER_TOKEN_GROUP) return f->group == 32 || f->group == 64 ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
  if (f->granularity != KVQ_PER_CHANNEL) return KVQ_ERR_UNSUPPORTED;
  if (f->role != KVQ_ROLE_KEY) return KVQ_ERR_UNSUPPORTED;
  if (f->group != 64 && f->group != 128) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// The format's constraints that depend on the head dimension.
static int validate_format_d(const kvq_format* f, int d) {
  if (d == 64 && (f->signs[2] | f->signs[3])) return KVQ_ERR_UNSUPPORTED;
  if (f->granularity == KVQ_PER_TOKEN_GROUP && f->group >= d) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

int validate_pack(const void* x, int B, int H, int n, int d, const kvq_format* f, int n_chunks, int chunk_idx,
                  const void* codes, const void* scale, const void* zero) {
  int st = validate_format(f);
  if (st) return st;
  if (!x || !codes || !scale || !zero) return KVQ_ERR_NULL;
  if (B < 1 || H < 1 || n < 1 || n_chunks < 1 || chunk_idx < 0 || chunk_idx >= n_chunks) return KVQ_ERR_SHAPE;
  if (d != 64 && d != 128) return KVQ_ERR_SHAPE;
  st = validate_format_d(f, d);
  if (st) return st;
  if ((long long)B * H > 65535) return KVQ_ERR_SHAPE;  // the grid's y dimension
  if (n > 0x7FFFFFFF - kTokenBlock) return KVQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scale) || !aligned16(zero)) return KVQ_ERR_ALIGN;
  return KVQ_OK;
}

int window_elems(const kvq_format* f, int B, int H, int d, int chunk_len, int n_chunks, size_t* code_words,
                 size_t* param_elems) {
  int st = validate_format(f);
  if (st) return st;
  if (!code_words || !param_elems) return KVQ_ERR_NULL;
  if (B < 1 || H < 1 || chunk_len < 1 || n_chunks < 0 || (d != 64 && d != 128)) return KVQ_ERR_SHAPE;
  if (chunk_len > 0x7FFFFFFF - kTokenBlock) return KVQ_ERR_SHAPE;
  st = validate_format_d(f, d);
  if (st) return st;
  const size_t cp = (size_t)chunk_pad(chunk_len);
  const size_t bh = (size_t)B * H;
  *code_words = bh * n_chunks * cp * d * f->bits / 32;
  if (f->granularity == KVQ_PER_TOKEN)
    *param_elems = bh * n_chunks * cp;
  else if (f->granularity == KVQ_PER_TOKEN_GROUP)
    *param_elems = bh * n_chunks * cp * (size_t)(d / f->group);
  else
    *param_elems = bh * n_chunks * (((size_t)chunk_len + f->group - 1) / f->group) * d;
  return KVQ_OK;
}

int validate_attn(const jb_attn_args* a, bool mass_only) {
  if (!a) return KVQ_ERR_NULL;
  const kvq_format& kf = a->k_fmt;
  const kvq_format& vf = a->v_fmt;
  if (kf.bits != 2 && kf.bits != 4) return KVQ_ERR_UNSUPPORTED;
  if (vf.bits != kf.bits) return KVQ_ERR_UNSUPPORTED;
  if (kf.role != KVQ_ROLE_KEY || vf.role != KVQ_ROLE_VALUE) return KVQ_ERR_UNSUPPORTED;
  if (kf.granularity == KVQ_PER_TOKEN_GROUP || vf.granularity == KVQ_PER_TOKEN_GROUP) {
    // group-wise keys and values together, one group size
    if (kf.granularity != vf.granularity || kf.group != vf.group) return KVQ_ERR_UNSUPPORTED;
    if ((kf.group != 32 && kf.group != 64) || kf.group >= a->d) return KVQ_ERR_UNSUPPORTED;
  } else {
    if (vf.granularity != KVQ_PER_TOKEN) return KVQ_ERR_UNSUPPORTED;
    if (kf.granularity != KVQ_PER_TOKEN && kf.granularity != KVQ_PER_CHANNEL) return KVQ_ERR_UNSUPPORTED;
  }
  if (kf.granularity == KVQ_PER_CHANNEL && kf.group != 64 && kf.group != 128) return KVQ_ERR_UNSUPPORTED;
  if ((kf.hadamard | vf.hadamard) & ~1) return KVQ_ERR_UNSUPPORTED;
  for (const kvq_format* f : {&kf, &vf}) {
    const uint32_t any = f->signs[0] | f->signs[1] | f->signs[2] | f->signs[3];
    if (any && !f->hadamard) return KVQ_ERR_UNSUPPORTED;
    if (a->d == 64 && (f->signs[2] | f->signs[3])) return KVQ_ERR_UNSUPPORTED;
  }
  if (a->correction != JB_CORR_NONE && a->correction != JB_CORR_TAYLOR && a->correction != JB_CORR_EXACT)
    return KVQ_ERR_UNSUPPORTED;
  if (a->d != 64 && a->d != 128) return KVQ_ERR_SHAPE;
  if (a->B < 1 || a->H < 1 || a->n_q < 1 || a->n_r < 0 || a->chunk_len < 1 || a->n_chunks < 0)
    return KVQ_ERR_SHAPE;
  if (a->chunk_len > 0x7FFFFFFF - kTokenBlock || a->n_r > 0x7FFFFFFF - kKeyTile ||
      a->n_q > 0x7FFFFFFF - kQueryBlock)
    return KVQ_ERR_SHAPE;
  if ((long long)a->n_chunks * a->chunk_len + a->n_r < 1) return KVQ_ERR_SHAPE;
  if (a->window_chunks < 0 || (a->window_chunks > 0 && a->window_chunks < a->n_chunks)) return KVQ_ERR_SHAPE;
  if (!(a->softmax_scale >= 0.f) || isinf(a->softmax_scale)) return KVQ_ERR_SHAPE;
  // the kernel addresses one head's attended window through 32-bit buffer offsets (the
  // products are bounded by division first: the sizes may be anywhere in int32's range)
  const long long head_bytes_per_token = (long long)a->d * kf.bits / 8;
  if ((long long)a->n_chunks > 0x7FFFFFFFLL / head_bytes_per_token / chunk_pad(a->chunk_len)) return KVQ_ERR_SHAPE;
  const long long nqblk = (a->n_q + kQueryBlock - 1) / kQueryBlock;
  if (nqblk > 0x7FFFFFFFLL / a->B / a->H) return KVQ_ERR_SHAPE;
  // workspace sizes (partial records of up to kMaxSplit shares) stay far inside size_t
  if ((double)a->B * a->H * a->n_q * (a->d + 4) * sizeof(float) * kMaxSplit > 0x1p62) return KVQ_ERR_SHAPE;
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

int validate_batch(const jb_attn_args* calls, int n, bool mass_only) {
  if (!calls) return KVQ_ERR_NULL;
  if (n < 1 || n > KVQ_BATCH_MAX) return KVQ_ERR_SHAPE;
  const jb_attn_args& a0 = calls[0];
  for (int c = 0; c < n; c++) {
    const int st = validate_attn(&calls[c], mass_only);
    if (st) return st;
    const jb_attn_args& a = calls[c];
    if (a.d != a0.d || a.k_fmt.bits != a0.k_fmt.bits || a.k_fmt.granularity != a0.k_fmt.granularity ||
        (a.k_fmt.granularity != KVQ_PER_TOKEN && a.k_fmt.group != a0.k_fmt.group) ||
        (a.correction == JB_CORR_EXACT) != (a0.correction == JB_CORR_EXACT))
      return KVQ_ERR_UNSUPPORTED;
  }
  long long total = 0;  // workgroups with up to kMaxSplit shares per call, each call's range on a multiple of 8
  for (int c = 0; c < n; c++)
    total += ((long long)(calls[c].n_q + kQueryBlock - 1) / kQueryBlock * calls[c].B * calls[c].H * kMaxSplit + 7) /
             8 * 8;
  if (total > 0x7FFFFFFFLL) return KVQ_ERR_SHAPE;
  return KVQ_OK;
}

int choose_split(long long grid, long long tiles, int cus) {
  if (cus < 1 || grid < 1 || tiles < 1) return 1;
  auto cost = [&](long long S) { return ((grid * S + cus - 1) / cus) * ((tiles + S - 1) / S); };
  long long best = cost(1);
  int n_split = 1;
  for (int S = 2; S <= kMaxSplit && S <= tiles; S++) {
    if (grid * S > 0x7FFFFFFFLL) break;
    const long long c = cost(S);
    if (4 * c <= 3 * best) {
      best = c;
      n_split = S;
    }
  }
  return n_split;
}

size_t partial_bytes(const jb_attn_args* a, long long shares) {
  return (size_t)shares * a->B * a->H * (size_t)a->n_q * (size_t)(a->d + 4) * sizeof(float);
}

long long call_tiles(const jb_attn_args* a) {
  return (long long)a->n_chunks * (chunk_pad(a->chunk_len) / kKeyTile) + (a->n_r + kKeyTile - 1) / kKeyTile;
}

AttnPlan plan_attn(const jb_attn_args* a, int cus) {
  AttnPlan pl;
  pl.n_qblk = (a->n_q + kQueryBlock - 1) / kQueryBlock;
  pl.n_split = 1;
  pl.part_bytes = 0;
  pl.dec_shares = 0;
  pl.dec_bytes = 0;
  if (cus < 1) return pl;
  // At most 32 queries (one stream) with per-token keys and a cached window: the decode
  // path, with as many one-wave shares (the window's, plus one per head for its current
  // chunk) as fit on the device at once (two per SIMD)
  const long long n_ct = (long long)a->n_chunks * (chunk_pad(a->chunk_len) / kKeyTile);
  if (a->n_q <= 32 && a->k_fmt.granularity == KVQ_PER_TOKEN && a->correction != JB_CORR_EXACT && n_ct > 0) {
    const long long bhc = (long long)a->B * a->H;
    const long long S = std::min(n_ct, std::max(1LL, 8LL * cus / bhc - (a->n_r > 0 ? 1 : 0)));
    if ((S + 1) * bhc <= 0x7FFFFFFFLL) {
      pl.dec_shares = (int)S;
      pl.dec_bytes = partial_bytes(a, S + (a->n_r > 0 ? 1 : 0));
    }
  }
  const long long grid = (long long)pl.n_qblk * a->B * a->H;
  pl.n_split = choose_split(grid, call_tiles(a), cus);
  if (pl.n_split > 1) pl.part_bytes = partial_bytes(a, pl.n_split);
  return pl;
}

int batch_split(const jb_attn_args* calls, int n, int cus) {
  long long grid = 0, tiles = 0;
  for (int c = 0; c < n; c++) {
    const jb_attn_args* a = &calls[c];
    grid += (long long)((a->n_q + kQueryBlock - 1) / kQueryBlock) * a->B * a->H;
    tiles = std::max(tiles, call_tiles(a));
  }
  const int S = choose_split(grid, tiles, cus);
  for (int c = 0; c < n; c++) {
    const jb_attn_args* a = &calls[c];
    if (S > 1 && (!a->workspace || !aligned16(a->workspace) || a->workspace_bytes < partial_bytes(a, S))) return 1;
  }
  return S;
}

}  // namespace kvq

extern "C" int32_t kvq_chunk_pad(int32_t chunk_len) {
  return chunk_len < 1 || chunk_len > 0x7FFFFFFF - kvq::kTokenBlock ? 0 : kvq::chunk_pad(chunk_len);
}

extern "C" int kvq_window_elems(const kvq_format* fmt, int32_t B, int32_t H, int32_t d, int32_t chunk_len,
                                int32_t n_chunks, size_t* code_words, size_t* param_elems) {
  return kvq::window_elems(fmt, B, H, d, chunk_len, n_chunks, code_words, param_elems);
}

extern "C" const char* kvq_status_str(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "a required pointer is NULL";
    case KVQ_ERR_SHAPE: return "a size is out of range or inconsistent";
    case KVQ_ERR_UNSUPPORTED: return "unsupported format or option combination";
    case KVQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KVQ_ERR_WORKSPACE: return "workspace smaller than the call needs (see jb_attn_workspace_bytes)";
    case KVQ_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}
