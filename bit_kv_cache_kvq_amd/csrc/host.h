// Host-side argument validation and launch planning of libkvq (plain C++, no HIP).
//
// Everything the entry points decide before a launch lives here: format and shape checks,
// window sizes, the split of a small grid over window shares, the few-query plan and the
// workspace each plan needs. The kernels' translation units call these functions; this
// unit is also built on its own (with host sanitizers) by the CPU tests.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kTokenBlock = 64;   // padding granularity of a chunk and size of a value block
constexpr int kQueryBlock = 256;  // queries per workgroup of the attention kernel
constexpr int kKeyTile = 64;      // keys per tile of the attention kernel
constexpr int kMaxSplit = 8;      // largest number of window shares per query block

constexpr int chunk_pad(int chunk_len) { return (chunk_len + kTokenBlock - 1) / kTokenBlock * kTokenBlock; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Status of a storage format on its own (bits, granularity, group, role, rotation flags).
int validate_format(const kvq_format* f);

// Status of kvq_pack's arguments (nothing is dereferenced but the format).
int validate_pack(const void* x, int B, int H, int n, int d, const kvq_format* f, int n_chunks, int chunk_idx,
                  const void* codes, const void* scale, const void* zero);

// kvq_window_elems.
int window_elems(const kvq_format* f, int B, int H, int d, int chunk_len, int n_chunks, size_t* code_words,
                 size_t* param_elems);

// Status of one attention call's arguments (mass_only: jb_attn_mass, which reads no values).
int validate_attn(const jb_attn_args* a, bool mass_only);

// Status of a batch: every call valid, and the calls agree on what one launch shares.
int validate_batch(const jb_attn_args* calls, int n, bool mass_only);

struct AttnPlan {
  int n_qblk;         // query blocks per head
  int n_split;        // window shares per query block (1: unsplit)
  size_t part_bytes;  // workspace of the split partials (0 for n_split == 1)
  int dec_shares;     // few queries: shares of the cached tiles per head (0: no decode path)
  size_t dec_bytes;   // workspace of the decode path's partial records
};

// Shares per query block for `grid` query-block workgroups over `tiles` tiles each on `cus`
// compute units: cost = device rounds x tiles of the longest share; a split is taken only
// for a predicted gain of a quarter or more.
int choose_split(long long grid, long long tiles, int cus);

// Plan of one valid call on a device with `cus` compute units (cus < 1: no split, no
// decode path).
AttnPlan plan_attn(const jb_attn_args* a, int cus);

// Workspace a plan uses: the decode records when the decode path is planned, else the
// split partials.
inline size_t plan_workspace(const AttnPlan& pl) { return pl.dec_shares ? pl.dec_bytes : pl.part_bytes; }

// Bytes of the partial records of `shares` shares of one call.
size_t partial_bytes(const jb_attn_args* a, long long shares);

// Tiles of one query block's sequence (cached window, then current chunk).
long long call_tiles(const jb_attn_args* a);

// The share count of a batch (one for all calls) on `cus` compute units, and whether every
// call's workspace holds its partials for it (else 1).
int batch_split(const jb_attn_args* calls, int n, int cus);

}  // namespace kvq
