// Randomized check of libkvq's host-side validation and launch planning, built with the
// host compiler's address and undefined-behaviour sanitizers by the CPU tests. Pointers
// handed to the validators are small integers: validation must never dereference them.
// Prints "host_check ok <cases>" and exits 0 when every invariant holds.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <climits>

#include "host.h"

using namespace kvq;

static unsigned long long rng_state = 0x9E3779B97F4A7C15ull;
static unsigned long long next_u64() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 2685821657736338717ull;
}
static int pick(const int* v, int n) { return v[next_u64() % (unsigned)n]; }
static int range(int lo, int hi) { return lo + (int)(next_u64() % (unsigned long long)(hi - lo + 1)); }

#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "host_check: %s failed at line %d\n", #cond, __LINE__); \
      exit(1);                                                              \
    }                                                                       \
  } while (0)

static kvq_format random_format() {
  static const int bits[] = {-1, 0, 2, 2, 3, 4, 4, 8};
  static const int gran[] = {-1, 0, 0, 1, 1, 2, 2, 3};
  static const int group[] = {0, 16, 32, 64, 64, 128, 128, 256};
  static const int flag[] = {0, 1, 1, 2};
  kvq_format f;
  f.bits = pick(bits, 8);
  f.granularity = pick(gran, 8);
  f.group = pick(group, 8);
  f.hadamard = pick(flag, 4);
  f.role = pick(flag, 4);
  for (int i = 0; i < 4; i++) f.signs[i] = next_u64() % 4 == 0 ? (uint32_t)next_u64() : 0u;
  return f;
}

static const void* ptr_or_null(bool aligned) {
  const unsigned r = (unsigned)(next_u64() % 16);
  if (r == 0) return nullptr;
  return reinterpret_cast<const void*>((uintptr_t)(4096 + 16 * r + (aligned ? 0 : (r % 2 ? 2 : 8))));
}

static int random_size(int lo, int typical_hi) {
  static const int edge[] = {INT_MIN, -1, 0, 1, 63, 64, 65, 4680, 8160, 0x7FFFFFFF - 64, 0x7FFFFFFF};
  if (next_u64() % 8 == 0) return pick(edge, 11);
  return range(lo, typical_hi);
}

static jb_attn_args random_args() {
  static const int ds[] = {32, 64, 64, 128, 128, 256};
  static const int corr[] = {-1, 0, 1, 1, 2, 3};
  jb_attn_args a;
  memset(&a, 0, sizeof(a));
  const bool al = next_u64() % 8 != 0;
  a.B = random_size(1, 3);
  a.H = random_size(1, 64);
  a.d = pick(ds, 6);
  a.n_q = random_size(1, 9000);
  a.n_r = random_size(0, 9000);
  a.chunk_len = random_size(1, 9000);
  a.n_chunks = random_size(0, 20);
  a.q = (const uint16_t*)ptr_or_null(al);
  a.k_cur = (const uint16_t*)ptr_or_null(al);
  a.v_cur = (const uint16_t*)ptr_or_null(al);
  a.k_codes = (const uint32_t*)ptr_or_null(al);
  a.k_scale = (const uint16_t*)ptr_or_null(al);
  a.k_zero = (const uint16_t*)ptr_or_null(al);
  a.v_codes = (const uint32_t*)ptr_or_null(al);
  a.v_scale = (const uint16_t*)ptr_or_null(al);
  a.v_zero = (const uint16_t*)ptr_or_null(al);
  a.k_fmt = random_format();
  a.v_fmt = random_format();
  if (next_u64() % 2) {  // mostly consistent formats, so that planning is reached often
    a.k_fmt.bits = a.v_fmt.bits = next_u64() % 2 ? 2 : 4;
    a.k_fmt.role = KVQ_ROLE_KEY;
    a.v_fmt.role = KVQ_ROLE_VALUE;
    a.k_fmt.hadamard = a.v_fmt.hadamard = 1;
    a.v_fmt.granularity = KVQ_PER_TOKEN;
    if (a.k_fmt.granularity == KVQ_PER_TOKEN_GROUP) a.k_fmt.granularity = KVQ_PER_TOKEN;
    for (int i = 0; i < 4; i++) a.k_fmt.signs[i] = a.v_fmt.signs[i] = 0;
  }
  static const float scales[] = {0.f, 0.125f, -1.f, 1e30f};
  a.softmax_scale = scales[next_u64() % 4];
  a.correction = pick(corr, 6);
  a.o = (float*)ptr_or_null(al);
  a.mass_s = next_u64() % 2 ? (float*)ptr_or_null(al) : nullptr;
  a.mass_r = next_u64() % 2 ? a.mass_s : (float*)ptr_or_null(al);
  a.workspace = next_u64() % 2 ? (void*)ptr_or_null(al) : nullptr;
  a.workspace_bytes = (size_t)(next_u64() % (1ull << 30));
  a.window_chunks = next_u64() % 4 == 0 ? random_size(-1, 30) : 0;
  return a;
}

static void check_plan(const jb_attn_args* a, int cus) {
  const AttnPlan pl = plan_attn(a, cus);
  CHECK(pl.n_qblk == (a->n_q + kQueryBlock - 1) / kQueryBlock);
  CHECK(pl.n_split >= 1 && pl.n_split <= kMaxSplit);
  CHECK(pl.n_split == 1 || pl.n_split <= call_tiles(a));
  CHECK((pl.n_split == 1) == (pl.part_bytes == 0));
  if (pl.n_split > 1) CHECK(pl.part_bytes == partial_bytes(a, pl.n_split));
  if (cus < 1) CHECK(pl.n_split == 1 && pl.dec_shares == 0);
  if (pl.dec_shares) {
    CHECK(a->n_q <= 32 && a->k_fmt.granularity == KVQ_PER_TOKEN && a->correction != JB_CORR_EXACT);
    CHECK(pl.dec_shares <= (long long)a->n_chunks * (chunk_pad(a->chunk_len) / kKeyTile));
    CHECK(pl.dec_bytes == partial_bytes(a, pl.dec_shares + (a->n_r > 0 ? 1 : 0)));
    CHECK(plan_workspace(pl) == pl.dec_bytes);
  } else {
    CHECK(plan_workspace(pl) == pl.part_bytes);
  }
  // a split is taken only for a gain of a quarter or more
  if (pl.n_split > 1) {
    const long long grid = (long long)pl.n_qblk * a->B * a->H, T = call_tiles(a);
    auto cost = [&](long long S) { return ((grid * S + cus - 1) / cus) * ((T + S - 1) / S); };
    CHECK(4 * cost(pl.n_split) <= 3 * cost(1));
  }
}

int main() {
  long long cases = 0, valid_attn = 0;
  for (int i = 0; i < 300000; i++) {
    const kvq_format f = random_format();
    const int st = validate_format(&f);
    CHECK(st == KVQ_OK || st == KVQ_ERR_UNSUPPORTED);
    size_t cw = 0, pe = 0;
    const int d = next_u64() % 2 ? 128 : 64;
    const int B = random_size(1, 4), H = random_size(1, 64), cl = random_size(1, 9000), nc = random_size(0, 20);
    const int ws = window_elems(&f, B, H, d, cl, nc, &cw, &pe);
    if (ws == KVQ_OK) {
      CHECK(st == KVQ_OK && B >= 1 && H >= 1 && cl >= 1 && nc >= 0);
      CHECK(cw == (size_t)B * H * nc * chunk_pad(cl) * d * f.bits / 32);
      CHECK(f.granularity != KVQ_PER_TOKEN_GROUP || f.group < d);
    }
    const int ps = validate_pack(ptr_or_null(true), B, H, cl, d, &f, nc, range(-1, 3), ptr_or_null(true),
                                 ptr_or_null(true), ptr_or_null(next_u64() % 4 != 0));
    CHECK(ps <= 0 && ps >= KVQ_ERR_HIP);
    cases += 3;
  }
  static const int cus_v[] = {0, 1, 80, 256, 304};
  for (int i = 0; i < 300000; i++) {
    const jb_attn_args a = random_args();
    const bool mass_only = next_u64() % 2;
    const int st = validate_attn(&a, mass_only);
    CHECK(st <= 0 && st >= KVQ_ERR_HIP && st != KVQ_ERR_WORKSPACE);
    cases++;
    if (st != KVQ_OK) continue;
    valid_attn++;
    CHECK(a.d == 64 || a.d == 128);
    CHECK((long long)a.n_chunks * a.chunk_len + a.n_r >= 1);
    for (int c : cus_v) check_plan(&a, c);
    jb_attn_args batch[3] = {a, a, a};
    batch[1].n_q = 1 + (a.n_q % 700);
    const int bs = validate_batch(batch, 3, mass_only);
    if (bs == KVQ_OK) {
      const int S = batch_split(batch, 3, pick(cus_v, 5));
      CHECK(S >= 1 && S <= kMaxSplit);
    }
  }
  CHECK(validate_attn(nullptr, false) == KVQ_ERR_NULL);
  CHECK(validate_batch(nullptr, 1, false) == KVQ_ERR_NULL);
  CHECK(validate_format(nullptr) == KVQ_ERR_NULL);
  for (int s = -10; s <= 2; s++) CHECK(kvq_status_str(s) != nullptr);
  CHECK(kvq_chunk_pad(0x7FFFFFFF) == 0 && kvq_chunk_pad(4680) == 4736);
  for (long long g = 1; g < 3000; g += 7)
    for (long long t = 1; t < 700; t += 13) CHECK(choose_split(g, t, 256) >= 1);
  if (valid_attn < 1000) {
    fprintf(stderr, "host_check: only %lld valid attention cases\n", valid_attn);
    return 1;
  }
  printf("host_check ok %lld cases (%lld valid attention calls)\n", cases, valid_attn);
  return 0;
}
