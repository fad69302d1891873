// Drives the host layer of libpkv (pkv_host.cpp) built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer, against stubs.cpp: the
// block allocator with prefix caching under random appends, forks and
// releases (reference counts checked against the live tables); slot
// mapping; the precondition checks, and their debug mode inside the entry
// points (a refused call launches nothing); argument checks and workspace
// sizing of the attention calls.  Exits non-zero at the first failed check.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <random>
#include <vector>

#include "pkv.h"

extern int g_launches;

#define CHECK(c)                                                                          \
  do {                                                                                    \
    if (!(c)) {                                                                           \
      std::fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", __LINE__, #c, \
                   pkv_last_error());                                                     \
      std::exit(1);                                                                       \
    }                                                                                     \
  } while (0)

struct Seq {
  std::vector<int32_t> table;
  int len = 0;
};

static void check_refcounts(pkv_pool* p, const std::vector<Seq>& live, int nb) {
  std::vector<int> held(nb, 0);
  for (const Seq& s : live)
    for (int i = 0; i < (s.len + 15) / 16; ++i) held[s.table[i]] += 1;
  int64_t zero = 0;
  for (int b = 0; b < nb; ++b) {
    CHECK(pkv_pool_refcnt(p, b) == held[b]);
    zero += held[b] == 0;
  }
  CHECK(pkv_pool_num_free(p) == zero);
}

static void allocator_random(unsigned seed) {
  std::mt19937 rng(seed);
  const int NB = 3000, MAXB = 64;
  std::vector<int32_t> order(NB);
  std::iota(order.begin(), order.end(), 0);
  std::shuffle(order.begin(), order.end(), rng);
  pkv_pool* p = pkv_pool_create(NB, order.data(), 16);
  CHECK(p);
  std::vector<int32_t> prefix(341);
  for (auto& t : prefix) t = (int32_t)(rng() % 32000);
  std::vector<Seq> live;
  for (int it = 0; it < 3000; ++it) {
    const unsigned op = rng() % 6;
    if (op <= 1 || live.empty()) {  // a new request: cached prefix, then the rest
      const int n = 16 + (int)(rng() % 400);
      std::vector<int32_t> toks(n);
      for (int i = 0; i < n; ++i) toks[i] = (rng() & 1) && i < 341 ? prefix[i] : (int32_t)(rng() % 32000);
      Seq s;
      s.table.assign(MAXB, -1);
      int32_t hit = 0;
      CHECK(pkv_pool_match_prefix(p, toks.data(), n, s.table.data(), MAXB, &hit) == PKV_OK);
      std::vector<int64_t> slots(n - hit * 16);
      int64_t cow[2];
      const int st = pkv_pool_append(p, s.table.data(), MAXB, hit * 16, n - hit * 16, slots.data(), cow);
      if (st == PKV_ERR_NOMEM) {
        CHECK(pkv_pool_release(p, s.table.data(), hit) == PKV_OK);
        continue;
      }
      CHECK(st == PKV_OK && cow[0] == -1);
      CHECK(pkv_pool_cache_blocks(p, toks.data(), n, s.table.data(), n / 16) == PKV_OK);
      s.len = n;
      live.push_back(s);
    } else if (op == 2) {  // parallel sampling: another holder of the same blocks
      const Seq& a = live[rng() % live.size()];
      Seq b;
      b.table.assign(MAXB, -1);
      b.len = a.len;
      CHECK(pkv_pool_fork(p, a.table.data(), (a.len + 15) / 16, b.table.data()) == PKV_OK);
      live.push_back(b);
    } else if (op == 3) {  // decode or chunk append, copy-on-write of a shared partial block
      Seq& a = live[rng() % live.size()];
      const int add = 1 + (int)(rng() % 20);
      if ((a.len + add + 15) / 16 > MAXB) continue;
      const int32_t last = a.len % 16 ? a.table[a.len / 16] : -1;
      const int32_t last_ref = last >= 0 ? pkv_pool_refcnt(p, last) : 0;
      std::vector<int64_t> slots(add);
      int64_t cow[2];
      const int st = pkv_pool_append(p, a.table.data(), MAXB, a.len, add, slots.data(), cow);
      if (st == PKV_ERR_NOMEM) continue;
      CHECK(st == PKV_OK);
      CHECK((cow[0] >= 0) == (last >= 0 && last_ref > 1));
      if (cow[0] >= 0) CHECK(cow[0] == last && pkv_pool_refcnt(p, (int32_t)cow[1]) == 1);
      for (int k = 0; k < add; ++k) {
        const int pos = a.len + k;
        CHECK(slots[k] == (int64_t)a.table[pos / 16] * 16 + pos % 16);
      }
      a.len += add;
    } else {  // a request ends
      const size_t i = rng() % live.size();
      CHECK(pkv_pool_release(p, live[i].table.data(), (live[i].len + 15) / 16) == PKV_OK);
      live.erase(live.begin() + (long)i);
    }
    if (it % 250 == 0) check_refcounts(p, live, NB);
  }
  for (const Seq& s : live) CHECK(pkv_pool_release(p, s.table.data(), (s.len + 15) / 16) == PKV_OK);
  live.clear();
  check_refcounts(p, live, NB);
  CHECK(pkv_pool_num_free(p) == NB);
  pkv_pool_destroy(p);
}

static void slot_mapping_random(unsigned seed) {
  std::mt19937 rng(seed);
  const int B = 37, MAXB = 40;
  std::vector<int32_t> bt(B * MAXB), lens(B), qsl(B + 1, 0);
  for (auto& x : bt) x = (int32_t)(rng() % 5000);
  for (int s = 0; s < B; ++s) {
    lens[s] = 1 + (int)(rng() % (MAXB * 16));
    qsl[s + 1] = qsl[s] + 1 + (int)(rng() % std::min(lens[s], 40));
  }
  std::vector<int64_t> slots(qsl[B]);
  CHECK(pkv_build_slot_mapping(bt.data(), MAXB, qsl.data(), lens.data(), B, 16, slots.data()) == PKV_OK);
  for (int s = 0; s < B; ++s)
    for (int i = qsl[s]; i < qsl[s + 1]; ++i) {
      const int pos = lens[s] - (qsl[s + 1] - qsl[s]) + (i - qsl[s]);
      CHECK(slots[i] == (int64_t)bt[s * MAXB + pos / 16] * 16 + pos % 16);
    }
  lens[3] = MAXB * 16 + 1;
  CHECK(pkv_build_slot_mapping(bt.data(), MAXB, qsl.data(), lens.data(), B, 16, slots.data()) == PKV_ERR_RANGE);
}

static void validators_and_debug_mode() {
  pkv_cache c = {nullptr, 100, 16, 2, 64, PKV_BF16, 1.f, 1.f};
  const size_t bb = pkv_block_bytes(&c);
  CHECK(bb == 2 * 16 * 2 * 64 * 2);
  std::vector<char> pool(100 * bb);
  c.kv = pool.data();
  int64_t good[] = {0, 1599, -1, 17}, dup[] = {5, 6, -3, 5}, big[] = {1600};
  CHECK(pkv_validate_slots(&c, good, 4) == PKV_OK);
  CHECK(pkv_validate_slots(&c, dup, 4) == PKV_ERR_RANGE);
  CHECK(pkv_validate_slots(&c, big, 1) == PKV_ERR_RANGE);
  int64_t pairs_ok[] = {1, 2, 1, 3}, pairs_bad[] = {1, 2, 2, 3};
  CHECK(pkv_validate_block_pairs(pairs_ok, 2, 100, 100, 1) == PKV_OK);
  CHECK(pkv_validate_block_pairs(pairs_bad, 2, 100, 100, 1) == PKV_ERR_RANGE);
  CHECK(pkv_validate_block_pairs(pairs_bad, 2, 100, 100, 0) == PKV_OK);

  setenv("PKV_DEBUG_VALIDATE", "1", 1);
  std::vector<uint16_t> kn(4 * 2 * 64), vn(4 * 2 * 64);
  int before = g_launches;
  CHECK(paged_kv_write(&c, kn.data(), vn.data(), dup, 4, nullptr) == PKV_ERR_RANGE);
  CHECK(g_launches == before);
  CHECK(paged_kv_write(&c, kn.data(), vn.data(), good, 4, nullptr) == PKV_OK);
  CHECK(g_launches == before + 1);
  CHECK(block_copy(&c, pairs_bad, 2, nullptr) == PKV_ERR_RANGE);
  CHECK(block_copy(&c, pairs_ok, 2, nullptr) == PKV_OK);
  CHECK(g_launches == before + 2);
  // decode: 3 sequences, tables of 4 entries, one entry past the pool
  int32_t bt[3 * 4] = {7, 8, 9, 10, 11, 12, 13, 14, 15, 100, 16, 17};
  int32_t lens[3] = {50, 3, 30};
  std::vector<uint16_t> q(3 * 4 * 64);
  std::vector<float> out(3 * 4 * 64);
  std::vector<char> ws(pkv_attention_workspace_bytes(&c, 4, nullptr, lens, 3) + 256);
  before = g_launches;
  CHECK(paged_attention_decode(&c, out.data(), q.data(), 4, bt, 4, lens, lens, 3, 0.125f, ws.data(),
                               ws.size(), nullptr) == PKV_ERR_RANGE);  // block_tables[2][1] = 100
  CHECK(paged_attention_decode_noalloc(&c, out.data(), q.data(), 4, bt, 4, lens, lens, 3, 0.125f,
                                       nullptr) == PKV_ERR_RANGE);
  CHECK(g_launches == before);
  bt[9] = 18;
  CHECK(paged_attention_decode(&c, out.data(), q.data(), 4, bt, 4, lens, lens, 3, 0.125f, ws.data(),
                               ws.size(), nullptr) == PKV_OK);
  CHECK(paged_attention_decode_noalloc(&c, out.data(), q.data(), 4, bt, 4, lens, lens, 3, 0.125f,
                                       nullptr) == PKV_OK);
  CHECK(g_launches == before + 2);
  int32_t lens_dev[3] = {50, 3, 31};  // device lengths differ from the host copy
  CHECK(paged_attention_decode(&c, out.data(), q.data(), 4, bt, 4, lens_dev, lens, 3, 0.125f,
                               ws.data(), ws.size(), nullptr) == PKV_ERR_RANGE);
  unsetenv("PKV_DEBUG_VALIDATE");
}

static void attention_sizes(unsigned seed) {
  std::mt19937 rng(seed);
  pkv_cache c = {reinterpret_cast<void*>(0x1000), 1 << 20, 16, 8, 128, PKV_BF16, 1.f, 1.f};
  for (int it = 0; it < 200; ++it) {
    const int B = 1 + (int)(rng() % 300);
    std::vector<int32_t> lens(B), qsl(B + 1, 0);
    bool mixed = rng() & 1;
    for (int s = 0; s < B; ++s) {
      lens[s] = (int)(rng() % 5000) + (mixed ? 1 : 0);
      const int ql = mixed && rng() % 8 == 0 ? 1 + (int)(rng() % std::min(lens[s], 300)) : 1;
      qsl[s + 1] = qsl[s] + ql;
    }
    const int maxb = 5000 / 16 + 1;
    std::vector<int32_t> bt((size_t)B * maxb, 0);
    const size_t need = pkv_attention_workspace_bytes(&c, 32, mixed ? qsl.data() : nullptr, lens.data(), B);
    std::vector<char> ws(need + 1);
    std::vector<float> out((size_t)qsl[B] * 32 * 128);
    std::vector<uint16_t> q((size_t)qsl[B] * 32 * 128);
    int st;
    if (mixed)
      st = paged_attention_mixed(&c, out.data(), q.data(), 32, qsl.data(), lens.data(), qsl.data(),
                                 lens.data(), bt.data(), maxb, B, qsl[B], 0.1f, ws.data(), need, nullptr);
    else
      st = paged_attention_decode(&c, out.data(), q.data(), 32, bt.data(), maxb, lens.data(),
                                  lens.data(), B, 0.1f, ws.data(), need, nullptr);
    CHECK(st == PKV_OK);
    if (need > 0) {
      st = mixed ? paged_attention_mixed(&c, out.data(), q.data(), 32, qsl.data(), lens.data(),
                                         qsl.data(), lens.data(), bt.data(), maxb, B, qsl[B], 0.1f,
                                         ws.data(), need - 1, nullptr)
                 : paged_attention_decode(&c, out.data(), q.data(), 32, bt.data(), maxb, lens.data(),
                                          lens.data(), B, 0.1f, ws.data(), need - 1, nullptr);
      CHECK(st == PKV_ERR_WORKSPACE);
    }
  }
  CHECK(paged_attention_decode(&c, nullptr, nullptr, 32, nullptr, 1, nullptr, nullptr, 1, 0.1f,
                               nullptr, 0, nullptr) != PKV_OK);
}

int main() {
  for (unsigned seed = 1; seed <= 3; ++seed) allocator_random(seed);
  slot_mapping_random(7);
  validators_and_debug_mode();
  attention_sizes(11);
  std::printf("host layer under ASan/UBSan: ok (%d launches counted)\n", g_launches);
  return 0;
}
