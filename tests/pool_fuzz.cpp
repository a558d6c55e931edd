// Randomised operations on the host block pool (pa_pool_*), built together
// with pool.cpp under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_pool_sanitized.py.  After every operation the pool's observable
// state must be consistent:
//   * every live sequence's table has ceil(len / block_size) entries, each a
//     valid block with a positive count;
//   * the counts equal the number of table entries naming each block;
//   * free blocks + blocks with a positive count = the pool size;
//   * slots returned by an append lie in the sequence's table at the right
//     offsets, and a copy-on-write pair names the old and the new block.
// Exit status 0 when every check holds; the first violation is printed.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pa.h"

// The pool reports errors through this hook (the full library records the
// message for pa_last_error).
pa_status pa_fail(pa_status st, const char*) { return st; }

namespace {

int failures = 0;

#define CHECK(cond, ...)                        \
  do {                                          \
    if (!(cond)) {                              \
      std::fprintf(stderr, "check failed: " __VA_ARGS__); \
      std::fprintf(stderr, "  (%s:%d)\n", __FILE__, __LINE__); \
      ++failures;                               \
      return false;                             \
    }                                           \
  } while (0)

bool consistent(const pa_pool* pool, int nb, int bs, const std::map<int, int>& live) {
  std::vector<int> uses(nb, 0);
  std::vector<int32_t> tab(1 << 16);
  for (const auto& kv : live) {
    const int sid = kv.first;
    const int len = pa_pool_seq_len(pool, sid);
    CHECK(len == kv.second, "seq %d length %d, expected %d\n", sid, len, kv.second);
    int32_t n = -1;
    CHECK(pa_pool_block_table(pool, sid, tab.data(), (int32_t)tab.size(), &n) == PA_OK,
          "block table of %d\n", sid);
    CHECK(n == (len + bs - 1) / bs, "seq %d has %d blocks for %d tokens\n", sid, n, len);
    for (int i = 0; i < n; ++i) {
      CHECK(tab[i] >= 0 && tab[i] < nb, "seq %d entry %d = %d\n", sid, i, tab[i]);
      ++uses[tab[i]];
    }
  }
  int used = 0;
  for (int b = 0; b < nb; ++b) {
    const int rc = pa_pool_refcount(pool, b);
    CHECK(rc == uses[b], "block %d count %d, %d table entries\n", b, rc, uses[b]);
    used += rc > 0;
  }
  CHECK(pa_pool_num_free(pool) + used == nb, "free %d + used %d != %d\n", pa_pool_num_free(pool),
        used, nb);
  CHECK(pa_pool_refcount(pool, nb) == -1 && pa_pool_refcount(pool, -1) == -1, "out-of-range count\n");
  return true;
}

bool run(uint32_t seed, int nb, int bs) {
  std::mt19937 rng(seed);
  std::vector<int32_t> order(nb);
  for (int i = 0; i < nb; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pa_pool* pool = nullptr;
  CHECK(pa_pool_create(nb, bs, order.data(), &pool) == PA_OK, "create\n");
  std::map<int, int> live;  // seq id -> length
  std::vector<int32_t> base_prompt(8 * bs);
  for (auto& t : base_prompt) t = (int32_t)(rng() % 50);
  for (int op = 0; op < 4000; ++op) {
    const int kind = (int)(rng() % 10);
    if (kind <= 1 || live.empty()) {  // new empty sequence
      int32_t sid = -1;
      CHECK(pa_pool_add_seq(pool, &sid) == PA_OK, "add_seq\n");
      live[sid] = 0;
    } else if (kind == 2) {  // prompt through the prefix cache: shared start, random tail
      const int n = (int)(rng() % (10 * bs)) + 1;
      std::vector<int32_t> toks(n);
      const int shared = (int)(rng() % (int)base_prompt.size());
      for (int i = 0; i < n; ++i) toks[i] = i < shared ? base_prompt[i] : (int32_t)(rng() % 50);
      int32_t sid = -1, cached = -1;
      const int free_before = pa_pool_num_free(pool);
      const pa_status st =
          pa_pool_add_seq_cached(pool, toks.data(), n, rng() % 2, &sid, &cached);
      if (st == PA_ERR_OUT_OF_BLOCKS) {
        CHECK(pa_pool_num_free(pool) == free_before, "failed cached add changed the pool\n");
      } else {
        CHECK(st == PA_OK, "add_seq_cached status %d\n", (int)st);
        CHECK(cached >= 0 && cached <= n && cached % bs == 0, "cached %d of %d\n", cached, n);
        live[sid] = n;
      }
    } else if (kind == 3) {  // fork a random live sequence
      auto it = live.begin();
      std::advance(it, rng() % live.size());
      int32_t child = -1;
      CHECK(pa_pool_fork(pool, it->first, &child) == PA_OK, "fork\n");
      live[child] = it->second;
    } else if (kind <= 7) {  // append
      auto it = live.begin();
      std::advance(it, rng() % live.size());
      const int n = (int)(rng() % (3 * bs)) + (rng() % 4 == 0 ? 0 : 1);
      std::vector<int64_t> slots(n + 1);
      int32_t cow[2] = {-1, -1}, n_cow = -1;
      const int old_len = it->second;
      const int free_before = pa_pool_num_free(pool);
      const pa_status st = pa_pool_append(pool, it->first, n, slots.data(), cow, 1, &n_cow);
      if (st == PA_ERR_OUT_OF_BLOCKS) {
        CHECK(pa_pool_num_free(pool) == free_before && pa_pool_seq_len(pool, it->first) == old_len,
              "failed append changed the pool\n");
      } else {
        CHECK(st == PA_OK, "append status %d\n", (int)st);
        it->second += n;
        std::vector<int32_t> tab(1 << 16);
        int32_t nt = 0;
        CHECK(pa_pool_block_table(pool, it->first, tab.data(), (int32_t)tab.size(), &nt) == PA_OK,
              "table\n");
        for (int i = 0; i < n; ++i) {
          const int pos = old_len + i;
          CHECK(slots[i] == (int64_t)tab[pos / bs] * bs + pos % bs, "slot of position %d\n", pos);
        }
        CHECK(n_cow == 0 || n_cow == 1, "n_cow %d\n", n_cow);
        if (n_cow == 1) {
          CHECK(cow[1] == tab[old_len / bs] && cow[0] != cow[1], "copy-on-write pair\n");
          CHECK(pa_pool_refcount(pool, cow[0]) >= 1, "source of a copy must stay referenced\n");
        }
      }
    } else {  // free
      auto it = live.begin();
      std::advance(it, rng() % live.size());
      CHECK(pa_pool_free_seq(pool, it->first) == PA_OK, "free\n");
      CHECK(pa_pool_seq_len(pool, it->first) == -1, "freed sequence still known\n");
      live.erase(it);
    }
    if (!consistent(pool, nb, bs, live)) {
      std::fprintf(stderr, "after operation %d (kind %d), seed %u\n", op, kind, seed);
      pa_pool_destroy(pool);
      return false;
    }
  }
  // bad arguments leave the pool as it was
  int32_t dummy = 0;
  CHECK(pa_pool_fork(pool, 1 << 30, &dummy) == PA_ERR_INVALID_ARGUMENT, "fork of unknown id\n");
  CHECK(pa_pool_append(pool, -5, 1, nullptr, nullptr, 0, nullptr) == PA_ERR_INVALID_ARGUMENT,
        "append to unknown id\n");
  CHECK(consistent(pool, nb, bs, live), "after bad arguments\n");
  pa_pool_destroy(pool);
  return true;
}

}  // namespace

int main() {
  const int cases[][2] = {{64, 16}, {40, 1}, {200, 4}, {17, 256}, {128, 32}};
  uint32_t seed = 1;
  for (const auto& c : cases)
    for (int r = 0; r < 3; ++r) run(seed++, c[0], c[1]);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("pool fuzz ok\n");
  return 0;
}
