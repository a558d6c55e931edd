// Host block manager: FIFO free queue, per-block reference counts, per-sequence
// block tables, fork (sharing) and append with copy-on-write.
//
// Follows the block manager of the "Paged attention" post (k4i.top, sections
// "block manager" and "copy-on-write"), the free-block queue of "PagedAttention
// 在 vLLM 中的实现分析" (§4.1: take from the front, return to the back) and the
// reference counting of the ATB PagedAttention article (a block is released
// only when its count reaches zero).  Unlike that article's allocation loop,
// every operation here checks the free count first and changes nothing when
// it cannot complete.
#include <cstring>
#include <deque>
#include <new>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_q;
  std::vector<int32_t> ref;
  struct Seq {
    bool live = false;
    int64_t len = 0;
    std::vector<int32_t> table;
  };
  std::vector<Seq> seqs;

  Seq* seq(int32_t id) {
    if (id < 0 || id >= (int32_t)seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  const Seq* seq(int32_t id) const {
    if (id < 0 || id >= (int32_t)seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  int32_t take() {
    int32_t b = free_q.front();
    free_q.pop_front();
    ref[b] = 1;
    return b;
  }
};

extern "C" pa_status pa_pool_create(int32_t num_blocks, int32_t block_size,
                                    const int32_t* free_order, pa_pool** out) {
  if (!out || num_blocks < 0 || block_size <= 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_create: bad sizes or null out");
  *out = nullptr;
  pa_pool* p = new (std::nothrow) pa_pool();
  if (!p) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_create: out of host memory");
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->ref.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_create: free_order is not a permutation");
      }
      seen[b] = 1;
      p->free_q.push_back(b);
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->free_q.push_back(i);
  }
  *out = p;
  return PA_OK;
}

extern "C" void pa_pool_destroy(pa_pool* pool) { delete pool; }

extern "C" pa_status pa_pool_add_seq(pa_pool* pool, int32_t* seq_id) {
  if (!pool || !seq_id) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_add_seq: null argument");
  pool->seqs.emplace_back();
  pool->seqs.back().live = true;
  *seq_id = (int32_t)pool->seqs.size() - 1;
  return PA_OK;
}

extern "C" pa_status pa_pool_fork(pa_pool* pool, int32_t parent, int32_t* child) {
  if (!pool || !child) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_fork: null argument");
  if (!pool->seq(parent)) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_fork: unknown parent");
  pool->seqs.emplace_back();
  pa_pool::Seq& c = pool->seqs.back();
  const pa_pool::Seq& p = pool->seqs[parent];
  c.live = true;
  c.len = p.len;
  c.table = p.table;
  for (int32_t b : c.table) pool->ref[b] += 1;
  *child = (int32_t)pool->seqs.size() - 1;
  return PA_OK;
}

extern "C" pa_status pa_pool_append(pa_pool* pool, int32_t seq_id, int32_t n,
                                    int64_t* slots_out, int32_t* cow_pairs,
                                    int32_t cow_cap, int32_t* n_cow) {
  if (!pool || n < 0) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_append: bad argument");
  pa_pool::Seq* s = pool->seq(seq_id);
  if (!s) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_append: unknown sequence");
  const int64_t bs = pool->block_size;
  const int64_t have = (int64_t)s->table.size();
  const int64_t want = (s->len + n + bs - 1) / bs;
  const bool cow = n > 0 && (s->len % bs) != 0 && pool->ref[s->table.back()] > 1;
  const int64_t need = (want - have) + (cow ? 1 : 0);
  if (need > (int64_t)pool->free_q.size())
    return pa_fail(PA_ERR_OUT_OF_BLOCKS, "pa_pool_append: not enough free blocks");
  if (cow && (cow_cap < 1 || !cow_pairs))
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_append: copy-on-write needs cow_pairs");
  if (n_cow) *n_cow = 0;
  if (cow) {
    const int32_t old = s->table.back();
    const int32_t fresh = pool->take();
    pool->ref[old] -= 1;
    s->table.back() = fresh;
    cow_pairs[0] = old;
    cow_pairs[1] = fresh;
    if (n_cow) *n_cow = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t p = s->len + i;
    const int64_t lb = p / bs;
    if (lb == (int64_t)s->table.size()) s->table.push_back(pool->take());
    if (slots_out) slots_out[i] = (int64_t)s->table[lb] * bs + p % bs;
  }
  s->len += n;
  return PA_OK;
}

extern "C" pa_status pa_pool_free_seq(pa_pool* pool, int32_t seq_id) {
  if (!pool) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_free_seq: null pool");
  pa_pool::Seq* s = pool->seq(seq_id);
  if (!s) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_free_seq: unknown sequence");
  for (int32_t b : s->table) {
    if (--pool->ref[b] == 0) pool->free_q.push_back(b);
  }
  s->table.clear();
  s->table.shrink_to_fit();
  s->len = 0;
  s->live = false;
  return PA_OK;
}

extern "C" pa_status pa_pool_block_table(const pa_pool* pool, int32_t seq_id, int32_t* out,
                                         int32_t cap, int32_t* n) {
  if (!pool) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_block_table: null pool");
  const pa_pool::Seq* s = pool->seq(seq_id);
  if (!s) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_block_table: unknown sequence");
  const int32_t len = (int32_t)s->table.size();
  if (n) *n = len;
  if (out) {
    if (cap < len) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_block_table: cap too small");
    if (len) std::memcpy(out, s->table.data(), sizeof(int32_t) * len);
  }
  return PA_OK;
}

extern "C" int32_t pa_pool_seq_len(const pa_pool* pool, int32_t seq_id) {
  if (!pool) return -1;
  const pa_pool::Seq* s = pool->seq(seq_id);
  return s ? (int32_t)s->len : -1;
}

extern "C" int32_t pa_pool_num_free(const pa_pool* pool) {
  return pool ? (int32_t)pool->free_q.size() : -1;
}

extern "C" int32_t pa_pool_refcount(const pa_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->ref[block];
}
