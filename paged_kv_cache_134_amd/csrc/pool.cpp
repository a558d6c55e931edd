// Host block manager: FIFO free queue, per-block reference counts, per-sequence
// block tables, fork (sharing), append with copy-on-write, and a prefix cache
// of full blocks.
//
// Follows the block manager of the "Paged attention" post (k4i.top, sections
// "block manager" and "copy-on-write"), the free-block queue of "PagedAttention
// 在 vLLM 中的实现分析" (§4.1: take from the front, return to the back) and the
// reference counting of the ATB PagedAttention article (a block is released
// only when its count reaches zero).  Unlike that article's allocation loop,
// every operation here checks the free count first and changes nothing when
// it cannot complete.
//
// Prefix cache ("Paged attention" post, section "prefix caching"; "PagedAttention
// 在 vLLM 中的实现分析" §4.2-4.3): a full block is known by a chained hash of
// (parent block's hash, its token ids, an extra key); a new prompt walks its
// full blocks from the left and reuses every block found (count + 1) up to
// the first miss, then takes fresh blocks and registers the hashes of the full
// ones.  A block whose count drops to zero keeps its hash and goes to the back
// of the free queue; a hit on it takes it out of the queue again, and the
// hash is dropped only when the queue hands the block out for new content
// (least recently freed first).  Hash matches are confirmed against the
// stored parent hash, extra key and token ids, so a hash collision is a miss.
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

// Doubly linked FIFO of free blocks: O(1) pop at the front, push at the back
// and removal from the middle.
struct FreeList {
  std::vector<int32_t> prev, next;
  std::vector<char> in;
  int32_t head = -1, tail = -1, count = 0;

  void init(int32_t n) {
    prev.assign(n, -1);
    next.assign(n, -1);
    in.assign(n, 0);
  }
  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in[b] = 1;
    ++count;
  }
  void remove(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in[b] = 0;
    --count;
  }
  int32_t pop_front() {
    const int32_t b = head;
    remove(b);
    return b;
  }
  size_t size() const { return (size_t)count; }
};

// 64-bit mixing (splitmix64 finaliser) for the chained block hash.
uint64_t mix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

constexpr uint64_t kRootHash = 0x243F6A8885A308D3ull;  // parent hash of a prompt's first block

uint64_t block_hash(uint64_t parent, uint64_t extra, const int32_t* tok, int32_t n) {
  uint64_t h = mix64(parent ^ mix64(extra));
  for (int32_t i = 0; i < n; ++i) h = mix64(h ^ (uint32_t)tok[i]);
  return h;
}

}  // namespace

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  FreeList free_q;
  std::vector<int32_t> ref;
  // prefix cache: hash -> block, and per block its key (valid while cached)
  std::unordered_map<uint64_t, int32_t> cache;
  std::vector<char> cached;
  std::vector<uint64_t> c_hash, c_parent, c_extra;
  std::vector<int32_t> c_tokens;  // [num_blocks * block_size]
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
  // Front of the free queue, now holding new content: its cache entry (if
  // any) is dropped.
  int32_t take() {
    const int32_t b = free_q.pop_front();
    ref[b] = 1;
    if (cached[b]) {
      auto it = cache.find(c_hash[b]);
      if (it != cache.end() && it->second == b) cache.erase(it);
      cached[b] = 0;
    }
    return b;
  }
  // Cached block holding exactly (parent, extra, tokens), or -1.
  int32_t lookup(uint64_t h, uint64_t parent, uint64_t extra, const int32_t* tok) const {
    auto it = cache.find(h);
    if (it == cache.end()) return -1;
    const int32_t b = it->second;
    if (c_parent[b] != parent || c_extra[b] != extra ||
        std::memcmp(&c_tokens[(size_t)b * block_size], tok, sizeof(int32_t) * block_size) != 0)
      return -1;
    return b;
  }
  void register_block(int32_t b, uint64_t h, uint64_t parent, uint64_t extra, const int32_t* tok) {
    auto it = cache.find(h);
    if (it != cache.end() && it->second != b) cached[it->second] = 0;  // collision: newest wins
    cache[h] = b;
    cached[b] = 1;
    c_hash[b] = h;
    c_parent[b] = parent;
    c_extra[b] = extra;
    std::memcpy(&c_tokens[(size_t)b * block_size], tok, sizeof(int32_t) * block_size);
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
  p->free_q.init(num_blocks);
  p->cached.assign(num_blocks, 0);
  p->c_hash.assign(num_blocks, 0);
  p->c_parent.assign(num_blocks, 0);
  p->c_extra.assign(num_blocks, 0);
  p->c_tokens.assign((size_t)num_blocks * block_size, 0);
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

extern "C" pa_status pa_pool_add_seq_cached(pa_pool* pool, const int32_t* token_ids,
                                            int32_t num_tokens, uint64_t extra_key,
                                            int32_t* seq_id, int32_t* cached_tokens) {
  if (!pool || !seq_id || num_tokens < 0 || (num_tokens > 0 && !token_ids))
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_pool_add_seq_cached: bad argument");
  const int32_t bs = pool->block_size;
  const int64_t nfull = num_tokens / bs;
  const int64_t nblocks = ((int64_t)num_tokens + bs - 1) / bs;
  // longest run of cached full blocks from the left
  std::vector<uint64_t> hashes((size_t)nfull), parents((size_t)nfull);
  std::vector<int32_t> hits;
  uint64_t parent = kRootHash;
  bool missed = false;
  int64_t revived = 0;  // hits whose count is zero: they leave the free queue
  for (int64_t i = 0; i < nfull; ++i) {
    const int32_t* tok = token_ids + i * bs;
    parents[i] = parent;
    hashes[i] = block_hash(parent, extra_key, tok, bs);
    if (!missed) {
      const int32_t b = pool->lookup(hashes[i], parent, extra_key, tok);
      if (b >= 0) {
        hits.push_back(b);
        if (pool->ref[b] == 0) ++revived;
      } else {
        missed = true;
      }
    }
    parent = hashes[i];
  }
  const int64_t fresh = nblocks - (int64_t)hits.size();
  if (fresh + revived > (int64_t)pool->free_q.size())
    return pa_fail(PA_ERR_OUT_OF_BLOCKS, "pa_pool_add_seq_cached: not enough free blocks");
  pool->seqs.emplace_back();
  pa_pool::Seq& s = pool->seqs.back();
  s.live = true;
  s.len = num_tokens;
  for (int32_t b : hits) {
    if (pool->ref[b] == 0) pool->free_q.remove(b);
    pool->ref[b] += 1;
    s.table.push_back(b);
  }
  for (int64_t i = (int64_t)hits.size(); i < nblocks; ++i) {
    const int32_t b = pool->take();
    s.table.push_back(b);
    if (i < nfull) pool->register_block(b, hashes[i], parents[i], extra_key, token_ids + i * bs);
  }
  *seq_id = (int32_t)pool->seqs.size() - 1;
  if (cached_tokens) *cached_tokens = (int32_t)(hits.size() * (size_t)bs);
  return PA_OK;
}

extern "C" int32_t pa_pool_num_cached(const pa_pool* pool) {
  return pool ? (int32_t)pool->cache.size() : -1;
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
