// Host block manager of libpa: the bookkeeping that produces block_tables and
// slot_mapping for the kernels.
//
// Follows the mini-llm-engine post, §3.1 (physical blocks with a ref count and
// a content hash; an O(1) free list; a per-sequence table from logical to
// physical blocks; a block is allocated when the previous one is full and all
// are released when the request ends), §3.4 (full blocks keyed by content hash
// are shared by sequences with the same prefix, ref_count > 1; a shared block
// is copied before it is written: copy-on-write) and §3.5 (swap-out to host
// slots and swap-in to new device blocks), and the Pico-vLLM write-up, §3
// (cached blocks evicted least-recently-used, with lazy deletion: a released
// cached block keeps its content and hash until a new allocation needs it).
//
// Policy details the pages leave open (stated once here):
//  * A block's content hash chains the previous block's hash with the block's
//    16 tokens, so equal hashes mean equal whole prefixes; a hit is confirmed
//    by comparing the stored tokens.
//  * Hashes are registered only when the caller commits computed tokens
//    (pa_bm_commit), i.e. once the block's K/V are written.
//  * Prefix reuse stops at the first miss, and never covers a whole prompt:
//    at least one prompt token is left to compute.
//  * Allocation takes never-cached free blocks first (FIFO), then evicts the
//    least recently released cached block.
//  * Forked sequences share every block; appending to a shared last block
//    first moves the sequence to a fresh copy (the caller runs the returned
//    copy with pa_copy_blocks before the store).

#include <cstdint>
#include <cstring>
#include <deque>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace {

uint64_t mix(uint64_t h, uint64_t x) {
  // splitmix64 finaliser over the running state (a published 64-bit mixer)
  h ^= x + 0x9E3779B97F4A7C15ULL + (h << 6) + (h >> 2);
  h ^= h >> 30;
  h *= 0xBF58476D1CE4E5B9ULL;
  h ^= h >> 27;
  h *= 0x94D049BB133111EBULL;
  h ^= h >> 31;
  return h;
}

struct Block {
  int32_t ref = 0;
  bool hashed = false;  // registered in the prefix map (content valid)
  bool in_lru = false;  // released while hashed: evictable
  uint64_t hash = 0;
  std::vector<int32_t> tokens;  // the block's tokens when hashed (hit confirmation)
  std::list<int32_t>::iterator lru_it;
};

struct Seq {
  std::vector<int32_t> table;   // physical block per logical block
  std::vector<int32_t> tokens;  // every token of the sequence
  int32_t committed_blocks = 0;  // full blocks whose hash is registered
  uint64_t chain = 0;            // hash of the last committed block
  bool swapped = false;
  std::vector<int32_t> host_table;
};

}  // namespace

struct pa_block_manager {
  int32_t bs;
  std::vector<Block> blocks;
  std::deque<int32_t> free_list;
  std::list<int32_t> lru;  // oldest first
  std::unordered_map<uint64_t, int32_t> prefix;
  std::unordered_map<int64_t, Seq> seqs;
  std::deque<int32_t> host_free;
  int32_t num_host;

  pa_block_manager(int32_t nb, int32_t nh, int32_t bsz) : bs(bsz), blocks(nb), num_host(nh) {
    for (int32_t i = 0; i < nb; ++i) free_list.push_back(i);
    for (int32_t i = 0; i < nh; ++i) host_free.push_back(i);
  }

  int32_t available() const { return (int32_t)(free_list.size() + lru.size()); }

  void lru_remove(int32_t b) {
    Block& k = blocks[b];
    if (k.in_lru) {
      lru.erase(k.lru_it);
      k.in_lru = false;
    }
  }

  // a free block: never-cached first, else evict the least recently released cached one
  int32_t allocate() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.front();
      free_list.pop_front();
    } else if (!lru.empty()) {
      b = lru.front();
      lru_remove(b);
      Block& k = blocks[b];
      auto it = prefix.find(k.hash);
      if (it != prefix.end() && it->second == b) prefix.erase(it);
      k.hashed = false;
      k.tokens.clear();
    } else {
      return -1;
    }
    blocks[b].ref = 1;
    return b;
  }

  void release(int32_t b) {
    Block& k = blocks[b];
    if (--k.ref > 0) return;
    if (k.hashed) {
      lru.push_back(b);
      k.lru_it = std::prev(lru.end());
      k.in_lru = true;
    } else {
      free_list.push_back(b);
    }
  }

  static uint64_t block_hash(uint64_t chain, const int32_t* t, int32_t n) {
    uint64_t h = mix(chain, 0x5041u);
    for (int32_t i = 0; i < n; ++i) h = mix(h, (uint32_t)t[i]);
    return h;
  }

  Seq* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
};

namespace {

bool valid(const pa_block_manager* m) { return m != nullptr; }

}  // namespace

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t num_host_blocks, int32_t block_size) {
  if (num_blocks <= 0 || num_host_blocks < 0 || block_size != 16) return nullptr;
  return new (std::nothrow) pa_block_manager(num_blocks, num_host_blocks, block_size);
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int32_t pa_bm_num_free_blocks(const pa_block_manager* m) { return valid(m) ? m->available() : -1; }

int32_t pa_bm_num_cached_blocks(const pa_block_manager* m) {
  return valid(m) ? (int32_t)m->lru.size() : -1;
}

int32_t pa_bm_num_free_host_blocks(const pa_block_manager* m) {
  return valid(m) ? (int32_t)m->host_free.size() : -1;
}

int32_t pa_bm_block_ref(const pa_block_manager* m, int32_t block) {
  if (!valid(m) || block < 0 || block >= (int32_t)m->blocks.size()) return -1;
  return m->blocks[block].ref;
}

pa_status pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* tokens,
                             int32_t n_tokens, int32_t* n_cached_tokens) {
  if (!valid(m) || (!tokens && n_tokens > 0) || !n_cached_tokens) return PA_ERR_NULL;
  if (n_tokens <= 0) return PA_ERR_SHAPE;
  if (m->seqs.count(seq_id)) return PA_ERR_SHAPE;
  const int32_t bs = m->bs;
  const int32_t nblk = (n_tokens + bs - 1) / bs;
  Seq s;
  // reuse cached full blocks of an identical prefix (never the whole prompt)
  const int32_t max_reuse = (n_tokens - 1) / bs;
  uint64_t chain = 0;
  int32_t reused = 0;
  for (int32_t i = 0; i < max_reuse; ++i) {
    const uint64_t h = pa_block_manager::block_hash(chain, tokens + i * bs, bs);
    auto it = m->prefix.find(h);
    if (it == m->prefix.end()) break;
    Block& k = m->blocks[it->second];
    if (std::memcmp(k.tokens.data(), tokens + i * bs, sizeof(int32_t) * bs) != 0) break;
    chain = h;
    ++reused;
  }
  // enough blocks for the rest?  (reused blocks sitting in the LRU stop being evictable)
  int32_t reused_in_lru = 0;
  {
    uint64_t c = 0;
    for (int32_t i = 0; i < reused; ++i) {
      c = pa_block_manager::block_hash(c, tokens + i * bs, bs);
      if (m->blocks[m->prefix[c]].in_lru) ++reused_in_lru;
    }
  }
  if (nblk - reused > m->available() - reused_in_lru) return PA_ERR_CAPACITY;
  chain = 0;
  for (int32_t i = 0; i < reused; ++i) {
    chain = pa_block_manager::block_hash(chain, tokens + i * bs, bs);
    const int32_t b = m->prefix[chain];
    m->lru_remove(b);
    ++m->blocks[b].ref;
    s.table.push_back(b);
  }
  for (int32_t i = reused; i < nblk; ++i) s.table.push_back(m->allocate());
  s.tokens.assign(tokens, tokens + n_tokens);
  s.committed_blocks = reused;
  s.chain = chain;
  m->seqs.emplace(seq_id, std::move(s));
  *n_cached_tokens = reused * bs;
  return PA_OK;
}

pa_status pa_bm_commit(pa_block_manager* m, int64_t seq_id, int32_t n_computed_tokens) {
  if (!valid(m)) return PA_ERR_NULL;
  Seq* s = m->find(seq_id);
  if (!s || s->swapped || n_computed_tokens < 0 || n_computed_tokens > (int32_t)s->tokens.size())
    return PA_ERR_SHAPE;
  const int32_t bs = m->bs;
  const int32_t full = n_computed_tokens / bs;
  for (int32_t i = s->committed_blocks; i < full; ++i) {
    const uint64_t h = pa_block_manager::block_hash(s->chain, s->tokens.data() + i * bs, bs);
    s->chain = h;
    Block& k = m->blocks[s->table[i]];
    if (!k.hashed && !m->prefix.count(h)) {  // first writer of this content registers it
      k.hashed = true;
      k.hash = h;
      k.tokens.assign(s->tokens.begin() + i * bs, s->tokens.begin() + (i + 1) * bs);
      m->prefix[h] = s->table[i];
    }
  }
  if (full > s->committed_blocks) s->committed_blocks = full;
  return PA_OK;
}

pa_status pa_bm_append_token(pa_block_manager* m, int64_t seq_id, int32_t token, int32_t* slot,
                             int32_t* cow_src, int32_t* cow_dst) {
  if (!valid(m) || !slot || !cow_src || !cow_dst) return PA_ERR_NULL;
  Seq* s = m->find(seq_id);
  if (!s || s->swapped) return PA_ERR_SHAPE;
  const int32_t bs = m->bs;
  const int32_t p = (int32_t)s->tokens.size();
  *cow_src = *cow_dst = -1;
  if (p % bs == 0) {
    const int32_t b = m->allocate();
    if (b < 0) return PA_ERR_CAPACITY;
    s->table.push_back(b);
  } else {
    const int32_t last = s->table.back();
    if (m->blocks[last].ref > 1) {  // shared partial block: copy before writing
      const int32_t b = m->allocate();
      if (b < 0) return PA_ERR_CAPACITY;
      m->release(last);
      s->table.back() = b;
      *cow_src = last;
      *cow_dst = b;
    }
  }
  s->tokens.push_back(token);
  *slot = s->table[p / bs] * bs + p % bs;
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* m, int64_t parent_id, int64_t child_id) {
  if (!valid(m)) return PA_ERR_NULL;
  Seq* s = m->find(parent_id);
  if (!s || s->swapped || m->seqs.count(child_id)) return PA_ERR_SHAPE;
  Seq c = *s;
  for (int32_t b : c.table) ++m->blocks[b].ref;
  m->seqs.emplace(child_id, std::move(c));
  return PA_OK;
}

pa_status pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id) {
  if (!valid(m)) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_SHAPE;
  Seq& s = it->second;
  if (s.swapped) {
    for (int32_t h : s.host_table) m->host_free.push_back(h);
  } else {
    for (int32_t b : s.table) m->release(b);
  }
  m->seqs.erase(it);
  return PA_OK;
}

int32_t pa_bm_seq_len(const pa_block_manager* m, int64_t seq_id) {
  if (!valid(m)) return -1;
  auto it = m->seqs.find(seq_id);
  return it == m->seqs.end() ? -1 : (int32_t)it->second.tokens.size();
}

pa_status pa_bm_block_table(const pa_block_manager* m, int64_t seq_id, int32_t* out,
                            int32_t capacity, int32_t* n_blocks) {
  if (!valid(m) || !n_blocks) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end() || it->second.swapped) return PA_ERR_SHAPE;
  const std::vector<int32_t>& t = it->second.table;
  *n_blocks = (int32_t)t.size();
  if ((int32_t)t.size() > capacity) return PA_ERR_CAPACITY;
  if (!t.empty()) {
    if (!out) return PA_ERR_NULL;
    std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  }
  return PA_OK;
}

pa_status pa_bm_slots(const pa_block_manager* m, int64_t seq_id, int32_t start, int32_t n,
                      int32_t* slot_mapping) {
  if (!valid(m) || (!slot_mapping && n > 0)) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end() || it->second.swapped) return PA_ERR_SHAPE;
  const Seq& s = it->second;
  if (start < 0 || n < 0 || (int64_t)start + n > (int64_t)s.tokens.size()) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t t = start + i;
    slot_mapping[i] = s.table[t / m->bs] * m->bs + t % m->bs;
  }
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_block_manager* m, int64_t seq_id, int32_t* device_blocks,
                         int32_t* host_blocks, int32_t capacity, int32_t* n) {
  if (!valid(m) || !n) return PA_ERR_NULL;
  Seq* s = m->find(seq_id);
  if (!s || s->swapped) return PA_ERR_SHAPE;
  const int32_t k = (int32_t)s->table.size();
  *n = k;
  if (k > capacity) return PA_ERR_CAPACITY;
  if (k > (int32_t)m->host_free.size()) return PA_ERR_CAPACITY;
  if (k > 0 && (!device_blocks || !host_blocks)) return PA_ERR_NULL;
  s->host_table.clear();
  for (int32_t i = 0; i < k; ++i) {
    const int32_t h = m->host_free.front();
    m->host_free.pop_front();
    device_blocks[i] = s->table[i];
    host_blocks[i] = h;
    s->host_table.push_back(h);
  }
  for (int32_t b : s->table) m->release(b);
  s->table.clear();
  s->swapped = true;
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_block_manager* m, int64_t seq_id, int32_t* host_blocks,
                        int32_t* device_blocks, int32_t capacity, int32_t* n) {
  if (!valid(m) || !n) return PA_ERR_NULL;
  Seq* s = m->find(seq_id);
  if (!s || !s->swapped) return PA_ERR_SHAPE;
  const int32_t k = (int32_t)s->host_table.size();
  *n = k;
  if (k > capacity) return PA_ERR_CAPACITY;
  if (k > m->available()) return PA_ERR_CAPACITY;
  if (k > 0 && (!device_blocks || !host_blocks)) return PA_ERR_NULL;
  s->table.clear();
  for (int32_t i = 0; i < k; ++i) {
    const int32_t b = m->allocate();
    host_blocks[i] = s->host_table[i];
    device_blocks[i] = b;
    s->table.push_back(b);
    m->host_free.push_back(s->host_table[i]);
  }
  s->host_table.clear();
  s->swapped = false;
  // the restored blocks are private copies: their hashes are registered again on commit
  s->committed_blocks = 0;
  s->chain = 0;
  return PA_OK;
}

}  // extern "C"
