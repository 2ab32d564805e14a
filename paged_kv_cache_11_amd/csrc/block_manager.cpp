// block_manager.cpp — the host-side block manager of the C ABI (pa_bm_*).
//
// It owns no device memory: it hands out physical block ids and produces
// the inputs of the device calls (slot mappings, copy-on-write pairs, swap
// pairs, block tables).  What it does follows the pages:
//   * a pool of preallocated physical blocks handed out in O(1) from a free
//     list ("vLLM：大语言模型推理与服务库" §4.2 item 3; "vLLM 深度解析" §3.1);
//   * one block table per sequence, token t at slot
//     table[t / block_size] * block_size + t % block_size (§4.2 item 2);
//   * a new token goes into the last block, a new block being taken first
//     when that one is full (§4.3 item 2);
//   * fork / append / free with reference counts and copy-on-write of a
//     shared, partly filled last block ("vLLM 高性能大语言模型推理引擎深度技术
//     评估与分布式架构展望", the three primitives; "vLLM 深度解析" §3.1);
//   * swap for preemption (the first of those pages, its section on
//     preemption; "vLLM 深度解析" §3.2): a set of sequences that holds its
//     blocks alone moves to a pool of host blocks and back;
//   * automatic prefix caching (the same page, its section on prefix
//     caching): full blocks carry a chained hash of (parent hash, token ids,
//     extra hash) in a table; a new prompt reuses the blocks of its longest
//     cached prefix (lookup), taking them off the free list (touch); blocks
//     enter the table when they fill (commit); the free list's front block
//     leaves the table when it is taken (eviction).
// Readings where the pages are silent or disagree:
//   * the free list is first in first out (the order that reproduces the
//     interleaved 9-block figure of "vLLM 深度解析" §3.1), and a freed
//     sequence returns its blocks last block first.  With caching, eviction
//     is therefore least recently released first and, within one release,
//     the leaf end of a chain before its root;
//   * a full shared last block stays shared (the new token opens a new
//     block); a batch append that the free list cannot cover changes nothing;
//   * swapped sets move each distinct block once, in order of first
//     appearance; a swapped-out sequence can only be freed; moved blocks
//     leave the prefix cache;
//   * the block hash is 64-bit FNV-1a over the little-endian bytes of the
//     parent hash (0 for the first block), the token ids (int32) and the
//     extra hash; a hit also compares the stored token ids and extra hash;
//     the first block committed under a hash keeps it.
//
// Host C++ only (built with the host compiler): a doubly linked free queue
// per pool, a reference count per block, hash maps of sequences and of
// cached blocks.
#include <stdint.h>
#include <string.h>

#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

#include "pa.h"
#include "pa_error.h"

namespace {

// Free blocks of one pool in a doubly linked queue over block ids (O(1)
// push at the back, pop at the front and unlink from the middle), with the
// reference count of every block.
struct BlockPool {
  int32_t num_blocks = 0;
  std::vector<int32_t> prev, next;  // links of free blocks; -1 ends
  int32_t head = -1, tail = -1;
  int64_t count = 0;
  std::vector<int32_t> ref;  // references per block (0 = free)

  void init(int32_t n) {
    num_blocks = n;
    prev.assign(n, -1);
    next.assign(n, -1);
    ref.assign(n, 0);
    head = tail = -1;
    count = 0;
    for (int32_t b = 0; b < n; ++b) push_back(b);
  }
  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b;
    else head = b;
    tail = b;
    ++count;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b];
    else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b];
    else tail = prev[b];
    prev[b] = next[b] = -1;
    --count;
  }
  int32_t pop_front() {
    const int32_t b = head;
    unlink(b);
    return b;
  }
};

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t fnv_u64(uint64_t h, uint64_t x) {
  for (int i = 0; i < 8; ++i) {
    h ^= (x >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  return h;
}

uint64_t fnv_u32(uint64_t h, uint32_t x) {
  for (int i = 0; i < 4; ++i) {
    h ^= (x >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  return h;
}

uint64_t hash_block(uint64_t parent, const int32_t* tokens, int32_t n, uint64_t extra) {
  uint64_t h = fnv_u64(kFnvOffset, parent);
  for (int32_t i = 0; i < n; ++i) h = fnv_u32(h, (uint32_t)tokens[i]);
  return fnv_u64(h, extra);
}

}  // namespace

struct pa_block_manager {
  int32_t block_size = 0;
  BlockPool dev, host;  // the HBM pool and the pool of host blocks for swap
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;
    bool swapped = false;  // blocks are host blocks
    // Prefix caching: whether the token ids are known, the hash of every
    // full block, the ids in the partly filled last block, the extra hash.
    bool tracked = false;
    std::vector<uint64_t> hashes;
    std::vector<int32_t> partial;
    uint64_t extra = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  // Prefix cache (device pool only).
  bool caching = false;
  std::unordered_map<uint64_t, int32_t> table;  // hash -> cached block
  std::vector<uint8_t> cached;                  // per block
  std::vector<uint64_t> bhash, bextra;          // per cached block
  std::vector<int32_t> btokens;                 // [num_blocks][block_size]

  // Scratch of the append dry run and of swaps, kept to avoid per-call allocation.
  std::unordered_map<int64_t, std::pair<int32_t, bool>> dry_seq;  // len, last block private
  std::unordered_map<int32_t, int32_t> dry_drop;                  // references dropped by CoW
  std::unordered_map<int32_t, int32_t> held;                      // block -> references in a set
  std::vector<int32_t> order;                                     // distinct blocks of a set
  std::unordered_set<int64_t> listed;                             // ids of a set
  std::vector<uint64_t> scratch_hashes;
  std::vector<int32_t> scratch_hits;

  void uncache(int32_t b) {
    if (caching && cached[b]) {
      table.erase(bhash[b]);
      cached[b] = 0;
    }
  }
  // A device block from the front of the free queue (evicting it from the
  // cache if it is still there), with one reference.
  int32_t take_dev() {
    const int32_t b = dev.pop_front();
    uncache(b);
    dev.ref[b] = 1;
    return b;
  }
  int32_t take_host() {
    const int32_t b = host.pop_front();
    host.ref[b] = 1;
    return b;
  }
  void commit(int32_t b, uint64_t h, const int32_t* tokens, uint64_t extra) {
    if (table.count(h)) return;  // the first block under a hash keeps it
    table.emplace(h, b);
    cached[b] = 1;
    bhash[b] = h;
    bextra[b] = extra;
    memcpy(&btokens[(size_t)b * block_size], tokens, sizeof(int32_t) * block_size);
  }
  int32_t hit(uint64_t h, const int32_t* tokens, uint64_t extra) const {
    const auto it = table.find(h);
    if (it == table.end()) return -1;
    const int32_t b = it->second;
    if (bextra[b] != extra ||
        memcmp(&btokens[(size_t)b * block_size], tokens, sizeof(int32_t) * block_size) != 0)
      return -1;
    return b;
  }
};

namespace {

int32_t invalid(const char* msg) { return pa::record_error(PA_ERR_INVALID, msg); }
int32_t done() { return pa::record_error(PA_OK, ""); }

// The append of pa_bm_append (tokens == NULL) and pa_bm_append_tokens.
int32_t append_batch(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                     const int32_t* tokens, int64_t* slot_mapping, int64_t* cow_pairs,
                     int32_t* num_cow) {
  if (!bm) return invalid("pa_bm_append: NULL manager");
  if (num_seqs < 0) return invalid("pa_bm_append: negative num_seqs");
  if (!num_cow) return invalid("pa_bm_append: NULL num_cow");
  *num_cow = 0;
  if (num_seqs == 0) return done();
  if (!seq_ids || !slot_mapping || !cow_pairs) return invalid("pa_bm_append: NULL array");
  const int32_t bs = bm->block_size;
  // Dry run: the blocks the batch takes, with the same decisions as below.
  bm->dry_seq.clear();
  bm->dry_drop.clear();
  int64_t need = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return invalid("pa_bm_append: unknown sequence id");
    if (it->second.swapped) return invalid("pa_bm_append: the sequence is swapped out");
    auto& st = bm->dry_seq.try_emplace(seq_ids[i], it->second.len, false).first->second;
    if (st.first % bs == 0) {
      ++need;  // opens a new block, private from then on
      st.second = true;
    } else if (!st.second) {
      const int32_t last = it->second.blocks.back();
      int32_t& drop = bm->dry_drop[last];
      if (bm->dev.ref[last] - drop > 1) {
        ++need;  // copy on write
        ++drop;
        st.second = true;
      }
    }
    ++st.first;
  }
  if (need > bm->dev.count)
    return pa::record_error(PA_ERR_NO_BLOCKS, "pa_bm_append: not enough free blocks");
  int32_t nc = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    pa_block_manager::Seq& s = bm->seqs.find(seq_ids[i])->second;
    const int32_t off = s.len % bs;
    if (off == 0) {
      s.blocks.push_back(bm->take_dev());
    } else {
      const int32_t last = s.blocks.back();
      if (bm->dev.ref[last] > 1) {
        const int32_t fresh = bm->take_dev();
        --bm->dev.ref[last];
        s.blocks.back() = fresh;
        cow_pairs[2 * nc] = last;
        cow_pairs[2 * nc + 1] = fresh;
        ++nc;
      }
    }
    slot_mapping[i] = (int64_t)s.blocks.back() * bs + off;
    ++s.len;
    if (!tokens || !s.tracked) {
      s.tracked = false;  // token ids unknown from here on: no more commits
      continue;
    }
    s.partial.push_back(tokens[i]);
    if ((int32_t)s.partial.size() == bs) {  // the block is full: commit it
      const uint64_t h = hash_block(s.hashes.empty() ? 0 : s.hashes.back(), s.partial.data(), bs,
                                    s.extra);
      bm->commit(s.blocks.back(), h, s.partial.data(), s.extra);
      s.hashes.push_back(h);
      s.partial.clear();
    }
  }
  *num_cow = nc;
  return done();
}

// Swap of a set of sequences from one pool to the other (to_host: out).
int32_t move_set(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids, bool to_host,
                 int64_t* pairs, int32_t max_pairs, int32_t* num_pairs, const char* who) {
  if (!bm) return invalid(who);
  if (num_seqs < 0 || max_pairs < 0) return invalid("swap: negative size");
  if (!num_pairs) return invalid("swap: NULL num_pairs");
  *num_pairs = 0;
  if (num_seqs == 0) return done();
  if (!seq_ids || !pairs) return invalid("swap: NULL array");
  BlockPool& src = to_host ? bm->dev : bm->host;
  BlockPool& dst = to_host ? bm->host : bm->dev;
  bm->held.clear();
  bm->order.clear();
  bm->listed.clear();
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return invalid("swap: unknown sequence id");
    if (it->second.swapped == to_host)
      return invalid(to_host ? "swap out: a sequence is already swapped out"
                             : "swap in: a sequence is not swapped out");
    if (!bm->listed.insert(seq_ids[i]).second) return invalid("swap: a sequence is listed twice");
    for (int32_t b : it->second.blocks) {
      auto r = bm->held.try_emplace(b, 0);
      if (r.second) bm->order.push_back(b);
      ++r.first->second;
    }
  }
  for (int32_t b : bm->order)
    if (bm->held[b] != src.ref[b])
      return invalid("swap: a block is shared with a sequence outside the set");
  const int64_t n = (int64_t)bm->order.size();
  if (n > max_pairs) return invalid("swap: max_pairs is smaller than the blocks to move");
  if (n > dst.count) return pa::record_error(PA_ERR_NO_BLOCKS, "swap: not enough free blocks");
  for (int64_t k = 0; k < n; ++k) {
    const int32_t b = bm->order[k];
    if (to_host) bm->uncache(b);
    const int32_t d = to_host ? bm->take_host() : bm->take_dev();
    dst.ref[d] = src.ref[b];
    src.ref[b] = 0;
    bm->held[b] = d;  // from here on: where block b went
    pairs[2 * k] = b;
    pairs[2 * k + 1] = d;
  }
  for (int32_t b : bm->order) src.push_back(b);
  for (int32_t i = 0; i < num_seqs; ++i) {
    pa_block_manager::Seq& s = bm->seqs.find(seq_ids[i])->second;
    for (int32_t& b : s.blocks) b = bm->held[b];
    s.swapped = to_host;
  }
  *num_pairs = (int32_t)n;
  return done();
}

}  // namespace

extern "C" {

pa_block_manager* pa_bm_create_swap(int32_t num_blocks, int32_t num_host_blocks,
                                    int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0 || num_host_blocks < 0) {
    invalid("pa_bm_create: num_blocks and block_size must be positive, num_host_blocks >= 0");
    return nullptr;
  }
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) {
    invalid("pa_bm_create: out of host memory");
    return nullptr;
  }
  try {
    bm->block_size = block_size;
    bm->dev.init(num_blocks);
    bm->host.init(num_host_blocks);
  } catch (...) {
    delete bm;
    invalid("pa_bm_create: out of host memory");
    return nullptr;
  }
  done();
  return bm;
}

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  return pa_bm_create_swap(num_blocks, 0, block_size);
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free(const pa_block_manager* bm) {
  if (!bm) return invalid("pa_bm_num_free: NULL manager");
  return (int32_t)bm->dev.count;
}

int32_t pa_bm_num_free_host(const pa_block_manager* bm) {
  if (!bm) return invalid("pa_bm_num_free_host: NULL manager");
  return (int32_t)bm->host.count;
}

int32_t pa_bm_add(pa_block_manager* bm, int64_t seq_id, int32_t num_tokens, int64_t* slot_mapping) {
  if (!bm) return invalid("pa_bm_add: NULL manager");
  if (num_tokens < 0) return invalid("pa_bm_add: negative num_tokens");
  if (num_tokens > 0 && !slot_mapping) return invalid("pa_bm_add: NULL slot_mapping");
  if (bm->seqs.count(seq_id)) return invalid("pa_bm_add: sequence id already in use");
  const int64_t need = ((int64_t)num_tokens + bm->block_size - 1) / bm->block_size;
  if (need > bm->dev.count)
    return pa::record_error(PA_ERR_NO_BLOCKS, "pa_bm_add: not enough free blocks");
  pa_block_manager::Seq& s = bm->seqs[seq_id];
  s.blocks.reserve((size_t)need);
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take_dev());
  s.len = num_tokens;
  for (int32_t t = 0; t < num_tokens; ++t)
    slot_mapping[t] = (int64_t)s.blocks[t / bm->block_size] * bm->block_size + t % bm->block_size;
  return done();
}

int32_t pa_bm_append(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                     int64_t* slot_mapping, int64_t* cow_pairs, int32_t* num_cow) {
  return append_batch(bm, num_seqs, seq_ids, nullptr, slot_mapping, cow_pairs, num_cow);
}

int32_t pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return invalid("pa_bm_fork: NULL manager");
  const auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end()) return invalid("pa_bm_fork: unknown parent id");
  if (it->second.swapped) return invalid("pa_bm_fork: the parent is swapped out");
  if (bm->seqs.count(child_id)) return invalid("pa_bm_fork: child id already in use");
  pa_block_manager::Seq child = it->second;  // copy before the map may rehash
  for (int32_t b : child.blocks) ++bm->dev.ref[b];
  bm->seqs.emplace(child_id, std::move(child));
  return done();
}

int32_t pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return invalid("pa_bm_free: NULL manager");
  const auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return invalid("pa_bm_free: unknown sequence id");
  BlockPool& pool = it->second.swapped ? bm->host : bm->dev;
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (size_t j = blocks.size(); j-- > 0;)  // last block first
    if (--pool.ref[blocks[j]] == 0) pool.push_back(blocks[j]);
  bm->seqs.erase(it);
  return done();
}

int32_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return invalid("pa_bm_seq_len: NULL manager");
  const auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return invalid("pa_bm_seq_len: unknown sequence id");
  return it->second.len;
}

int32_t pa_bm_block_tables(const pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                           int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* seq_lens) {
  if (!bm) return invalid("pa_bm_block_tables: NULL manager");
  if (num_seqs < 0 || max_blocks_per_seq < 0) return invalid("pa_bm_block_tables: negative size");
  if (num_seqs == 0) return done();
  if (!seq_ids || !block_tables || !seq_lens) return invalid("pa_bm_block_tables: NULL array");
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return invalid("pa_bm_block_tables: unknown sequence id");
    if (it->second.swapped) return invalid("pa_bm_block_tables: a sequence is swapped out");
    if ((int64_t)it->second.blocks.size() > max_blocks_per_seq)
      return invalid("pa_bm_block_tables: a table is longer than max_blocks_per_seq");
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pa_block_manager::Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    const int32_t nb = (int32_t)s.blocks.size();
    for (int32_t j = 0; j < nb; ++j) row[j] = s.blocks[j];
    for (int32_t j = nb; j < max_blocks_per_seq; ++j) row[j] = -1;
    seq_lens[i] = s.len;
  }
  return done();
}

int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block) {
  if (!bm) return invalid("pa_bm_ref_count: NULL manager");
  if (block < 0 || block >= bm->dev.num_blocks) return invalid("pa_bm_ref_count: block out of range");
  return bm->dev.ref[block];
}

int32_t pa_bm_is_swapped(const pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return invalid("pa_bm_is_swapped: NULL manager");
  const auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return invalid("pa_bm_is_swapped: unknown sequence id");
  return it->second.swapped ? 1 : 0;
}

int32_t pa_bm_swap_out(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                       int64_t* pairs, int32_t max_pairs, int32_t* num_pairs) {
  return move_set(bm, num_seqs, seq_ids, true, pairs, max_pairs, num_pairs,
                  "pa_bm_swap_out: NULL manager");
}

int32_t pa_bm_swap_in(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                      int64_t* pairs, int32_t max_pairs, int32_t* num_pairs) {
  return move_set(bm, num_seqs, seq_ids, false, pairs, max_pairs, num_pairs,
                  "pa_bm_swap_in: NULL manager");
}

uint64_t pa_bm_block_hash(uint64_t parent_hash, const int32_t* tokens, int32_t num_tokens,
                          uint64_t extra_hash) {
  if (num_tokens < 0 || (num_tokens > 0 && !tokens)) return 0;
  return hash_block(parent_hash, tokens, num_tokens, extra_hash);
}

int32_t pa_bm_enable_prefix_caching(pa_block_manager* bm) {
  if (!bm) return invalid("pa_bm_enable_prefix_caching: NULL manager");
  if (!bm->seqs.empty()) return invalid("pa_bm_enable_prefix_caching: sequences exist");
  if (bm->caching) return done();
  try {
    const size_t n = (size_t)bm->dev.num_blocks;
    bm->cached.assign(n, 0);
    bm->bhash.assign(n, 0);
    bm->bextra.assign(n, 0);
    bm->btokens.assign(n * (size_t)bm->block_size, 0);
  } catch (...) {
    return invalid("pa_bm_enable_prefix_caching: out of host memory");
  }
  bm->caching = true;
  return done();
}

int32_t pa_bm_num_cached_blocks(const pa_block_manager* bm) {
  if (!bm) return invalid("pa_bm_num_cached_blocks: NULL manager");
  return (int32_t)bm->table.size();
}

int32_t pa_bm_add_prompt(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                         int32_t num_tokens, uint64_t extra_hash, int64_t* slot_mapping,
                         int32_t* num_cached_tokens) {
  if (!bm) return invalid("pa_bm_add_prompt: NULL manager");
  if (!bm->caching) return invalid("pa_bm_add_prompt: prefix caching is off");
  if (num_tokens < 0) return invalid("pa_bm_add_prompt: negative num_tokens");
  if (!num_cached_tokens) return invalid("pa_bm_add_prompt: NULL num_cached_tokens");
  if (num_tokens > 0 && (!tokens || !slot_mapping)) return invalid("pa_bm_add_prompt: NULL array");
  if (bm->seqs.count(seq_id)) return invalid("pa_bm_add_prompt: sequence id already in use");
  const int32_t bs = bm->block_size;
  const int32_t nfull = num_tokens / bs, nblk = (num_tokens + bs - 1) / bs;
  // Lookup: the chain of hashes, matched block by block up to the first miss.
  std::vector<uint64_t>& hs = bm->scratch_hashes;
  std::vector<int32_t>& hits = bm->scratch_hits;
  hs.clear();
  hits.clear();
  uint64_t h = 0;
  for (int32_t i = 0; i < nfull; ++i) {
    h = hash_block(h, tokens + (int64_t)i * bs, bs, extra_hash);
    hs.push_back(h);
  }
  int64_t hits_free = 0;
  for (int32_t i = 0; i < nfull; ++i) {
    const int32_t b = bm->hit(hs[i], tokens + (int64_t)i * bs, extra_hash);
    if (b < 0) break;
    hits.push_back(b);
    if (bm->dev.ref[b] == 0) ++hits_free;
  }
  const int64_t need = nblk - (int64_t)hits.size();
  if (need > bm->dev.count - hits_free)
    return pa::record_error(PA_ERR_NO_BLOCKS, "pa_bm_add_prompt: not enough free blocks");
  // Touch the hits, then take and commit the rest.
  pa_block_manager::Seq& s = bm->seqs[seq_id];
  s.blocks.reserve((size_t)nblk);
  for (int32_t b : hits) {
    if (bm->dev.ref[b] == 0) bm->dev.unlink(b);
    ++bm->dev.ref[b];
    s.blocks.push_back(b);
  }
  for (int32_t i = (int32_t)hits.size(); i < nblk; ++i) {
    const int32_t b = bm->take_dev();
    s.blocks.push_back(b);
    if (i < nfull) bm->commit(b, hs[i], tokens + (int64_t)i * bs, extra_hash);
  }
  s.len = num_tokens;
  s.tracked = true;
  s.hashes.assign(hs.begin(), hs.end());
  s.partial.assign(tokens + (int64_t)nfull * bs, tokens + num_tokens);
  s.extra = extra_hash;
  for (int32_t t = 0; t < num_tokens; ++t)
    slot_mapping[t] = (int64_t)s.blocks[t / bs] * bs + t % bs;
  *num_cached_tokens = (int32_t)hits.size() * bs;
  return done();
}

int32_t pa_bm_append_tokens(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                            const int32_t* tokens, int64_t* slot_mapping, int64_t* cow_pairs,
                            int32_t* num_cow) {
  if (num_seqs > 0 && !tokens) return invalid("pa_bm_append_tokens: NULL tokens");
  return append_batch(bm, num_seqs, seq_ids, tokens, slot_mapping, cow_pairs, num_cow);
}

}  // extern "C"
