// block_manager.cpp — the host-side block manager of the C ABI (pa_bm_*).
//
// It owns no device memory: it hands out physical block ids and produces
// the inputs of the device calls (slot mappings, copy-on-write pairs, block
// tables).  What it does follows the pages:
//   * a pool of preallocated physical blocks handed out in O(1) from a free
//     list ("vLLM：大语言模型推理与服务库" §4.2 item 3; "vLLM 深度解析" §3.1);
//   * one block table per sequence, token t at slot
//     table[t / block_size] * block_size + t % block_size (§4.2 item 2);
//   * a new token goes into the last block, a new block being taken first
//     when that one is full (§4.3 item 2);
//   * fork / append / free with reference counts and copy-on-write of a
//     shared, partly filled last block ("vLLM 高性能大语言模型推理引擎深度技术
//     评估与分布式架构展望", the three primitives; "vLLM 深度解析" §3.1).
// Readings where the pages are silent or disagree: the free list is first in
// first out (the order that reproduces the interleaved 9-block figure of
// "vLLM 深度解析" §3.1); a full shared last block stays shared (the new
// token opens a new block); a batch append that the free list cannot cover
// changes nothing; a freed sequence returns its blocks in table order.
//
// Swap (the SWAP mode of preemption: the first of those pages, its section
// on preemption; "vLLM 深度解析" §3.2): a set of sequences that holds its
// blocks alone moves to a pool of host blocks and back; each distinct block
// moves once, in order of first appearance, into a block from the front of
// the other pool's free list, its reference count with it.  A swapped-out
// sequence can be freed but not appended to or forked.
//
// Host C++ only (built with the host compiler): a ring buffer of block ids
// for each free list, a reference count per block, a hash map of sequences.
#include <stdint.h>

#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

#include "pa.h"
#include "pa_error.h"

namespace {

// A first-in first-out free list of block ids over a ring buffer, with the
// reference count of every block of the pool.
struct BlockPool {
  int32_t num_blocks = 0;
  std::vector<int32_t> ring;  // free ids: ring[head .. head+count) mod num_blocks
  int64_t head = 0, count = 0;
  std::vector<int32_t> ref;   // references per block (0 = free)

  void init(int32_t n) {
    num_blocks = n;
    ring.resize(n);
    for (int32_t b = 0; b < n; ++b) ring[b] = b;
    head = 0;
    count = n;
    ref.assign(n, 0);
  }
  int32_t take() {
    const int32_t b = ring[head];
    head = head + 1 == num_blocks ? 0 : head + 1;
    --count;
    ref[b] = 1;
    return b;
  }
  void give_back(int32_t b) {
    ring[(head + count) % num_blocks] = b;
    ++count;
  }
};

}  // namespace

struct pa_block_manager {
  int32_t block_size = 0;
  BlockPool dev, host;  // the HBM pool and the pool of host blocks for swap
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;
    bool swapped = false;  // blocks are host blocks
  };
  std::unordered_map<int64_t, Seq> seqs;
  // Scratch of the append dry run and of swaps, kept to avoid per-call allocation.
  std::unordered_map<int64_t, std::pair<int32_t, bool>> dry_seq;  // len, last block private
  std::unordered_map<int32_t, int32_t> dry_drop;                  // references dropped by CoW
  std::unordered_map<int32_t, int32_t> held;                      // block -> references in a set
  std::vector<int32_t> order;                                     // distinct blocks of a set
  std::unordered_set<int64_t> listed;                             // ids of a set
};

namespace {

int32_t invalid(const char* msg) { return pa::record_error(PA_ERR_INVALID, msg); }
int32_t done() { return pa::record_error(PA_OK, ""); }

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
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->dev.take());
  s.len = num_tokens;
  for (int32_t t = 0; t < num_tokens; ++t)
    slot_mapping[t] = (int64_t)s.blocks[t / bm->block_size] * bm->block_size + t % bm->block_size;
  return done();
}

int32_t pa_bm_append(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                     int64_t* slot_mapping, int64_t* cow_pairs, int32_t* num_cow) {
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
    pa_block_manager::Seq& s = bm->seqs[seq_ids[i]];
    const int32_t off = s.len % bs;
    if (off == 0) {
      s.blocks.push_back(bm->dev.take());
    } else {
      const int32_t last = s.blocks.back();
      if (bm->dev.ref[last] > 1) {
        const int32_t fresh = bm->dev.take();
        --bm->dev.ref[last];
        s.blocks.back() = fresh;
        cow_pairs[2 * nc] = last;
        cow_pairs[2 * nc + 1] = fresh;
        ++nc;
      }
    }
    slot_mapping[i] = (int64_t)s.blocks.back() * bs + off;
    ++s.len;
  }
  *num_cow = nc;
  return done();
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
  for (int32_t b : it->second.blocks)
    if (--pool.ref[b] == 0) pool.give_back(b);
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

}  // extern "C"

namespace {

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
    const int32_t d = dst.take();
    dst.ref[d] = src.ref[b];
    src.ref[b] = 0;
    bm->held[b] = d;  // from here on: where block b went
    pairs[2 * k] = b;
    pairs[2 * k + 1] = d;
  }
  for (int32_t b : bm->order) src.give_back(b);
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

}  // extern "C"
