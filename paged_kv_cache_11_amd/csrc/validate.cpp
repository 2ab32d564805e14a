// validate.cpp — host-side checks of the data arrays the device calls read
// (declared at the end of include/pa.h).
//
// The block table is the only map from a sequence's logical blocks to
// physical ones ("vLLM：大语言模型推理与服务库" §4.2 item 2), and the kernels
// follow it without a bounds check, as hardware follows a page table: an id
// past the pool, a length past its table or a slot outside the pool would
// make them read or write outside the pools.  These functions check host
// copies of those arrays and name the first bad entry, so a caller (or a
// debug mode of a binding) can stop before the launch.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <unordered_set>

#include "../../include/pa.h"
#include "pa_error.h"

namespace {

int32_t bad(int64_t* bad_index, int64_t idx, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (bad_index) *bad_index = idx;
  return pa::record_error(PA_ERR_INVALID, buf);
}

int32_t good(int64_t* bad_index) {
  if (bad_index) *bad_index = -1;
  return pa::record_error(PA_OK, "");
}

// The table row of one sequence: entries 0 .. ceil(L / bs) - 1 must be pool
// blocks.  Returns PA_OK or the error for the first bad entry.
int32_t check_row(const int32_t* block_tables, int64_t row, int32_t max_blocks_per_seq,
                  int64_t L, int32_t num_blocks, int32_t block_size, const char* len_name,
                  int64_t* bad_index) {
  const int64_t nblk = (L + block_size - 1) / block_size;
  if (nblk > max_blocks_per_seq)
    return bad(bad_index, row,
               "%s[%lld] = %lld needs %lld blocks, more than max_blocks_per_seq %d", len_name,
               (long long)row, (long long)L, (long long)nblk, max_blocks_per_seq);
  const int32_t* r = block_tables + row * max_blocks_per_seq;
  for (int64_t j = 0; j < nblk; ++j)
    if (r[j] < 0 || r[j] >= num_blocks)
      return bad(bad_index, row * max_blocks_per_seq + j,
                 "block_tables[%lld][%lld] = %d is not a block of the %d-block pool "
                 "(read for %s[%lld] = %lld)",
                 (long long)row, (long long)j, r[j], num_blocks, len_name, (long long)row,
                 (long long)L);
  return PA_OK;
}

bool pool_ok(int32_t num_blocks, int32_t block_size) { return num_blocks > 0 && block_size > 0; }

}  // namespace

extern "C" {

int32_t pa_validate_decode(const int32_t* block_tables, int32_t num_seqs,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           int32_t max_seq_len, int32_t num_blocks, int32_t block_size,
                           int64_t* bad_index) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_seq_len < 0 || !pool_ok(num_blocks, block_size))
    return bad(bad_index, -1, "pa_validate_decode: bad sizes");
  if (num_seqs > 0 && (!block_tables || !seq_lens))
    return bad(bad_index, -1, "pa_validate_decode: NULL array");
  for (int64_t s = 0; s < num_seqs; ++s) {
    const int64_t L = seq_lens[s];
    if (L < 0 || L > max_seq_len)
      return bad(bad_index, s, "seq_lens[%lld] = %lld is outside [0, max_seq_len %d]",
                 (long long)s, (long long)L, max_seq_len);
    if (int32_t r = check_row(block_tables, s, max_blocks_per_seq, L, num_blocks, block_size,
                              "seq_lens", bad_index))
      return r;
  }
  return good(bad_index);
}

int32_t pa_validate_prefill(const int32_t* query_start_loc, int32_t num_chunks,
                            int32_t num_tokens, int32_t max_query_len,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t num_blocks, int32_t block_size,
                            int64_t* bad_index) {
  if (num_chunks < 0 || num_tokens < 0 || max_query_len < 0 || max_blocks_per_seq <= 0 ||
      !pool_ok(num_blocks, block_size))
    return bad(bad_index, -1, "pa_validate_prefill: bad sizes");
  if (!query_start_loc || (num_chunks > 0 && (!block_tables || !seq_lens)))
    return bad(bad_index, -1, "pa_validate_prefill: NULL array");
  if (query_start_loc[0] != 0)
    return bad(bad_index, 0, "query_start_loc[0] = %d, not 0", query_start_loc[0]);
  for (int64_t c = 0; c < num_chunks; ++c) {
    const int64_t n = (int64_t)query_start_loc[c + 1] - query_start_loc[c];
    if (n < 0)
      return bad(bad_index, c + 1, "query_start_loc[%lld] = %d is below query_start_loc[%lld] = %d",
                 (long long)(c + 1), query_start_loc[c + 1], (long long)c, query_start_loc[c]);
    if (n > max_query_len)
      return bad(bad_index, c + 1, "chunk %lld has %lld queries, more than max_query_len %d",
                 (long long)c, (long long)n, max_query_len);
    const int64_t L = seq_lens[c];
    if (L < n)
      return bad(bad_index, c, "seq_lens[%lld] = %lld is below the chunk's %lld queries",
                 (long long)c, (long long)L, (long long)n);
    if (int32_t r = check_row(block_tables, c, max_blocks_per_seq, L, num_blocks, block_size,
                              "seq_lens", bad_index))
      return r;
  }
  if (query_start_loc[num_chunks] != num_tokens)
    return bad(bad_index, num_chunks, "query_start_loc[%d] = %d, not num_tokens %d", num_chunks,
               query_start_loc[num_chunks], num_tokens);
  return good(bad_index);
}

int32_t pa_validate_slots(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                          int32_t block_size, int64_t* bad_index) {
  if (num_tokens < 0 || !pool_ok(num_blocks, block_size))
    return bad(bad_index, -1, "pa_validate_slots: bad sizes");
  if (num_tokens > 0 && !slot_mapping) return bad(bad_index, -1, "pa_validate_slots: NULL array");
  const int64_t pool = (int64_t)num_blocks * block_size;
  std::unordered_set<int64_t> seen;
  seen.reserve((size_t)num_tokens * 2);
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int64_t s = slot_mapping[t];
    if (s < 0) continue;
    if (s >= pool)
      return bad(bad_index, t, "slot_mapping[%lld] = %lld is past the pool's %lld slots",
                 (long long)t, (long long)s, (long long)pool);
    if (!seen.insert(s).second)
      return bad(bad_index, t, "slot_mapping[%lld] = %lld repeats an earlier token's slot",
                 (long long)t, (long long)s);
  }
  return good(bad_index);
}

int32_t pa_validate_shared_prefix(const int32_t* block_tables, int32_t num_seqs,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t prefix_len, int32_t num_blocks, int32_t block_size,
                                  int64_t* bad_index) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || prefix_len < 0 || !pool_ok(num_blocks, block_size))
    return bad(bad_index, -1, "pa_validate_shared_prefix: bad sizes");
  if (prefix_len % block_size != 0)
    return bad(bad_index, -1, "prefix_len %d is not a multiple of block_size %d", prefix_len,
               block_size);
  const int64_t np = prefix_len / block_size;
  if (np > max_blocks_per_seq)
    return bad(bad_index, -1, "prefix_len %d needs %lld blocks, more than max_blocks_per_seq %d",
               prefix_len, (long long)np, max_blocks_per_seq);
  if (num_seqs > 0 && (!block_tables || !seq_lens))
    return bad(bad_index, -1, "pa_validate_shared_prefix: NULL array");
  for (int64_t j = 0; j < (num_seqs > 0 ? np : 0); ++j)
    if (block_tables[j] < 0 || block_tables[j] >= num_blocks)
      return bad(bad_index, j, "block_tables[0][%lld] = %d is not a block of the %d-block pool",
                 (long long)j, block_tables[j], num_blocks);
  for (int64_t s = 0; s < num_seqs; ++s) {
    if (seq_lens[s] < prefix_len)
      return bad(bad_index, s, "seq_lens[%lld] = %d is shorter than the shared prefix (%d)",
                 (long long)s, seq_lens[s], prefix_len);
    const int32_t* r = block_tables + s * max_blocks_per_seq;
    for (int64_t j = 0; j < np; ++j)
      if (r[j] != block_tables[j])
        return bad(bad_index, s * max_blocks_per_seq + j,
                   "block_tables[%lld][%lld] = %d differs from row 0's shared block %d",
                   (long long)s, (long long)j, r[j], block_tables[j]);
  }
  return good(bad_index);
}

int32_t pa_validate_block_pairs(const int64_t* block_mapping, int32_t num_pairs,
                                int32_t src_num_blocks, int32_t dst_num_blocks,
                                int32_t same_pool, int64_t* bad_index) {
  if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
    return bad(bad_index, -1, "pa_validate_block_pairs: bad sizes");
  if (num_pairs > 0 && !block_mapping)
    return bad(bad_index, -1, "pa_validate_block_pairs: NULL array");
  std::unordered_set<int64_t> dsts, srcs;
  for (int64_t i = 0; i < num_pairs; ++i) {
    const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
    if (src < 0 || src >= src_num_blocks)
      return bad(bad_index, 2 * i, "block_mapping[%lld][0] = %lld is not a block of the "
                 "%d-block source pool", (long long)i, (long long)src, src_num_blocks);
    if (dst < 0 || dst >= dst_num_blocks)
      return bad(bad_index, 2 * i + 1, "block_mapping[%lld][1] = %lld is not a block of the "
                 "%d-block destination pool", (long long)i, (long long)dst, dst_num_blocks);
    if (!dsts.insert(dst).second)
      return bad(bad_index, 2 * i + 1, "block_mapping[%lld][1] = %lld is an earlier pair's "
                 "destination", (long long)i, (long long)dst);
    srcs.insert(src);
  }
  if (same_pool) {
    for (int64_t i = 0; i < num_pairs; ++i) {
      const int64_t dst = block_mapping[2 * i + 1];
      if (srcs.count(dst))
        return bad(bad_index, 2 * i + 1, "block_mapping[%lld][1] = %lld is also a source: the "
                   "copies run concurrently", (long long)i, (long long)dst);
    }
  }
  return good(bad_index);
}

}  // extern "C"
