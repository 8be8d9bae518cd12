// Host-side prefill chunk planner.
//
// What a chunk is (split_indexer_prefill_chunks and
// build_prefill_chunk_metadata on the vLLM DeepSeek-V3.2 indexer backend
// page): a run of consecutive requests whose keys fit the gather workspace
// (N = sum of seq_lens) and whose logits fit the byte budget
// (M * N * 4 bytes, M = sum of query_lens), as long as possible from where
// the previous chunk stopped; a request too large even alone is a chunk of
// its own.  A chunk's query tokens are then scored in slices of
// max(1, budget / 4 / N) tokens, every slice after the first reusing the keys
// the first one gathered (skip_kv_gather), and a chunk without keys yields
// nothing.
#include <stdint.h>

#include <algorithm>

#include "../../include/idx.h"

namespace {

// The two limits a chunk must respect.
struct ChunkBudget {
  int64_t key_tokens;  // gather workspace, in keys
  int64_t logit_elems; // logits budget, in fp32 elements
  bool admits(int64_t queries, int64_t keys) const {
    return keys <= key_tokens && queries * keys <= logit_elems;
  }
};

// Appends the slices of one chunk (requests [first, last), its query tokens
// starting at batch token `token0`) to `out`, counting those that do not fit.
void emit_slices(const ChunkBudget& budget, int32_t first, int32_t last, int64_t queries, int64_t keys,
                 int64_t token0, bool alone, int32_t request_offset, idx_chunk* out, int32_t cap,
                 int32_t& count) {
  if (keys == 0) return;  // nothing to gather or score
  const int64_t width = std::max<int64_t>(1, budget.logit_elems / keys);
  for (int64_t a = 0; a < queries; a += width) {
    const int64_t b = std::min(queries, a + width);
    if (count < cap) {
      idx_chunk& c = out[count];
      c.req_begin = first + request_offset;
      c.req_end = last + request_offset;
      c.q_begin = static_cast<int32_t>(a);
      c.q_end = static_cast<int32_t>(b);
      c.total_seq_lens = keys;
      c.token_begin = token0 + a;
      c.token_end = token0 + b;
      c.skip_kv_gather = a != 0;
      c.over_budget = alone && !budget.admits(b - a, keys);
    }
    ++count;
  }
}

}  // namespace

extern "C" idx_status idx_prefill_chunks(const int32_t* seq_lens, const int32_t* query_lens,
                                         int32_t num_req, int64_t workspace_tokens,
                                         int64_t max_logits_bytes, int32_t request_offset,
                                         idx_chunk* out, int32_t out_cap, int32_t* n_out) {
  if (!n_out) return IDX_EINVAL;
  *n_out = 0;
  if (num_req < 0 || out_cap < 0 || workspace_tokens < 0 || max_logits_bytes < 0) return IDX_EINVAL;
  if (num_req > 0 && (!seq_lens || !query_lens)) return IDX_EINVAL;
  if (out_cap > 0 && !out) return IDX_EINVAL;
  for (int32_t i = 0; i < num_req; ++i)
    if (seq_lens[i] < 0 || query_lens[i] < 0) return IDX_EINVAL;

  const ChunkBudget budget{workspace_tokens, max_logits_bytes / 4};
  int32_t count = 0;
  int64_t token0 = 0;  // first query token of the chunk being formed
  for (int32_t first = 0; first < num_req;) {
    // grow [first, last) while the grown chunk is still admitted
    int64_t queries = 0, keys = 0;
    int32_t last = first;
    for (; last < num_req && budget.admits(queries + query_lens[last], keys + seq_lens[last]); ++last) {
      queries += query_lens[last];
      keys += seq_lens[last];
    }
    const bool alone = last == first;  // `first` does not fit even by itself
    if (alone) {
      queries = query_lens[first];
      keys = seq_lens[first];
      last = first + 1;
    }
    emit_slices(budget, first, last, queries, keys, token0, alone, request_offset, out, out_cap, count);
    token0 += queries;
    first = last;
  }
  *n_out = count;
  return count > out_cap ? IDX_ENOSPC : IDX_OK;
}
