// Host-side prefill chunk planner.
//
// Rules (split_indexer_prefill_chunks and build_prefill_chunk_metadata on the
// vLLM DeepSeek-V3.2 indexer backend page):
//   * requests are taken in order into a chunk while the chunk's key count
//     N = sum(seq_lens) stays within the gather workspace and its logits
//     M * N * 4 bytes (M = sum(query_lens)) within the logits budget;
//   * a request that does not fit even alone is taken alone anyway;
//   * the chunk's M query tokens are cut into slices of
//     max(1, (budget / 4) / N) tokens (all M at once when N == 0), so the
//     lone over-sized request still proceeds one token at a time;
//   * a slice that does not start at token 0 reuses the keys gathered for
//     the chunk's first slice (skip_kv_gather);
//   * chunks without keys produce no record.
#include <stdint.h>

#include "../../include/idx.h"

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

  const int64_t elems = max_logits_bytes / 4;
  int32_t count = 0;
  int64_t token_base = 0;  // first query token of request `start`
  int32_t end = 0;
  while (end < num_req) {
    const int32_t start = end;
    int64_t m = 0, n = 0;
    while (end < num_req) {
      const int64_t nm = m + query_lens[end];
      const int64_t nn = n + seq_lens[end];
      if (nn <= workspace_tokens && nm * nn <= elems) {
        m = nm;
        n = nn;
        ++end;
      } else {
        break;
      }
    }
    bool lone = false;
    if (end == start) {
      m = query_lens[end];
      n = seq_lens[end];
      ++end;
      lone = true;
    }
    const int64_t max_q = n > 0 ? (elems / n > 1 ? elems / n : 1) : m;
    for (int64_t q0 = 0; q0 < m; q0 += max_q) {
      const int64_t sub = (m - q0) < max_q ? (m - q0) : max_q;
      if (n > 0) {
        if (count < out_cap) {
          idx_chunk& c = out[count];
          c.req_begin = start + request_offset;
          c.req_end = end + request_offset;
          c.q_begin = static_cast<int32_t>(q0);
          c.q_end = static_cast<int32_t>(q0 + sub);
          c.total_seq_lens = n;
          c.token_begin = token_base + q0;
          c.token_end = token_base + q0 + sub;
          c.skip_kv_gather = q0 > 0 ? 1 : 0;
          c.over_budget = (lone && (n > workspace_tokens || sub * n > elems)) ? 1 : 0;
        }
        ++count;
      }
    }
    token_base += m;
  }
  *n_out = count;
  return count > out_cap ? IDX_ENOSPC : IDX_OK;
}
