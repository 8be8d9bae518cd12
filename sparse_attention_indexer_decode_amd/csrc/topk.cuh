// Standalone top-k over rows of logits: one workgroup per row.
#pragma once

#include "device_common.cuh"
#include "select.cuh"

namespace idx {

struct TopkParams {
  const float* logits;
  int64_t stride;
  RowArgs rows;
  int32_t k;
  int32_t* out;
  // long rows split over workgroups (topk_chunk_kernel / topk_merge_kernel)
  int32_t chunks;     // chunk slots per row (ceil(max_keys / kRowCap))
  float* cand_val;    // [rows][chunks * k] candidate logits in position order
  int32_t* cand_pos;  // [rows][chunks * k] their positions in the row
};

// Key count L and logits column base of row r (DECODE grid row or PREFILL
// chunk row); every thread of the workgroup gets the same values.  `scan`
// holds NT / 64 ints of LDS.
template <int NT>
__device__ __forceinline__ void row_window(const RowArgs& R, int r, int& L_out, int& col0_out, int* scan,
                                           int (&info)[2]) {
  int L = 0, col0 = 0;
  if (R.kind == 0) {
    const int b = r / R.next_n;
    const int i = r - b * R.next_n;
    int seq = R.seq_lens[b];
    seq = seq > R.max_len ? R.max_len : seq;
    const int dl = R.decode_lens ? R.decode_lens[b] : R.next_n;
    L = decode_row_len(seq, dl, i, R.max_len, R.ratio);
  } else {
    // request of chunk token q_begin + r, then its column base
    const int q0 = R.qsl[0];
    const int tok = R.q_begin + r;
    if (threadIdx.x == 0) {
      int lo = 0, hi = R.num_req;  // last b with qsl[b] - q0 <= tok
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (R.qsl[mid] - q0 <= tok) lo = mid; else hi = mid;
      }
      info[0] = lo;
    }
    __syncthreads();
    const int b = info[0];
    int part = 0;
    for (int j = threadIdx.x; j < b; j += NT) {
      part += request_keys(R.seq_lens[j], R.max_len, R.ratio);
    }
    col0 = block_sum_int(part, scan, NT);
    int seq = R.seq_lens[b];
    seq = seq > R.max_len ? R.max_len : seq;
    const int qlen = R.qsl[b + 1] - R.qsl[b];
    const int j = tok - (R.qsl[b] - q0);
    L = seq - qlen + j + 1;
    L = L < 0 ? 0 : (L > seq ? seq : L);
    L = R.ratio == 1 ? L : L / R.ratio;
  }
  L_out = L;
  col0_out = col0;
}

// kReg: see select_row.
template <int NT, bool kReg = true>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(kReg ? 1 : 6))) void topk_kernel(TopkParams p) {
  __shared__ SelectShared<NT> sm;
  __shared__ int info[2];
  const int r = blockIdx.x;
  int L, col0;
  row_window<NT>(p.rows, r, L, col0, sm.scan, info);
  select_row<NT, kReg>(p.logits + static_cast<int64_t>(r) * p.stride + col0, L, p.k,
                       p.out + static_cast<int64_t>(r) * p.k, sm);
}

// Rows longer than kRowCap keys split over workgroups (few rows, many CUs).
// Chunk c of a row holds its keys [c kRowCap, min(L, (c + 1) kRowCap)); the
// chunk's own top-k holds every key of the row's top-k that lies in it (ties
// go to the lower position inside a chunk as in the row).  Workgroup
// c * rows + r of topk_chunk_kernel selects k positions of chunk c of row r
// (into dynamic LDS); a row of at most kRowCap keys is finished there by
// its chunk 0.  The chunk also
// writes its candidates' logits and row positions, so that a row's
// candidates lie in position order -- chunk by chunk, each chunk's list
// ascending.  Then one workgroup per long row (topk_merge_kernel) selects k
// of them with the same rule (ties to the lower candidate index, which is
// the lower position) and writes their positions.
template <int NT>
__global__ __launch_bounds__(NT) void topk_chunk_kernel(TopkParams p) {
  __shared__ SelectShared<NT> sm;
  __shared__ int info[2];
  // chunk-major numbering: workgroup i runs on XCD i % 8, so the chunk-0
  // workgroups (all the work of rows of at most kRowCap keys) are spread
  // over every XCD by row, and are dispatched first
  const int nr = gridDim.x / p.chunks;
  const int c = blockIdx.x / nr;
  const int r = blockIdx.x - c * nr;
  int L, col0;
  row_window<NT>(p.rows, r, L, col0, sm.scan, info);
  const float* row = p.logits + static_cast<int64_t>(r) * p.stride + col0;
  if (L <= kRowCap) {
    if (c == 0) select_row<NT>(row, L, p.k, p.out + static_cast<int64_t>(r) * p.k, sm);
    return;
  }
  const int lo = c * kRowCap;
  if (lo >= L) return;
  const int Lc = L - lo < kRowCap ? L - lo : kRowCap;
  const int64_t slot = (static_cast<int64_t>(r) * p.chunks + c) * p.k;
  // the chunk's k selected positions go to the launch's dynamic LDS
  extern __shared__ int sel_pos[];
  select_row<NT>(row + lo, Lc, p.k, sel_pos, sm);
  // the candidates' logits and row positions, laid out for the merge while
  // the chunk is still in cache (every chunk but the last has more than k
  // keys, so the row's candidates are contiguous)
  __syncthreads();  // the selected positions are visible to every thread
  const int m = Lc < p.k ? Lc : p.k;
  for (int j = threadIdx.x; j < m; j += NT) {
    const int t = lo + sel_pos[j];
    p.cand_pos[slot + j] = t;
    p.cand_val[slot + j] = row[t];
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_merge_kernel(TopkParams p) {
  __shared__ SelectShared<NT> sm;
  __shared__ int info[2];
  const int r = blockIdx.x;
  int L, col0;
  row_window<NT>(p.rows, r, L, col0, sm.scan, info);
  if (L <= kRowCap) return;  // finished by its chunk
  const int k = p.k;
  const int nc = (L + kRowCap - 1) / kRowCap;
  const int last = L - (nc - 1) * kRowCap;  // keys of the last chunk
  // every chunk but the last has more than k keys (kRowCap > k): its k
  // entries are all positions; the last has min(last, k)
  const int n = (nc - 1) * k + (last < k ? last : k);
  const int64_t base = static_cast<int64_t>(r) * p.chunks * k;
  const float* val = p.cand_val + base;
  const int32_t* pos = p.cand_pos + base;
  int32_t* out = p.out + static_cast<int64_t>(r) * k;
  // n > k: k candidate indices, ascending, into the launch's dynamic LDS;
  // the register path sized to n (its passes cost the keys per thread it
  // is built for, not n)
  extern __shared__ int sel_idx[];
  if (n <= 8 * NT) select_row_reg<NT, 8>(val, n, k, sel_idx, sm);
  else if (n <= 16 * NT) select_row_reg<NT, 16>(val, n, k, sel_idx, sm);
  else select_row_reg<NT, kRowCap / NT>(val, n, k, sel_idx, sm);
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += NT) out[j] = pos[sel_idx[j]];
}

}  // namespace idx
