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
};

// kReg: see select_row.
template <int NT, bool kReg = true>
__global__ __launch_bounds__(NT) void topk_kernel(TopkParams p) {
  __shared__ SelectShared<NT> sm;
  __shared__ int info[2];
  const int r = blockIdx.x;
  const RowArgs& R = p.rows;
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
    col0 = block_sum_int(part, sm.scan, NT);
    int seq = R.seq_lens[b];
    seq = seq > R.max_len ? R.max_len : seq;
    const int qlen = R.qsl[b + 1] - R.qsl[b];
    const int j = tok - (R.qsl[b] - q0);
    L = seq - qlen + j + 1;
    L = L < 0 ? 0 : (L > seq ? seq : L);
    L = R.ratio == 1 ? L : L / R.ratio;
  }
  select_row<NT, kReg>(p.logits + static_cast<int64_t>(r) * p.stride + col0, L, p.k,
                 p.out + static_cast<int64_t>(r) * p.k, sm);
}

}  // namespace idx
