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
  // long rows split over workgroups (topk_chunk_kernel / topk_merge_kernel,
  // or topk_split_collect_kernel / topk_split_merge_kernel)
  int32_t chunks;     // chunk slots per row (ceil(max_keys / kRowCap))
  int32_t cap;        // candidates per chunk slot
  float* cand_val;    // [rows][chunks][cap] candidate logits
  int32_t* cand_pos;  // [rows][chunks][cap] their positions in the row
  int32_t* cand_cnt;  // [rows][chunks] candidates per chunk, -1: none usable (split collect only)
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
  const int64_t slot = (static_cast<int64_t>(r) * p.chunks + c) * p.cap;
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
  const int64_t base = static_cast<int64_t>(r) * p.chunks * p.cap;  // (cap = k here)
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

// Long rows split over workgroups with one threshold (k <= kSampleMaxK):
// the one-read selection of select_row_sampled cut at its collection.
// Every workgroup of a long row bins the same sample of the whole row
// (sample_threshold), so all of them hold the same threshold, and each
// collects the keys of its kRowCap-key chunk at or above it -- together
// exactly the row's keys at or above it -- into its slot of the candidate
// arrays, with their row positions and their count (-1 when the sample
// gave no threshold or the chunk holds more than kCandCap).  A row of at
// most kRowCap keys is finished by its chunk 0.  Then one workgroup per long
// row (topk_split_merge_kernel) gathers the chunks' candidates and, when
// they number at least k and at most kCandCap, selects exactly among them
// (select_candidates: the row's top k are among the keys at or above a
// value that at least k keys reach); otherwise it selects from the whole row
// by the two-read path.  Workgroup numbering as in topk_chunk_kernel.
template <int NT>
__global__ __launch_bounds__(NT) void topk_split_collect_kernel(TopkParams p) {
  static_assert(kRowCap <= NT * collect_chunk_keys<NT>(), "a chunk is one collection step");
  __shared__ SelectShared<NT> sm;
  __shared__ int info[2];
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
  const int64_t slot = static_cast<int64_t>(r) * p.chunks + c;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;  // (lo keeps the alignment)
  float fa[collect_chunk_keys<NT>()], fb[collect_chunk_keys<NT>()];
  LinearBins lb;
  float t0;
  int n = -1;
  if (L <= kBitmapWords * 32 && sample_threshold<NT>(row, L, p.k, aligned, row + lo, Lc, fa, sm, lb, t0)) {
    n = collect_by<NT>(row + lo, Lc, aligned, [&](float v) { return lb.raw(v) >= t0; }, sm, fa, fb);
    if (n > kCandCap) n = -1;
  }
  if (n > 0) {
    float* val = p.cand_val + slot * p.cap;
    int32_t* pos = p.cand_pos + slot * p.cap;
    for (int i = threadIdx.x; i < n; i += NT) {
      val[i] = __uint_as_float(sm.c.ckey[i]);
      pos[i] = lo + sm.c.cidx[i];
    }
  }
  if (threadIdx.x == 0) p.cand_cnt[slot] = n;
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_split_merge_kernel(TopkParams p) {
  __shared__ SelectShared<NT> sm;
  __shared__ int info[2];
  __shared__ int cnt[kMaxTopkChunks];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t slot0 = static_cast<int64_t>(r) * p.chunks;
  // requested with the row's length, in one round trip: the slots' counts
  // and candidate tid of every slot (all of a slot of at most NT)
  const int cnt_mine = tid < p.chunks ? p.cand_cnt[slot0 + tid] : 0;
  float v0[kMaxTopkChunks];
  int t0[kMaxTopkChunks];
#pragma unroll
  for (int c = 0; c < kMaxTopkChunks; ++c) {
    if (c < p.chunks) {
      v0[c] = p.cand_val[(slot0 + c) * p.cap + tid];
      t0[c] = p.cand_pos[(slot0 + c) * p.cap + tid];
    }
  }
  int L, col0;
  row_window<NT>(p.rows, r, L, col0, sm.scan, info);
  if (L <= kRowCap) return;  // finished by its chunk
  const int k = p.k;
  const int nc = (L + kRowCap - 1) / kRowCap;
  if (tid < nc) cnt[tid] = cnt_mine;
  __syncthreads();
  int total = 0;
  bool ok = true;
  for (int c = 0; c < nc; ++c) {
    ok = ok && cnt[c] >= 0;
    total += cnt[c] > 0 ? cnt[c] : 0;
  }
  const float* row = p.logits + static_cast<int64_t>(r) * p.stride + col0;
  int32_t* out = p.out + static_cast<int64_t>(r) * k;
  if (!ok || total < k || total > kCandCap) {
    select_row_stream<NT>(row, L, k, out, sm, false);
    return;
  }
  // the chunks' candidates, one after another, into the candidate area;
  // past a slot's first NT, every lane's loads in flight together (lanes
  // past the count load its last candidate again and store nothing)
  int off = 0;
#pragma unroll
  for (int c = 0; c < kMaxTopkChunks; ++c) {
    if (c < nc) {
      const int n = cnt[c];
      if (tid < n) {
        sm.c.ckey[off + tid] = __float_as_uint(v0[c]);
        sm.c.cidx[off + tid] = t0[c];
      }
      if (n > NT) {
        const float* val = p.cand_val + (slot0 + c) * p.cap;
        const int32_t* pos = p.cand_pos + (slot0 + c) * p.cap;
        constexpr int S = (kCandCap + NT - 1) / NT;
        float v[S];
        int t[S];
#pragma unroll
        for (int s = 1; s < S; ++s) {
          const int i = tid + s * NT;
          const int ic = i < n ? i : n - 1;
          v[s] = val[ic];
          t[s] = pos[ic];
        }
#pragma unroll
        for (int s = 1; s < S; ++s) {
          const int i = tid + s * NT;
          if (i < n) {
            sm.c.ckey[off + i] = __float_as_uint(v[s]);
            sm.c.cidx[off + i] = t[s];
          }
        }
      }
      off += n;
    }
  }
  __syncthreads();
  select_candidates<NT>(L, k, total, out, sm);
}

}  // namespace idx
