// Block-wide exact top-k selection of one row of fp32 logits (radix select).
//
// Semantics (the indexer's top-k as the glm5next sparse_indexer page and the
// DeepSeek-V3.2 indexer page use it): L == 0 -> all -1 (padded row); L <= k
// -> 0..L-1 then -1 (exact causal fill); otherwise the k positions with the
// largest logits, ties at the threshold going to the lowest positions,
// written in ascending position order.
//
// Method: floats are mapped to order-preserving 32-bit keys; three histogram
// passes over 11/11/10 key bits (in LDS) find the key of the k-th largest
// element and how many elements equal to it are needed; a final pass
// compacts the winners in position order with block prefix sums.  A pass
// stops early when the remaining count equals a whole bin.
#pragma once

#include "device_common.cuh"

namespace idx {

constexpr int kSelBins = 2048;

template <int NT>
struct SelectShared {
  int hist[kSelBins];
  int scan[NT / kWave];
  int bcast[4];
};

// Four consecutive keys starting at i0 (vector load when the row is 16-byte
// aligned and the quad is in range).
__device__ __forceinline__ void load_keys4(const float* __restrict__ row, int i0, int L,
                                           bool aligned, uint32_t (&u)[4], bool (&v)[4]) {
  if (aligned && i0 + 3 < L) {
    float4 f = *reinterpret_cast<const float4*>(row + i0);
    u[0] = ordered_key(f.x);
    u[1] = ordered_key(f.y);
    u[2] = ordered_key(f.z);
    u[3] = ordered_key(f.w);
    v[0] = v[1] = v[2] = v[3] = true;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = (i0 + j) < L;
      u[j] = v[j] ? ordered_key(row[i0 + j]) : 0u;
    }
  }
}

template <int NT>
__device__ void select_row(const float* __restrict__ row, int L, int k, int* __restrict__ out,
                           SelectShared<NT>& sm) {
  const int tid = threadIdx.x;
  if (L <= k) {
    for (int j = tid; j < k; j += NT) out[j] = (j < L) ? j : -1;
    return;
  }
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;

  uint32_t prefix = 0u, pmask = 0u;
  int need = k;
  const int shifts[3] = {21, 10, 0};
  const int nbins_of[3] = {2048, 2048, 1024};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nbins = nbins_of[pass];
    for (int j = tid; j < nbins; j += NT) sm.hist[j] = 0;
    __syncthreads();
    for (int base = 0; base < L; base += NT * 4) {
      uint32_t u[4];
      bool v[4];
      load_keys4(row, base + tid * 4, L, aligned, u, v);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (v[j] && (u[j] & pmask) == prefix) atomicAdd(&sm.hist[(u[j] >> shift) & (nbins - 1)], 1);
    }
    __syncthreads();
    // Thread t owns digits [hi - per, hi), hi = nbins - t * per: thread 0 the top.
    const int per = nbins / NT;
    const int hi = nbins - tid * per;
    int s = 0;
    for (int d = hi - per; d < hi; ++d) s += sm.hist[d];
    int tot;
    const int above = block_exclusive_scan<NT>(s, tot, sm.scan);
    if (above < need && need <= above + s) {
      int acc = above;
      for (int d = hi - 1; d >= hi - per; --d) {
        const int c = sm.hist[d];
        if (acc + c >= need) {
          sm.bcast[0] = d;
          sm.bcast[1] = acc;
          sm.bcast[2] = c;
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
    const int digit = sm.bcast[0];
    const int cnt_above = sm.bcast[1];
    const int cnt_digit = sm.bcast[2];
    __syncthreads();
    prefix |= static_cast<uint32_t>(digit) << shift;
    pmask |= static_cast<uint32_t>(nbins - 1) << shift;
    need -= cnt_above;
    if (need == cnt_digit) break;  // the whole bin is selected
  }

  // Compaction in position order: keep (key above the prefix) or (key on the
  // prefix and among the first `need` such positions).
  int run_sel = 0, run_eq = 0;
  for (int base = 0; base < L && run_sel < k; base += NT * 4) {
    const int i0 = base + tid * 4;
    uint32_t u[4];
    bool v[4];
    load_keys4(row, i0, L, aligned, u, v);
    bool gt[4], eq[4];
    int c_eq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = u[j] & pmask;
      gt[j] = v[j] && m > prefix;
      eq[j] = v[j] && m == prefix;
      c_eq += eq[j] ? 1 : 0;
    }
    int tot_eq;
    int eq_rank = block_exclusive_scan<NT>(c_eq, tot_eq, sm.scan) + run_eq;
    bool sel[4];
    int c_sel = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sel[j] = gt[j];
      if (eq[j]) {
        sel[j] = eq_rank < need;
        ++eq_rank;
      }
      c_sel += sel[j] ? 1 : 0;
    }
    int tot_sel;
    int pos = block_exclusive_scan<NT>(c_sel, tot_sel, sm.scan) + run_sel;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (sel[j]) out[pos++] = i0 + j;
    run_eq += tot_eq;
    run_sel += tot_sel;
  }
}

}  // namespace idx
