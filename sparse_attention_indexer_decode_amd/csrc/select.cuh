// Block-wide exact top-k selection of one row of fp32 logits.
//
// Semantics (the indexer's top-k as the glm5next sparse_indexer page and the
// DeepSeek-V3.2 indexer page use it): L == 0 -> all -1 (padded row); L <= k
// -> 0..L-1 then -1 (exact causal fill); otherwise the k positions with the
// largest logits, ties at the threshold going to the lowest positions,
// written in ascending position order.
//
// Keys: floats map to order-preserving 32-bit keys (-0.0 folded onto +0.0).
// Digits: d1 = key[31:20] (4096 bins), then key[19:10] and key[9:0].
//
// Method (few dependent global round trips):
//   1. d1 histogram of the row in LDS, one pass with many coalesced loads in
//      flight.
//   2. The d1 bin B1 holding the k-th largest; every element with d1 >= B1
//      is a candidate.  One pass appends the candidates (key, position) to
//      LDS (one reservation per wave, order irrelevant).
//   3. Two LDS histogram passes over the candidates of bin B1 fix the exact
//      threshold key T and how many elements equal to T are taken.
//   4. Winners are marked in an LDS bitmap over positions: every candidate
//      above T, and of those equal to T the `need` lowest positions (found by
//      a radix select on the positions themselves when T is tied); one
//      ordered scan over the bitmap words writes the k positions in
//      ascending order.
// Rows whose candidates exceed LDS capacity (very many equal keys) or whose
// length exceeds the bitmap use multi-pass global refinement and a global
// ordered compaction instead; both paths select the same set.
#pragma once

#include "device_common.cuh"

namespace idx {

constexpr int kD1Bins = 4096;
constexpr int kD1Shift = 20;
constexpr int kCandCap = 4096;
constexpr int kBitmapWords = 4096;  // bitmap path for rows up to 131072 keys

template <int NT>
struct SelectShared {
  uint32_t ckey[kCandCap];
  int cidx[kCandCap];
  union {
    int hist1[kD1Bins];          // first-digit histogram (when not given)
    uint32_t sel[kBitmapWords];  // winners, one bit per position
  } u;
  int hist2[1024];
  int scan[NT / kWave];
  int bc[8];
};

struct SelectState {
  uint32_t prefix;
  uint32_t pmask;
  int need;  // elements equal (under pmask) to prefix still to take
};

// Loads keys [i0, i0 + 4*V) of a row into registers (vector loads when the
// row is 16-byte aligned), so that all V loads are in flight together.
template <int V>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int i0, int L, bool aligned,
                                          uint32_t (&u)[4 * V], bool (&v)[4 * V]) {
  float f[4 * V];
  if (aligned && i0 + 4 * V <= L) {
#pragma unroll
    for (int c = 0; c < V; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(row + i0 + 4 * c);
      f[4 * c] = x.x;
      f[4 * c + 1] = x.y;
      f[4 * c + 2] = x.z;
      f[4 * c + 3] = x.w;
    }
#pragma unroll
    for (int j = 0; j < 4 * V; ++j) v[j] = true;
  } else {
#pragma unroll
    for (int j = 0; j < 4 * V; ++j) {
      v[j] = (i0 + j) < L;
      f[j] = v[j] ? row[i0 + j] : 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 4 * V; ++j) u[j] = ordered_key(f[j]);
}

// Loads, for passes where order does not matter, the V float4 quads
// q = c * NT + tid (c < V) of the chunk starting at `base`: each load
// instruction of a wave covers 1 KiB of consecutive keys.  Element j of the
// thread is position base + 4 (c * NT + tid) + (j % 4), c = j / 4.
template <int V, int NT>
__device__ __forceinline__ void load_keys_strided(const float* __restrict__ row, int base, int L, bool aligned,
                                                  uint32_t (&u)[4 * V], bool (&v)[4 * V]) {
  const int tid = threadIdx.x;
  float f[4 * V];
#pragma unroll
  for (int c = 0; c < V; ++c) {
    const int i0 = base + 4 * (c * NT + tid);
    if (aligned && i0 + 4 <= L) {
      const float4 x = *reinterpret_cast<const float4*>(row + i0);
      f[4 * c] = x.x;
      f[4 * c + 1] = x.y;
      f[4 * c + 2] = x.z;
      f[4 * c + 3] = x.w;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * c + j] = true;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[4 * c + j] = (i0 + j) < L;
        f[4 * c + j] = v[4 * c + j] ? row[i0 + j] : 0.0f;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4 * V; ++j) u[j] = ordered_key(f[j]);
}

template <int NT>
__device__ __forceinline__ int strided_pos(int base, int j) {
  return base + 4 * ((j / 4) * NT + static_cast<int>(threadIdx.x)) + (j % 4);
}

// Finds the digit bin holding the need-th largest element among `nbins`
// bins read through `bin(d)`; returns (digit, count above it, count in it).
template <int NT, class BinFn>
__device__ __forceinline__ void find_digit(int nbins, int need, BinFn bin, SelectShared<NT>& sm, int& digit,
                                           int& above_out, int& cnt_out) {
  const int tid = threadIdx.x;
  const int per = nbins / NT;
  const int hi = nbins - tid * per;
  int s = 0;
  for (int d = hi - per; d < hi; ++d) s += bin(d);
  int tot;
  const int above = block_exclusive_scan<NT>(s, tot, sm.scan);
  if (above < need && need <= above + s) {
    int acc = above;
    for (int d = hi - 1; d >= hi - per; --d) {
      const int c = bin(d);
      if (acc + c >= need) {
        sm.bc[0] = d;
        sm.bc[1] = acc;
        sm.bc[2] = c;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  digit = sm.bc[0];
  above_out = sm.bc[1];
  cnt_out = sm.bc[2];
  __syncthreads();
}

// d1 histogram of a row into sm.u.hist1.
template <int NT>
__device__ void row_histogram(const float* __restrict__ row, int L, bool aligned, SelectShared<NT>& sm) {
  const int tid = threadIdx.x;
  for (int j = tid; j < kD1Bins; j += NT) sm.u.hist1[j] = 0;
  __syncthreads();
  constexpr int V = 8;
  for (int base = 0; base < L; base += NT * 4 * V) {
    uint32_t u[4 * V];
    bool v[4 * V];
    load_keys_strided<V, NT>(row, base, L, aligned, u, v);
#pragma unroll
    for (int j = 0; j < 4 * V; ++j)
      if (v[j]) atomicAdd(&sm.u.hist1[u[j] >> kD1Shift], 1);
  }
  __syncthreads();
}

// Narrows st (prefix, pmask, need) among the elements matching st.prefix
// under st.pmask, over two digit passes (shift, bits); `for_each(fn)`
// visits the key of every element to consider and is called once per pass
// by all threads.  Returns the number of elements matching the final
// prefix (equal to st.need when the last bin examined is taken whole).
template <int NT, class ForEach>
__device__ int refine(SelectState& st, int shift0, int bits0, int shift1, int bits1, ForEach for_each,
                      SelectShared<NT>& sm) {
  const int tid = threadIdx.x;
  int cnt = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? shift0 : shift1;
    const int nb = 1 << (pass == 0 ? bits0 : bits1);
    const uint32_t dmask = static_cast<uint32_t>(nb - 1);
    for (int j = tid; j < nb; j += NT) sm.hist2[j] = 0;
    __syncthreads();
    const uint32_t prefix = st.prefix, pmask = st.pmask;
    for_each([&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&sm.hist2[(key >> shift) & dmask], 1);
    });
    __syncthreads();
    int digit, above;
    if (nb >= NT) {
      find_digit<NT>(nb, st.need, [&](int d) { return sm.hist2[d]; }, sm, digit, above, cnt);
    } else {
      // fewer bins than threads: pad the digit space to NT bins
      find_digit<NT>(NT, st.need, [&](int d) { return d < nb ? sm.hist2[d] : 0; }, sm, digit, above, cnt);
    }
    st.prefix |= static_cast<uint32_t>(digit) << shift;
    st.pmask |= dmask << shift;
    st.need -= above;
    if (st.need == cnt) break;  // the whole bin is taken
  }
  return cnt;
}

// Ordered compaction straight from the global row (fallback path).
template <int NT>
__device__ void compact_global(const float* __restrict__ row, int L, int k, bool aligned, const SelectState& st,
                               int* __restrict__ out, SelectShared<NT>& sm) {
  const int tid = threadIdx.x;
  int run_sel = 0, run_eq = 0;
  constexpr int V = 2;
  for (int base = 0; base < L && run_sel < k; base += NT * 4 * V) {
    const int i0 = base + tid * 4 * V;
    uint32_t u[4 * V];
    bool v[4 * V];
    load_keys<V>(row, i0, L, aligned, u, v);
    bool gt[4 * V], eq[4 * V];
    int c_eq = 0;
#pragma unroll
    for (int j = 0; j < 4 * V; ++j) {
      const uint32_t m = u[j] & st.pmask;
      gt[j] = v[j] && m > st.prefix;
      eq[j] = v[j] && m == st.prefix;
      c_eq += eq[j] ? 1 : 0;
    }
    int tot_eq;
    int eq_rank = block_exclusive_scan<NT>(c_eq, tot_eq, sm.scan) + run_eq;
    bool sel[4 * V];
    int c_sel = 0;
#pragma unroll
    for (int j = 0; j < 4 * V; ++j) {
      sel[j] = gt[j];
      if (eq[j]) {
        sel[j] = eq_rank < st.need;
        ++eq_rank;
      }
      c_sel += sel[j] ? 1 : 0;
    }
    int tot_sel;
    int pos = block_exclusive_scan<NT>(c_sel, tot_sel, sm.scan) + run_sel;
#pragma unroll
    for (int j = 0; j < 4 * V; ++j)
      if (sel[j]) out[pos++] = i0 + j;
    run_eq += tot_eq;
    run_sel += tot_sel;
  }
}

// Top-k of one row (kept out of line: it runs once per row, and inlining it
// would raise the scorer's register pressure).
template <int NT>
__device__ __noinline__ void select_row(const float* __restrict__ row, int L, int k, int* __restrict__ out,
                                        SelectShared<NT>& sm) {
  const int tid = threadIdx.x;
  if (L <= k) {
    for (int j = tid; j < k; j += NT) out[j] = (j < L) ? j : -1;
    return;
  }
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;

  // 1. first digit
  int B1, above1, cnt1;
  row_histogram<NT>(row, L, aligned, sm);
  find_digit<NT>(kD1Bins, k, [&](int d) { return sm.u.hist1[d]; }, sm, B1, above1, cnt1);
  SelectState st{static_cast<uint32_t>(B1) << kD1Shift, 0xFFFu << kD1Shift, k - above1};
  const int n_cand = above1 + cnt1;
  const bool fast = n_cand <= kCandCap && L <= kBitmapWords * 32;

  if (!fast) {
    // global refinement + global ordered compaction
    if (st.need != cnt1) {
      constexpr int V = 4;
      refine<NT>(st, 10, 10, 0, 10, [&](auto fn) {
        for (int base = 0; base < L; base += NT * 4 * V) {
          uint32_t u[4 * V];
          bool v[4 * V];
          load_keys_strided<V, NT>(row, base, L, aligned, u, v);
#pragma unroll
          for (int j = 0; j < 4 * V; ++j)
            if (v[j]) fn(u[j]);
        }
      }, sm);
    }
    compact_global<NT>(row, L, k, aligned, st, out, sm);
    return;
  }

  // 2. candidates (d1 >= B1) -> LDS: per-thread counts, one wave scan and
  //    one reservation per wave and chunk
  if (tid == 0) sm.bc[4] = 0;
  __syncthreads();
  {
    constexpr int V = 8;
    const uint32_t lo_key = static_cast<uint32_t>(B1) << kD1Shift;
    const int lane = lane_id();
    for (int base = 0; base < L; base += NT * 4 * V) {
      uint32_t u[4 * V];
      bool v[4 * V];
      load_keys_strided<V, NT>(row, base, L, aligned, u, v);
      int c = 0;
#pragma unroll
      for (int j = 0; j < 4 * V; ++j) c += (v[j] && u[j] >= lo_key) ? 1 : 0;
      const int incl = wave_inclusive_scan(c);
      const int wave_total = __shfl(incl, kWave - 1, kWave);
      int wbase = 0;
      if (lane == kWave - 1 && wave_total > 0) wbase = atomicAdd(&sm.bc[4], wave_total);
      wbase = __shfl(wbase, kWave - 1, kWave);
      int pos = wbase + incl - c;
#pragma unroll
      for (int j = 0; j < 4 * V; ++j) {
        if (v[j] && u[j] >= lo_key) {
          if (pos < kCandCap) {
            sm.ckey[pos] = u[j];
            sm.cidx[pos] = strided_pos<NT>(base, j);
          }
          ++pos;
        }
      }
    }
  }
  __syncthreads();
  const int nc = sm.bc[4];

  // 3. exact threshold among the candidates of bin B1
  int n_eq = cnt1;
  if (st.need != cnt1) {
    n_eq = refine<NT>(st, 10, 10, 0, 10, [&](auto fn) {
      for (int i = tid; i < nc; i += NT) fn(sm.ckey[i]);
    }, sm);
  }

  // 4. winners -> position bitmap
  const int W = (L + 31) >> 5;
  for (int j = tid; j < W; j += NT) sm.u.sel[j] = 0u;
  __syncthreads();
  const bool take_all_eq = st.need == n_eq;
  for (int i = tid; i < nc; i += NT) {
    const uint32_t m = sm.ckey[i] & st.pmask;
    const int p = sm.cidx[i];
    if (m > st.prefix || (take_all_eq && m == st.prefix)) atomicOr(&sm.u.sel[p >> 5], 1u << (p & 31));
  }
  if (!take_all_eq) {
    // equal keys at the threshold: the `need` lowest positions among them,
    // i.e. the largest of (2^17 - 1 - position), by radix select on 17 bits
    const uint32_t tprefix = st.prefix, tmask = st.pmask;
    SelectState ts{0u, 0u, st.need};
    refine<NT>(ts, 8, 9, 0, 8, [&](auto fn) {
      for (int i = tid; i < nc; i += NT)
        if ((sm.ckey[i] & tmask) == tprefix) fn(0x1FFFFu - static_cast<uint32_t>(sm.cidx[i]));
    }, sm);
    for (int i = tid; i < nc; i += NT) {
      const int p = sm.cidx[i];
      if ((sm.ckey[i] & tmask) == tprefix && (0x1FFFFu - static_cast<uint32_t>(p)) >= ts.prefix)
        atomicOr(&sm.u.sel[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();

  // 5. ordered emission
  const int wpt = (W + NT - 1) / NT;
  const int w0 = tid * wpt;
  const int w1 = (w0 + wpt < W) ? w0 + wpt : W;
  int c_sel = 0;
  for (int wd = w0; wd < w1; ++wd) c_sel += __popc(sm.u.sel[wd]);
  int tot;
  int pos = block_exclusive_scan<NT>(c_sel, tot, sm.scan);
  for (int wd = w0; wd < w1; ++wd) {
    uint32_t sel = sm.u.sel[wd];
    while (sel) {
      const int bpos = __builtin_ctz(sel);
      sel &= sel - 1u;
      out[pos++] = wd * 32 + bpos;
    }
  }
  __syncthreads();
}

}  // namespace idx
