// Block-wide exact top-k selection of one row of fp32 logits.
//
// Semantics (the indexer's top-k as the glm5next sparse_indexer page and the
// DeepSeek-V3.2 indexer page use it): L == 0 -> all -1 (padded row); L <= k
// -> 0..L-1 then -1 (exact causal fill); otherwise the k positions with the
// largest logits, ties at the threshold going to the lowest positions,
// written in ascending position order.
//
// Keys: floats map to order-preserving 32-bit keys (-0.0 folded onto +0.0).
// Digits of the radix passes: d1 = key[31:20] (4096 bins), then key[19:10]
// and key[9:0].
//
// Rows of up to kRowCap keys (the common case) stay in registers, 32 keys
// (eight 16-byte quads) per thread (select_row_reg):
//   1. the whole row is loaded at once; one block reduction gives its min and
//      max;
//   2. first digit = a linear map of the value onto 4096 bins between min and
//      max (monotone, so the bin order is the value order); an LDS histogram
//      gives the bin B1 holding the k-th largest;
//   3. keys above B1 go straight into an LDS bitmap over positions (a quad's
//      4 keys form a nibble, eight lanes OR theirs into a 32-bit word); the
//      keys of bin B1 go to a short list (position and key);
//   4. the winners of bin B1 are decided exactly (pairwise ranks for a short
//      list, radix passes on the 32-bit key and then on positions otherwise)
//      and added to the bitmap;
//   5. one ordered scan over the bitmap writes the k positions.
// Longer rows stream from global memory.  Rows of 16384..131072 keys with
// k <= 2048 first try one read (select_row_sampled): a systematic sample in
// linear bins over its own range gives a threshold that about 1.5 k keys
// reach, one pass collects the keys at or above it (ballot-compacted into
// LDS), and when at least k and at most kCandCap were collected the exact
// selection runs on them (select_candidates: linear bins over their range,
// the threshold bin's keys ranked or radix-selected, the bitmap, the ordered
// scan).  Otherwise, and for other rows:
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
//   Rows whose candidates exceed LDS capacity (very many equal keys) or whose
//   length exceeds the bitmap use multi-pass global refinement and a global
//   ordered compaction instead.
// Every path selects the same set.
#pragma once

#include "device_common.cuh"

namespace idx {

constexpr int kD1Bins = 4096;
constexpr int kD1Shift = 20;
constexpr int kCandCap = 4096;
constexpr int kBitmapWords = 4096;  // bitmap path for rows up to 131072 keys
constexpr int kRankCap = 256;       // threshold-bin keys ranked pairwise
constexpr int kRowCap = 32768;      // keys of an LDS-resident row

// The 512-thread instantiation is the streaming-only kernel (no register
// path): its second-digit histogram shares the union below with the first
// digit's histogram and the bitmap, which are never live at the same time on
// the streaming path, so that three of its workgroups fit a CU's LDS.
template <int NT>
struct SelectShared {
  static constexpr bool kShareHist2 = NT == 512;
  struct {
    uint32_t ckey[kCandCap];
    int cidx[kCandCap];
  } c;
  union {
    int hist1[kD1Bins];          // first-digit histogram (when not given)
    uint32_t sel[kBitmapWords];  // winners, one bit per position
    int hist2s[2048];            // second-digit histogram (streaming-only kernel)
  } u;
  int hist2o[kShareHist2 ? 1 : 2048];
  int scan[NT / kWave];
  int bc[8];
  __device__ __forceinline__ int* hist2() { return kShareHist2 ? u.hist2s : hist2o; }
};

struct SelectState {
  uint32_t prefix;
  uint32_t pmask;
  int need;  // elements equal (under pmask) to prefix still to take
};

// Streaming loads.  No load may sit under a lane-dependent branch: both
// sides of such a branch run, they share registers, and the compiler then
// waits for every earlier load before each one -- one memory round trip per
// load instead of all of them in flight together.  The form is chosen by
// conditions that are the same on every lane.

// The keys base + 4 (c NT + tid) + e (c < V, e < 4) of a row of L >= 1
// keys, keys past L read as `pad`.  A 16-byte aligned row is read in 16-byte
// quads at clamped quad positions (the 1..3 keys after the row's last whole
// quad come from three loads every lane makes alike); an unaligned row key
// by key, one quad's four loads at a time.
template <int V, int NT>
__device__ __forceinline__ void load_quads(const float* __restrict__ row, int base, int L, bool aligned, float pad,
                                           float (&f)[4 * V]) {
  const int tid = threadIdx.x;
  if (aligned && base + 4 * V * NT <= L) {  // every quad whole
#pragma unroll
    for (int c = 0; c < V; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(row + base + 4 * (c * NT + tid));
      f[4 * c] = x.x;
      f[4 * c + 1] = x.y;
      f[4 * c + 2] = x.z;
      f[4 * c + 3] = x.w;
    }
  } else if (aligned && L >= 4) {
    const int Lq = L & ~3;  // keys [0, Lq) form whole quads
    const float t0 = row[Lq < L ? Lq : L - 1];
    const float t1 = row[Lq + 1 < L ? Lq + 1 : L - 1];
    const float t2 = row[Lq + 2 < L ? Lq + 2 : L - 1];
#pragma unroll
    for (int c = 0; c < V; ++c) {
      const int i0 = base + 4 * (c * NT + tid);  // a multiple of 4, as is Lq
      const float4 x = *reinterpret_cast<const float4*>(row + (i0 + 4 <= Lq ? i0 : Lq - 4));
      const float xe[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        const int d = i - Lq;
        const float tail = d == 0 ? t0 : (d == 1 ? t1 : t2);
        f[4 * c + e] = i < Lq ? xe[e] : (i < L ? tail : pad);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < V; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = base + 4 * (c * NT + tid) + e;
        const float x = row[i < L ? i : L - 1];
        f[4 * c + e] = i < L ? x : pad;
      }
      // this quad's loads complete before the next quad's are issued, so
      // that the unrolled loads do not all hold address registers at once
      __asm__ volatile("" : "+v"(f[4 * c]), "+v"(f[4 * c + 1]), "+v"(f[4 * c + 2]), "+v"(f[4 * c + 3]));
    }
  }
}

// Loads keys [i0, i0 + 4*V) of a row into registers (contiguous per lane),
// all V loads in flight together: `whole` (the same on every lane) says
// that every lane's keys lie in the row and the row is 16-byte aligned;
// otherwise each key is loaded from a clamped position (L >= 1), one quad
// at a time, and the keys past L are flagged.
template <int V>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int i0, int L, bool whole,
                                          uint32_t (&u)[4 * V], bool (&v)[4 * V]) {
  float f[4 * V];
  if (whole) {
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
    for (int c = 0; c < V; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 4 * c + e;
        v[4 * c + e] = i < L;
        const float x = row[i < L ? i : L - 1];
        f[4 * c + e] = i < L ? x : 0.0f;
      }
      __asm__ volatile("" : "+v"(f[4 * c]), "+v"(f[4 * c + 1]), "+v"(f[4 * c + 2]), "+v"(f[4 * c + 3]));
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
  load_quads<V, NT>(row, base, L, aligned, 0.0f, f);
#pragma unroll
  for (int j = 0; j < 4 * V; ++j) {
    v[j] = base + 4 * ((j / 4) * NT + tid) + (j % 4) < L;
    u[j] = ordered_key(f[j]);
  }
}

template <int NT>
__device__ __forceinline__ int strided_pos(int base, int j) {
  return base + 4 * ((j / 4) * NT + static_cast<int>(threadIdx.x)) + (j % 4);
}

// Finds the digit bin holding the need-th largest element among `nbins`
// bins read through `bin(d)`; returns (digit, count above it, count in it).
// Without the trailing barrier the caller must not write sm.bc[0..2] or
// sm.scan before its next barrier.
template <int NT, bool kTrailingSync = true, class BinFn>
__device__ __forceinline__ void find_digit(int nbins, int need, BinFn bin, SelectShared<NT>& sm, int& digit,
                                           int& above_out, int& cnt_out) {
  const int tid = threadIdx.x;
  const int per = nbins / NT;
  const int hi = nbins - tid * per;
  if (tid == 0) {  // a defined result even when fewer than `need` elements are binned
    sm.bc[0] = 0;
    sm.bc[1] = 0;
    sm.bc[2] = 0;
  }
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
  if (kTrailingSync) __syncthreads();
}

// d1 histogram of a row into sm.u.hist1.
template <int NT>
__device__ __forceinline__ void row_histogram(const float* __restrict__ row, int L, bool aligned, SelectShared<NT>& sm) {
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

// One radix step: among the elements whose key matches st.prefix under
// st.pmask, histogram digit (key >> shift) & (2^bits - 1) and narrow st to
// the digit holding the st.need-th largest.  `for_each(fn)` visits the key
// of every element to consider and is called by all threads.  Returns the
// number of elements in the chosen digit (equal to the updated st.need when
// that digit is taken whole).
template <int NT, class ForEach>
__device__ __forceinline__ int refine_pass(SelectState& st, int shift, int bits, ForEach for_each, SelectShared<NT>& sm) {
  const int tid = threadIdx.x;
  const int nb = 1 << bits;
  const uint32_t dmask = static_cast<uint32_t>(nb - 1);
  for (int j = tid; j < nb; j += NT) sm.hist2()[j] = 0;
  __syncthreads();
  const uint32_t prefix = st.prefix, pmask = st.pmask;
  for_each([&](uint32_t key) {
    if ((key & pmask) == prefix) atomicAdd(&sm.hist2()[(key >> shift) & dmask], 1);
  });
  __syncthreads();
  int digit, above, cnt;
  if (nb >= NT) {
    find_digit<NT>(nb, st.need, [&](int d) { return sm.hist2()[d]; }, sm, digit, above, cnt);
  } else {
    // fewer bins than threads: pad the digit space to NT bins
    find_digit<NT>(NT, st.need, [&](int d) { return d < nb ? sm.hist2()[d] : 0; }, sm, digit, above, cnt);
  }
  st.prefix |= static_cast<uint32_t>(digit) << shift;
  st.pmask |= dmask << shift;
  st.need -= above;
  return cnt;
}

// Two radix steps (the second skipped when the first digit is taken whole).
template <int NT, class ForEach>
__device__ __forceinline__ int refine(SelectState& st, int shift0, int bits0, int shift1, int bits1, ForEach for_each,
                      SelectShared<NT>& sm) {
  int cnt = refine_pass<NT>(st, shift0, bits0, for_each, sm);
  if (st.need != cnt) cnt = refine_pass<NT>(st, shift1, bits1, for_each, sm);
  return cnt;
}

// Ordered compaction straight from the global row (fallback path).
template <int NT>
__device__ __forceinline__ void compact_global(const float* __restrict__ row, int L, int k, bool aligned, const SelectState& st,
                               int* __restrict__ out, SelectShared<NT>& sm) {
  const int tid = threadIdx.x;
  int run_sel = 0, run_eq = 0;
  constexpr int V = 2;
  for (int base = 0; base < L && run_sel < k; base += NT * 4 * V) {
    const int i0 = base + tid * 4 * V;
    uint32_t u[4 * V];
    bool v[4 * V];
    load_keys<V>(row, i0, L, aligned && base + NT * 4 * V <= L, u, v);
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

// Appends every key of the row at or above `lo_key` (with its position) to
// the LDS candidate list, at most kCandCap of them; returns how many there
// are (also when more than fit).  Per-thread counts, one wave scan and one
// reservation per wave and chunk; order irrelevant.
template <int NT>
__device__ __forceinline__ int collect_candidates(const float* __restrict__ row, int L, bool aligned,
                                                  uint32_t lo_key, SelectShared<NT>& sm) {
  if (threadIdx.x == 0) sm.bc[4] = 0;
  __syncthreads();
  constexpr int V = 8;
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
          sm.c.ckey[pos] = u[j];
          sm.c.cidx[pos] = strided_pos<NT>(base, j);
        }
        ++pos;
      }
    }
  }
  __syncthreads();
  return sm.bc[4];
}

// Steps 4 and 5 of a streamed row whose `nc` candidates (every key of the
// top k among them) are in LDS and whose threshold state `st` has been
// refined to the digit holding the k-th largest (n_eq keys match it): the
// winners go to a position bitmap (those equal to the threshold key, when
// not all are taken, by lowest position), then one ordered scan writes the k
// positions.  Needs L <= kBitmapWords * 32.
template <int NT>
__device__ __forceinline__ void finish_candidates(int L, int k, const SelectState& st, int n_eq, int nc,
                                                  int* __restrict__ out, SelectShared<NT>& sm) {
  const int tid = threadIdx.x;
  const int W = (L + 31) >> 5;
  const bool take_all_eq = st.need == n_eq;
  const uint32_t tprefix = st.prefix, tmask = st.pmask;
  // keys equal to the threshold, when not all are taken: the `need` lowest
  // positions among them, i.e. the largest of (2^17 - 1 - position), by radix
  // select on 17 bits (before the bitmap: the second-digit histogram may
  // share its memory)
  SelectState ts{0u, 0u, st.need};
  if (!take_all_eq) {
    refine<NT>(ts, 8, 9, 0, 8, [&](auto fn) {
      for (int i = tid; i < nc; i += NT)
        if ((sm.c.ckey[i] & tmask) == tprefix) fn(0x1FFFFu - static_cast<uint32_t>(sm.c.cidx[i]));
    }, sm);
  }
  for (int j = tid; j < W; j += NT) sm.u.sel[j] = 0u;
  __syncthreads();
  for (int i = tid; i < nc; i += NT) {
    const uint32_t m = sm.c.ckey[i] & tmask;
    const int p = sm.c.cidx[i];
    const bool win = m > tprefix ||
                     (m == tprefix && (take_all_eq || (0x1FFFFu - static_cast<uint32_t>(p)) >= ts.prefix));
    if (win) atomicOr(&sm.u.sel[p >> 5], 1u << (p & 31));
  }
  __syncthreads();

  // ordered emission
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

// Linear bins over a value range [lo, hi]: bin(v) = clamp(fma(v, a, b), 0,
// kD1Bins - 1) truncated, with a = kD1Bins / (hi - lo) and b = -lo a: one
// rounding of (v - lo) a, so monotone non-decreasing in v.  (hi - lo is
// formed from halves so that it cannot overflow; when a or b is not finite
// every value goes to bin 0, which is slow but still exact.)
struct LinearBins {
  float a, b;
  __device__ __forceinline__ static LinearBins over(float lo, float hi) {
    const float half_range = hi * 0.5f - lo * 0.5f;
    float a = half_range > 0.0f ? static_cast<float>(kD1Bins / 2) / half_range : 0.0f;
    float b = -(lo * a);
    if (!(__builtin_fabsf(a) <= 3.0e38f) || !(__builtin_fabsf(b) <= 3.0e38f)) a = b = 0.0f;
    return {a, b};
  }
  __device__ __forceinline__ float raw(float v) const { return __builtin_fmaf(v, a, b); }
  __device__ __forceinline__ int bin(float v) const {
    return static_cast<int>(__builtin_amdgcn_fmed3f(raw(v), 0.0f, static_cast<float>(kD1Bins - 1)));
  }
};

// The V float4 quads q = c NT + tid (c < V) of the chunk at `base` (V
// loads in flight together; each load instruction of a wave covers 1 KiB of
// consecutive keys); element j of the thread is position
// base + 4 (j / 4 NT + tid) + j % 4, or -inf past the row's end.
template <int V, int NT>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int base, int L, bool aligned,
                                           float (&f)[4 * V]) {
  load_quads<V, NT>(row, base, L, aligned, -__builtin_inff(), f);
}

// Appends every key of the row that passes `test` (monotone in the value,
// false for -inf) to the LDS candidate list as (float bits, position), at
// most kCandCap of them; returns how many there are (also when more than
// fit).  Per chunk, each wave counts its passing keys with ballots,
// reserves that many slots at once and writes its keys at ballot offsets;
// the loads of the next chunk are in flight while a chunk is tested.  The
// caller has requested the first two chunks (collect_chunk_keys keys per
// lane each, load_chunk) into fa and fb.
template <int NT>
constexpr int collect_chunk_keys() { return NT == 512 ? 16 : 32; }

template <int NT, class Test>
__device__ __forceinline__ int collect_by(const float* __restrict__ row, int L, bool aligned, Test test,
                                          SelectShared<NT>& sm, float (&fa)[collect_chunk_keys<NT>()],
                                          float (&fb)[collect_chunk_keys<NT>()]) {
  if (threadIdx.x == 0) sm.bc[4] = 0;
  __syncthreads();
  constexpr int V = collect_chunk_keys<NT>() / 4;
  constexpr int kStep = NT * 4 * V;
  const int lane = lane_id();
  auto process = [&](const float (&f)[4 * V], int base) {
    // one ballot per key slot; the writes below take their lanes from the
    // same masks (as exec), not from a second evaluation of the test
    uint64_t mk[4 * V];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 4 * V; ++j) {
      mk[j] = __ballot(test(f[j]));
      cnt += __popcll(mk[j]);
    }
    int wbase = 0;
    if (lane == 0 && cnt > 0) wbase = atomicAdd(&sm.bc[4], cnt);
    wbase = __builtin_amdgcn_readfirstlane(wbase);
    if (wbase + cnt <= kCandCap) {  // (else the list is full: counted only)
      const int pbase = base + 4 * static_cast<int>(threadIdx.x);
#pragma unroll
      for (int j = 0; j < 4 * V; ++j) {
        const uint64_t m = mk[j];
        if (m) {
          if (__builtin_amdgcn_inverse_ballot_w64(m)) {
            const int off = wbase + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                        static_cast<uint32_t>(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
            sm.c.ckey[off] = __float_as_uint(f[j]);
            sm.c.cidx[off] = pbase + 4 * NT * (j / 4) + (j % 4);
          }
          wbase += __popcll(m);
        }
      }
    }
  };
  // two register buffers in turn: a chunk's loads are in flight while the
  // chunk before it is tested
  for (int base = 0; base < L; base += 2 * kStep) {
    process(fa, base);
    if (base + kStep >= L) break;
    if (base + 2 * kStep < L) load_chunk<V, NT>(row, base + 2 * kStep, L, aligned, fa);
    process(fb, base + kStep);
    if (base + 3 * kStep < L) load_chunk<V, NT>(row, base + 3 * kStep, L, aligned, fb);
  }
  __syncthreads();
  return sm.bc[4];
}

// Exact top k of a row from its `nc` candidates in LDS (float bits and
// positions; every key of the row's top k is among them, k <= nc <=
// kCandCap): linear bins over the candidates' range give the bin B1 holding
// the k-th largest; candidates above it win, and the `need` winners of bin
// B1 are decided on the exact key (rank against each other when few, radix
// passes otherwise), ties to the lower position.  Winners go to an LDS
// position bitmap and one ordered scan writes the k positions.  Needs
// L <= kBitmapWords * 32.
template <int NT>
__device__ __forceinline__ void select_candidates(int L, int k, int nc, int* __restrict__ out, SelectShared<NT>& sm) {
  constexpr int CPT = kCandCap / NT;  // candidates per thread: i = tid + NT c
  static_assert(kRankCap <= NT, "a rank verdict per thread");
  const int tid = threadIdx.x;
  float cv[CPT];
  int cp[CPT];
  float lo = __builtin_inff(), hi = -__builtin_inff();
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int i = tid + NT * c;
    cv[c] = i < nc ? __uint_as_float(sm.c.ckey[i]) : 0.0f;
    cp[c] = i < nc ? sm.c.cidx[i] : -1;
    if (i < nc) {
      lo = fminf(lo, cv[c]);
      hi = fmaxf(hi, cv[c]);
    }
  }
  __syncthreads();  // the list is in registers: its LDS is free
  for (int j = tid; j < kD1Bins; j += NT) sm.u.hist1[j] = 0;
  block_min_max<NT>(lo, hi, sm.c.cidx);  // (its barrier also publishes the cleared bins)
  const LinearBins lb = LinearBins::over(lo, hi);
  int bn[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    bn[c] = cp[c] >= 0 ? lb.bin(cv[c]) : -1;
    if (bn[c] >= 0) atomicAdd(&sm.u.hist1[bn[c]], 1);
  }
  __syncthreads();
  if (tid == 0) sm.bc[4] = 0;  // eq-list counter, published by find_digit's barrier
  int B1, above1, m;
  find_digit<NT, false>(kD1Bins, k, [&](int d) { return sm.u.hist1[d]; }, sm, B1, above1, m);
  const int need = k - above1;  // keys of bin B1 to take
  // keys of bin B1 -> the front of the (free) candidate area, exact keys
  uint32_t* eq_key = sm.c.ckey;
  int* eq_pos = sm.c.cidx;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    if (bn[c] == B1) {
      const int slot = atomicAdd(&sm.bc[4], 1);
      eq_key[slot] = ordered_key(cv[c]);
      eq_pos[slot] = cp[c];
    }
  }
  __syncthreads();

  // the `need` winners of bin B1, decided before the bitmap exists (the
  // second-digit histogram may share its memory): all of them, a rank
  // verdict per thread (few keys: entry tid), or a radix rule on (key,
  // position)
  const bool take_all = need == m;
  bool rank_win = false;
  SelectState st{0u, 0u, need};
  SelectState ts{0u, 0u, 0};
  bool rule_all_eq = true;
  if (!take_all) {
    if (m <= kRankCap) {
      if (tid < m) {
        const uint32_t ki = eq_key[tid];
        const int pi = eq_pos[tid];
        int rank = 0;
        for (int u = 0; u < m; ++u) {
          const uint32_t ku = eq_key[u];
          rank += (ku > ki || (ku == ki && eq_pos[u] < pi)) ? 1 : 0;
        }
        rank_win = rank < need;
      }
    } else {
      auto in_bin = [&](auto fn) {
        for (int i = tid; i < m; i += NT) fn(eq_key[i]);
      };
      int n_eq = refine_pass<NT>(st, 21, 11, in_bin, sm);
      if (st.need != n_eq) n_eq = refine_pass<NT>(st, 10, 11, in_bin, sm);
      if (st.need != n_eq) n_eq = refine_pass<NT>(st, 0, 10, in_bin, sm);
      rule_all_eq = st.need == n_eq;
      if (!rule_all_eq) {
        // keys equal to the threshold: the `need` lowest positions among
        // them, i.e. the largest of (2^17 - 1 - position)
        ts.need = st.need;
        const uint32_t prefix = st.prefix, pmask = st.pmask;
        refine<NT>(ts, 8, 9, 0, 8, [&](auto fn) {
          for (int i = tid; i < m; i += NT)
            if ((eq_key[i] & pmask) == prefix) fn(0x1FFFFu - static_cast<uint32_t>(eq_pos[i]));
        }, sm);
      }
    }
  }
  const int W = (L + 31) >> 5;
  uint32_t* bits = sm.u.sel;
  __syncthreads();  // every histogram read is done: the bitmap may take the memory
  for (int j = tid; j < W; j += NT) bits[j] = 0u;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CPT; ++c)
    if (bn[c] > B1) atomicOr(&bits[cp[c] >> 5], 1u << (cp[c] & 31));
  if (take_all) {
    for (int i = tid; i < m; i += NT) atomicOr(&bits[eq_pos[i] >> 5], 1u << (eq_pos[i] & 31));
  } else if (m <= kRankCap) {
    if (rank_win) atomicOr(&bits[eq_pos[tid] >> 5], 1u << (eq_pos[tid] & 31));
  } else {
    const uint32_t prefix = st.prefix, pmask = st.pmask;
    for (int i = tid; i < m; i += NT) {
      const uint32_t mk = eq_key[i] & pmask;
      const int pi = eq_pos[i];
      const bool win = mk > prefix ||
                       (mk == prefix && (rule_all_eq || (0x1FFFFu - static_cast<uint32_t>(pi)) >= ts.prefix));
      if (win) atomicOr(&bits[pi >> 5], 1u << (pi & 31));
    }
  }
  __syncthreads();

  // ordered emission: thread t owns bitmap words [t wpt, (t + 1) wpt)
  const int wpt = (W + NT - 1) / NT;
  const int w0 = tid * wpt;
  const int w1 = (w0 + wpt < W) ? w0 + wpt : W;
  int c_sel = 0;
  for (int wd = w0; wd < w1; ++wd) c_sel += __popc(bits[wd]);
  int tot;
  int o = block_exclusive_scan<NT>(c_sel, tot, sm.scan);
  for (int wd = w0; wd < w1; ++wd) {
    uint32_t sel = bits[wd];
    while (sel) {
      const int bpos = __builtin_ctz(sel);
      sel &= sel - 1u;
      if (o < k) out[o] = wd * 32 + bpos;
      ++o;
    }
  }
  __syncthreads();
}

// Rows this long (and of at most kBitmapWords * 32 keys) with k at most
// kSampleMaxK first try one read (the candidate window [k, kCandCap] around
// the expected 1.5 k keeps a fallback rare):
constexpr int kSampleMinLen = 16384;
constexpr int kSampleMaxK = 2048;

// One-read selection of a streamed row: a systematic sample (every S-th
// 64-key block, at most kCandCap keys) in linear bins over its own range
// gives the bin holding its ceil(1.5 k / S)-th largest value, i.e. a
// threshold that about 1.5 k of the row's keys reach; one pass collects every
// key at or above it (a test monotone in the value).  When that holds at
// least k and at most kCandCap keys, every key of the top k is among them
// (the top k are >= the k-th largest, which passes the test since at least k
// keys do) and the exact selection runs on them; otherwise (a skewed sample,
// heavy ties) nothing is written and the caller takes the two-read path.
// Returns whether it finished the row (the same on every thread).
//
// sample_threshold is its first part: the sample, its bins and the bin B0;
// the keys to collect are those with lb.raw(v) >= t0.  It also requests
// the first collection chunk of the keys (crow, cL) into fa, after the
// sample's own loads.  Returns false (the same on every thread) when the
// sample gives no threshold.  Its result depends on the row only, so
// workgroups that collect different parts of one row agree on it.
template <int NT>
__device__ __forceinline__ bool sample_threshold(const float* __restrict__ row, int L, int k, bool aligned,
                                                 const float* __restrict__ crow, int cL,
                                                 float (&fa)[collect_chunk_keys<NT>()], SelectShared<NT>& sm,
                                                 LinearBins& lb_out, float& t0_out) {
  const int tid = threadIdx.x;
  const int nb = L >> 6;                                  // full 64-key blocks
  const int S = (nb + 63) / 64 > 16 ? (nb + 63) / 64 : 16;   // stride: >= 16, and <= 64 sampled blocks
  const int ns_blocks = (nb + S - 1) / S;
  const int ns = ns_blocks * 64;                         // <= 64 * 64 = kCandCap keys
  static_assert(64 * 64 <= kCandCap, "the sample must fit the candidate area");
  const int r = (3 * k + 2 * S - 1) / (2 * S);            // ceil(1.5 k / S)
  if (r < 1 || r > ns) return false;
  // the sample's quads (at most kCandCap / 4 of them, CQ per thread) are
  // requested first and the collection's first chunk right after, so that
  // it is in flight while the sample is binned (its second chunk, requested
  // here too, measured no better)
  constexpr int CQ = (kCandCap / 4 + NT - 1) / NT;
  float sv[CQ][4];
#pragma unroll
  for (int c = 0; c < CQ; ++c) {
    // lanes past the sample load its last quad again (unused), so that no
    // load sits under a lane-dependent branch
    const int qi = tid + NT * c < ns_blocks * 16 ? tid + NT * c : ns_blocks * 16 - 1;
    const int pos = (qi >> 4) * S * 64 + (qi & 15) * 4;
    if (aligned) {
      const float4 x = *reinterpret_cast<const float4*>(row + pos);
      sv[c][0] = x.x; sv[c][1] = x.y; sv[c][2] = x.z; sv[c][3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[c][e] = row[pos + e];
    }
  }
  constexpr int V = collect_chunk_keys<NT>() / 4;
  load_chunk<V, NT>(crow, 0, cL, aligned, fa);
  float lo = __builtin_inff(), hi = -__builtin_inff();
#pragma unroll
  for (int c = 0; c < CQ; ++c) {
    const int qi = tid + NT * c;
    if (qi < ns_blocks * 16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.c.ckey[4 * qi + e] = __float_as_uint(sv[c][e]);
        lo = fminf(lo, sv[c][e]);
        hi = fmaxf(hi, sv[c][e]);
      }
    }
  }
  for (int j = tid; j < kD1Bins; j += NT) sm.u.hist1[j] = 0;
  block_min_max<NT>(lo, hi, sm.c.cidx);  // (its barrier also publishes the sample and the cleared bins)
  const LinearBins lb = LinearBins::over(lo, hi);
  if (!(lb.a > 0.0f)) return false;  // one value, or an infinite range: the two-read path
  for (int i = tid; i < ns; i += NT) atomicAdd(&sm.u.hist1[lb.bin(__uint_as_float(sm.c.ckey[i]))], 1);
  __syncthreads();
  int B0, above0, cnt0;
  find_digit<NT>(kD1Bins, r, [&](int d) { return sm.u.hist1[d]; }, sm, B0, above0, cnt0);
  // keys whose unclamped bin value reaches B0: monotone in the value, and
  // every sample key of bin B0 and above passes
  lb_out = lb;
  t0_out = static_cast<float>(B0);
  return true;
}

template <int NT>
__device__ __forceinline__ bool select_row_sampled(const float* __restrict__ row, int L, int k, bool aligned,
                                                   int* __restrict__ out, SelectShared<NT>& sm) {
  constexpr int V = collect_chunk_keys<NT>() / 4;
  constexpr int kStep = NT * 4 * V;
  float fa[4 * V], fb[4 * V];
  LinearBins lb;
  float t0;
  if (!sample_threshold<NT>(row, L, k, aligned, row, L, fa, sm, lb, t0)) return false;
  if (kStep < L) load_chunk<V, NT>(row, kStep, L, aligned, fb);
  const int nc = collect_by<NT>(row, L, aligned, [&](float v) { return lb.raw(v) >= t0; }, sm, fa, fb);
  if (nc < k || nc > kCandCap) return false;
  select_candidates<NT>(L, k, nc, out, sm);
  return true;
}

// Top-k of a row streamed from global memory (k < L); try_sampled = false
// skips the one-read attempt (known to fail).
template <int NT>
__device__ __forceinline__ void select_row_stream(const float* __restrict__ row, int L, int k, int* __restrict__ out,
                                  SelectShared<NT>& sm, bool try_sampled = true) {
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  if (try_sampled && L >= kSampleMinLen && L <= kBitmapWords * 32 && k <= kSampleMaxK &&
      select_row_sampled<NT>(row, L, k, aligned, out, sm))
    return;

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

  // 2. candidates (d1 >= B1) -> LDS
  const int nc = collect_candidates<NT>(row, L, aligned, static_cast<uint32_t>(B1) << kD1Shift, sm);

  // 3. exact threshold among the candidates of bin B1
  int n_eq = cnt1;
  if (st.need != cnt1) {
    n_eq = refine<NT>(st, 10, 10, 0, 10, [&](auto fn) {
      for (int i = threadIdx.x; i < nc; i += NT) fn(sm.c.ckey[i]);
    }, sm);
  }

  // 4, 5. winners -> position bitmap -> ordered emission
  finish_candidates<NT>(L, k, st, n_eq, nc, out, sm);
}

// Top-k of a row held in registers (k < L <= kRowCap).  Thread t holds
// keys t + NT j, j < E.  The first digit is linear in the value between the
// row's minimum and maximum (monotone, so any such digit works), which
// spreads the keys over the 4096 bins instead of crowding them into the few
// exponent bins the key's top bits would give; the exact 32-bit key only
// decides within the threshold bin.
template <int NT, int E>
__device__ __forceinline__ void select_row_reg(const float* __restrict__ row, int L, int k, int* __restrict__ out,
                               SelectShared<NT>& sm) {
  static_assert(E % 4 == 0, "keys per thread come in quads");
  constexpr int EQ = E / 4;  // quads per thread: quad q = tid + NT j holds keys 4q .. 4q + 3
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int nq = ((L + 3) / 4 + NT - 1) / NT;  // quad slots in use (uniform)
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;

  // 1. load (all loads in flight at once; 16-byte loads for whole quads of
  //    an aligned row, clamped 4-byte loads otherwise) and the row's range
  float x[E];
#pragma unroll
  for (int j = 0; j < EQ; ++j) {
    if (j < nq) {
      const int p0 = 4 * (tid + NT * j);
      if (aligned && p0 + 4 <= L) {
        const float4 v = *reinterpret_cast<const float4*>(row + p0);
        x[4 * j] = v.x;
        x[4 * j + 1] = v.y;
        x[4 * j + 2] = v.z;
        x[4 * j + 3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * j + e] = row[p0 + e < L ? p0 + e : L - 1];
      }
    }
  }
  float lo = __builtin_inff(), hi = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < EQ; ++j) {
    if (j < nq) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo = fminf(lo, x[4 * j + e]);
        hi = fmaxf(hi, x[4 * j + e]);
      }
    }
  }
  for (int j = tid; j < kD1Bins; j += NT) sm.u.hist1[j] = 0;
  block_min_max<NT>(lo, hi, sm.hist2());  // hist2 is free until the exact resolution
  // bin(v) = clamp(fma(v, a, b), 0, 4095) truncated, with a = 4096 / (hi - lo)
  // and b = -lo a: one rounding of (v - lo) a, so monotone non-decreasing in
  // v.  (hi - lo is formed from halves so that it cannot overflow; when a or
  // b is not finite every key goes to bin 0, which is slow but still exact.)
  const float half_range = hi * 0.5f - lo * 0.5f;
  float a = half_range > 0.0f ? static_cast<float>(kD1Bins / 2) / half_range : 0.0f;
  float b = -(lo * a);
  if (!(__builtin_fabsf(a) <= 3.0e38f) || !(__builtin_fabsf(b) <= 3.0e38f)) a = b = 0.0f;

  // 2. first-digit histogram (bins kept; -1 marks slots past L) and the bin
  //    B1 holding the k-th largest
  int bn[E];
#pragma unroll
  for (int j = 0; j < EQ; ++j) {
    if (j < nq) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = 4 * (tid + NT * j) + e;
        const int v = static_cast<int>(
            __builtin_amdgcn_fmed3f(__builtin_fmaf(x[4 * j + e], a, b), 0.0f, static_cast<float>(kD1Bins - 1)));
        bn[4 * j + e] = p < L ? v : -1;
        if (p < L) atomicAdd(&sm.u.hist1[v], 1);
      }
    }
  }
  __syncthreads();
  int B1, above1, cnt1;
  if (tid == 0) sm.bc[4] = 0;  // eq-list counter, published by find_digit's barrier
  find_digit<NT, false>(kD1Bins, k, [&](int d) { return sm.u.hist1[d]; }, sm, B1, above1, cnt1);
  if (cnt1 > kCandCap) {
    // too many keys in the threshold bin (large ties): radix-select from
    // global memory
    __syncthreads();  // every thread has read find_digit's result
    select_row_stream<NT>(row, L, k, out, sm);
    return;
  }

  // 3. winners above bin B1 straight into the position bitmap: the 4 keys
  //    of a quad give a nibble, the 8 quads of a 32-position word sit in 8
  //    consecutive lanes (q % 8 == lane % 8), and an OR over those lanes
  //    gives the word, stored by its first lane.  Keys in bin B1 go to a
  //    short list (positions only) for the exact decision.
  uint32_t* bits = sm.u.sel;  // hist1 is dead once B1 is known (every thread has passed find_digit's barrier)
  int* eq_pos = sm.c.cidx;
  uint32_t* eq_key = sm.c.ckey;
  const int need = k - above1;  // keys of bin B1 to take
#pragma unroll
  for (int j = 0; j < EQ; ++j) {
    if (j < nq) {
      const int q = tid + NT * j;
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gt |= (bn[4 * j + e] > B1 ? 1u : 0u) << e;
        eq |= (bn[4 * j + e] == B1 ? 1u : 0u) << e;
      }
      uint32_t w = gt << (4 * (lane & 7));
      w |= __builtin_amdgcn_update_dpp(0u, w, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
      w |= __builtin_amdgcn_update_dpp(0u, w, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
      w |= __builtin_amdgcn_update_dpp(0u, w, 0x141, 0xF, 0xF, false);  // row_half_mirror
      if ((lane & 7) == 0) bits[q >> 3] = w;
      while (eq) {
        const int e = __builtin_ctz(eq);
        eq &= eq - 1u;
        const float v = e == 0 ? x[4 * j] : e == 1 ? x[4 * j + 1] : e == 2 ? x[4 * j + 2] : x[4 * j + 3];
        const int slot = atomicAdd(&sm.bc[4], 1);
        if (slot < kCandCap) {
          eq_pos[slot] = 4 * q + e;
          eq_key[slot] = ordered_key(v);
        }
      }
    }
  }
  __syncthreads();
  const int m = cnt1;

  // 4. the `need` winners of bin B1: largest exact key, ties to the lowest
  //    position.  Few keys: rank each against all; more: radix passes.
  if (need == m) {
    for (int i = tid; i < m; i += NT) atomicOr(&bits[eq_pos[i] >> 5], 1u << (eq_pos[i] & 31));
  } else if (m <= kRankCap) {
    for (int i = tid; i < m; i += NT) {
      const uint32_t ki = eq_key[i];
      const int pi = eq_pos[i];
      int rank = 0;
      for (int u = 0; u < m; ++u) {
        const uint32_t ku = eq_key[u];
        rank += (ku > ki || (ku == ki && eq_pos[u] < pi)) ? 1 : 0;
      }
      if (rank < need) atomicOr(&bits[pi >> 5], 1u << (pi & 31));
    }
  } else {
    SelectState st{0u, 0u, need};
    auto in_bin = [&](auto fn) {
      for (int i = tid; i < m; i += NT) fn(eq_key[i]);
    };
    int n_eq = refine_pass<NT>(st, 21, 11, in_bin, sm);
    if (st.need != n_eq) n_eq = refine_pass<NT>(st, 10, 11, in_bin, sm);
    if (st.need != n_eq) n_eq = refine_pass<NT>(st, 0, 10, in_bin, sm);
    const bool take_all_eq = st.need == n_eq;
    const uint32_t prefix = st.prefix, pmask = st.pmask;
    for (int i = tid; i < m; i += NT) {
      const uint32_t mk = eq_key[i] & pmask;
      if (mk > prefix || (take_all_eq && mk == prefix)) atomicOr(&bits[eq_pos[i] >> 5], 1u << (eq_pos[i] & 31));
    }
    if (!take_all_eq) {
      // keys equal to the threshold: the `need` lowest positions among them,
      // i.e. the largest of (2^17 - 1 - position), by radix select on 17 bits
      SelectState ts{0u, 0u, st.need};
      auto tied = [&](auto fn) {
        for (int i = tid; i < m; i += NT)
          if ((eq_key[i] & pmask) == prefix) fn(0x1FFFFu - static_cast<uint32_t>(eq_pos[i]));
      };
      refine<NT>(ts, 8, 9, 0, 8, tied, sm);
      for (int i = tid; i < m; i += NT) {
        const int pi = eq_pos[i];
        if ((eq_key[i] & pmask) == prefix && (0x1FFFFu - static_cast<uint32_t>(pi)) >= ts.prefix)
          atomicOr(&bits[pi >> 5], 1u << (pi & 31));
      }
    }
  }
  __syncthreads();
  const int W = (L + 31) >> 5;

  // 5. ordered emission: thread t owns bitmap words [t wpt, (t + 1) wpt)
  const int wpt = (W + NT - 1) / NT;
  const int w0 = tid * wpt;
  const int w1 = (w0 + wpt < W) ? w0 + wpt : W;
  int c_sel = 0;
  for (int wd = w0; wd < w1; ++wd) c_sel += __popc(bits[wd]);
  int tot;
  int o = block_exclusive_scan<NT>(c_sel, tot, sm.scan);
  for (int wd = w0; wd < w1; ++wd) {
    uint32_t sel = bits[wd];
    while (sel) {
      const int bpos = __builtin_ctz(sel);
      sel &= sel - 1u;
      if (o < k) out[o] = wd * 32 + bpos;  // never more than k, whatever the input bits
      ++o;
    }
  }
  __syncthreads();
}

// Top-k of one row.  kReg = false leaves the register path out (every row
// longer than k streams from memory), for a lean kernel that fits several
// workgroups per CU.
template <int NT, bool kReg = true>
__device__ __forceinline__ void select_row(const float* __restrict__ row, int L, int k, int* __restrict__ out, SelectShared<NT>& sm) {
  static_assert(!(kReg && SelectShared<NT>::kShareHist2), "the register path needs its own second-digit histogram");
  if (L <= k) {
    for (int j = threadIdx.x; j < k; j += NT) out[j] = (j < L) ? j : -1;
  } else if (kReg && L <= kRowCap) {
    select_row_reg<NT, kRowCap / NT>(row, L, k, out, sm);
  } else {
    select_row_stream<NT>(row, L, k, out, sm);
  }
}

}  // namespace idx
