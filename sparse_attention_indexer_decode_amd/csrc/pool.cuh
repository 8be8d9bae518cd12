// Pool-level (block-level) top-k of rows of logits: one workgroup per row.
//
// The pool variant of the indexer (pool_topk, then expand_pools_and_append_tail
// on the glm5next sparse_indexer page; topk_blocks / init_blocks /
// local_blocks of the MiniMax-M3 mono runner page's indexer).  Reading: a
// pool is B = 2^pool_log2 consecutive key positions; a row of L keys has
// n = L / B complete pools and a tail of L - n B keys; a pool scores the
// largest logit of its keys; the first init and the last local complete
// pools are always kept and count toward topk; the other places go to the
// highest-scoring complete pools, ties to the lower pool index (-0.0 equal to
// +0.0); every complete pool is kept when n <= topk.  Output: the kept pools'
// positions ascending, then the tail, -1 padded to (topk + 1) B per row;
// optionally the kept pool indices, ascending, -1 padded to topk.
//
// Per row: (1) pool maxima of the candidate pools -> order-preserving keys in
// LDS (B / 4 lanes per pool, one float4 each, a shuffle max); (2) exact radix
// select of the free places over the keys (four 8-bit digits, LDS histogram,
// the digit found by one wave scan), ties at the threshold resolved by rank
// in pool order (a block scan); (3) kept pools as an LDS bitmap, ranked by a
// block scan of its words into an ascending pool list; (4) coalesced output:
// entry i of the row is pool list[i / B] position i % B, then the tail.
#pragma once

#include "device_common.cuh"
#include "topk.cuh"

namespace idx {

constexpr int kPoolThreads = 512;
constexpr int kMaxPools = 8192;     // complete pools of one row
constexpr int kMaxPoolTopk = 512;   // pools kept per row

struct PoolParams {
  const float* logits;
  int64_t stride;
  RowArgs rows;
  int32_t pool_log2;    // pool size 16, 32, 64 or 128
  int32_t topk;         // pools kept per row
  int32_t init_pools;
  int32_t local_pools;
  int32_t* out_tokens;  // [rows][(topk + 1) << pool_log2]
  int32_t* out_pools;   // [rows][topk] or null
};

template <int NT>
struct PoolShared {
  uint32_t key[kMaxPools];         // candidate pools' maxima as ordered keys
  uint32_t sel[kMaxPools / 32];    // kept pools, one bit each
  int list[kMaxPoolTopk];          // kept pools in ascending order
  int hist[256];
  int scan[NT / kWave];
  int misc[4];
};

// Digit of the `need`-th largest key among those counted in hist (wave 0
// only; lane l owns bins 255 - 4l .. 252 - 4l): misc[0] = digit, misc[1] =
// keys in higher bins.
__device__ __forceinline__ void top_digit(const int* hist, int need, int* misc) {
  const int lane = lane_id();
  int c[4], tot = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = hist[255 - 4 * lane - j];
    tot += c[j];
  }
  const int incl = wave_inclusive_scan(tot);
  int run = incl - tot;
  if (run < need && need <= incl) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (run + c[j] >= need) {
        misc[0] = 255 - 4 * lane - j;
        misc[1] = run;
        break;
      }
      run += c[j];
    }
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void pool_topk_kernel(PoolParams p) {
  __shared__ PoolShared<NT> sm;
  __shared__ int info[2];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  int L, col0;
  row_window<NT>(p.rows, r, L, col0, sm.scan, info);
  const int lg = p.pool_log2;
  const int B = 1 << lg;
  const int W = (p.topk + 1) << lg;
  int32_t* out = p.out_tokens + static_cast<int64_t>(r) * W;
  int32_t* pout = p.out_pools ? p.out_pools + static_cast<int64_t>(r) * p.topk : nullptr;
  const int n_full = L >> lg;
  const int tail0 = n_full << lg;

  if (n_full <= p.topk) {
    // every complete pool, then the tail: exactly the positions 0 .. L - 1
    for (int i = tid; i < W; i += NT) out[i] = i < L ? i : -1;
    if (pout)
      for (int i = tid; i < p.topk; i += NT) pout[i] = i < n_full ? i : -1;
    return;
  }

  const int a = p.init_pools < n_full ? p.init_pools : n_full;
  const int z = p.local_pools < n_full - a ? p.local_pools : n_full - a;
  const int e = n_full - z;
  const int n = e - a;             // candidate pools [a, e)
  const int free = p.topk - a - z; // their places (n > free >= 0)
  const int nw = (n_full + 31) >> 5;
  for (int i = tid; i < nw; i += NT) {
    // kept-by-position pools [0, a) and [e, n_full)
    uint32_t m = 0;
    const int p0 = i << 5;
#pragma unroll 4
    for (int b = 0; b < 32; ++b) {
      const int q = p0 + b;
      m |= (q < n_full && (q < a || q >= e)) ? (1u << b) : 0u;
    }
    sm.sel[i] = m;
  }

  if (free > 0) {
    // (1) pool maxima of the candidates
    const float* row = p.logits + static_cast<int64_t>(r) * p.stride + col0;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    const int lpp = B >> 2;                  // lanes per pool
    const int gpw = kWave / lpp;             // pools per wave and step
    const int g = lane / lpp;
    const int sub = lane - g * lpp;
    // kBatch steps' loads in flight together; lanes past the last pool load
    // it again (no load under a lane-dependent branch, which would cost a
    // round trip per load) and store nothing
    constexpr int kBatch = 8;
    const int step = (NT / kWave) * gpw;
    for (int c0 = wave * gpw; c0 < n; c0 += kBatch * step) {  // wave-uniform trip count
      float v[kBatch][4];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int c = c0 + t * step + g;
        const float* src = row + (static_cast<int64_t>(a + (c < n ? c : n - 1)) << lg) + 4 * sub;
        if (aligned) {
          const float4 x = *reinterpret_cast<const float4*>(src);
          v[t][0] = x.x; v[t][1] = x.y; v[t][2] = x.z; v[t][3] = x.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[t][e] = src[e];
        }
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int c = c0 + t * step + g;
        float m = fmaxf(fmaxf(v[t][0], v[t][1]), fmaxf(v[t][2], v[t][3]));
        for (int d = lpp >> 1; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
        if (c < n && sub == 0) sm.key[c] = ordered_key(m);
      }
    }
    __syncthreads();

    // (2) radix select of the `free` largest keys
    uint32_t prefix = 0, mask = 0;
    int need = free;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t k = sm.key[i];
        if ((k & mask) == prefix) atomicAdd(&sm.hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      if (wave == 0) top_digit(sm.hist, need, sm.misc);
      __syncthreads();
      need -= sm.misc[1];
      prefix |= static_cast<uint32_t>(sm.misc[0]) << shift;
      mask |= 0xFFu << shift;
      __syncthreads();  // misc is rewritten by the next pass
    }
    // keys above the threshold, and the `need` lowest pools equal to it
    const int chunk = (n + NT - 1) / NT;
    const int i0 = tid * chunk;
    const int i1 = i0 + chunk < n ? i0 + chunk : n;
    int eq = 0;
    for (int i = i0; i < i1; ++i) eq += sm.key[i] == prefix ? 1 : 0;
    int tot;
    int rank = block_exclusive_scan<NT>(eq, tot, sm.scan);
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = sm.key[i];
      bool take = k > prefix;
      if (k == prefix) take = rank++ < need;
      if (take) atomicOr(&sm.sel[(a + i) >> 5], 1u << ((a + i) & 31));
    }
  }
  __syncthreads();

  // (3) kept pools in ascending order
  {
    const int wpt = (nw + NT - 1) / NT;
    const int w0 = tid * wpt;
    const int w1 = w0 + wpt < nw ? w0 + wpt : nw;
    int cnt = 0;
    for (int wd = w0; wd < w1; ++wd) cnt += __popc(sm.sel[wd]);
    int tot;
    int pos = block_exclusive_scan<NT>(cnt, tot, sm.scan);
    for (int wd = w0; wd < w1; ++wd) {
      uint32_t bits = sm.sel[wd];
      while (bits) {
        const int b = __builtin_ctz(bits);
        bits &= bits - 1u;
        sm.list[pos++] = (wd << 5) + b;
      }
    }
  }
  __syncthreads();

  // (4) the kept pools' positions, the tail, -1 padding (p.topk pools kept)
  const int kept = p.topk;
  const int tail_end = (kept << lg) + (L - tail0);
  for (int i = tid; i < W; i += NT) {
    int v = -1;
    if (i < (kept << lg)) v = (sm.list[i >> lg] << lg) + (i & (B - 1));
    else if (i < tail_end) v = tail0 + (i - (kept << lg));
    out[i] = v;
  }
  if (pout)
    for (int i = tid; i < p.topk; i += NT) pout[i] = sm.list[i];
}

}  // namespace idx
