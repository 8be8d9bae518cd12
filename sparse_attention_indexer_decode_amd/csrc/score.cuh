// Paged indexer scorer for gfx950:
//   logit[r, t] = scale_t * sum_h w[r,h] * relu(q[r,h,:] . code_t)   (t < L_r)
//
// Work decomposition.  Rows are bundled into "groups" of up to RG rows that
// share one request (the next_n decode rows of a request, or consecutive
// query rows of a prefill request); a group reads the pages of its request
// once for all its rows.  The pages of all groups form one global list
// (prefix sums in LDS, rebuilt by every workgroup from the device lengths, so
// the host never reads device data); each workgroup takes a contiguous slice
// of that list and its four waves take every fourth page of the slice.
//
// Per page (64 keys) a wave: copies the page's token rows into its LDS
// buffer with 16-byte loads (issued one page ahead into registers), decodes
// its B fragments (32 keys per 32x32x16 MFMA) from LDS to bf16, and runs
// bf16 MFMAs against query fragments held in registers for the whole group.
//
// Precision.  Every e4m3 code and every e2m1 value times its power-of-two
// MX block scale is exactly a bf16, and q is bf16, so the products are
// exact and the MFMA accumulates them in fp32.  (The fp8 f8f6f4 MFMA of
// gfx950 was measured to sum its products to about 1e-5 of sum|products|,
// too coarse for 1e-4 absolute logits after the head sum cancels; the bf16
// MFMA sums to ~5e-8, like sequential fp32.  Issued work is the same as an
// exact two-term fp8 split of q would need.)  The fp8 per-token scale
// multiplies the head sum (scale_t >= 0 commutes with relu).
//
// Operand layout (32x32x16 bf16): lane l holds A row / B column l % 32 and
// 8 consecutive k of block l / 32.  Lane block g carries key dims
// [g*D/2, g*D/2 + D/2) over the D/16 k-steps (8 dims per step); A uses the
// same dims, so the contraction covers all D.  Accumulator lane l, register
// v: key l % 32, head 8 (v / 4) + 4 (l / 32) + v % 4, so the head sum is 16
// in-lane terms per M-tile plus one swap of the lane halves.
#pragma once

#include "device_common.cuh"
#include "select.cuh"

namespace idx {

struct ScoreParams {
  CacheArgs cache;
  RowArgs rows;
  const uint16_t* q;
  const float* w;
  int32_t heads;
  int32_t k;              // fused mode: top-k
  float* logits;          // row r at logits + r * logits_stride (+ column base)
  int64_t logits_stride;
  int32_t* out;           // fused mode: [rows, k]
  int32_t* counters;      // fused mode: per-group completion counters
  uint32_t* status;
  int32_t num_groups;     // host bound on groups (table size)
};

template <int D, bool MX>
struct Geometry {
  static constexpr int kRowBytes = MX ? (D / 2 + D / 32) : (D + 4);
  static constexpr int kPageBytes = kPage * kRowBytes;
  static constexpr int kChunks = (kPageBytes / 16 + kWave - 1) / kWave;  // 16-B loads per lane
  static constexpr int kKSteps = D / 16;  // 32x32x16 steps over the head dim
};

template <int D, bool MX, int RG>
struct ScoreShared {
  int gprefix[kMaxGroups + 1];
  int req_tab[4][kMaxReqPrefill + 1];  // prefill: groups, rows, columns, first query; decode: packed offsets
  float wbuf[4][RG][kMaxHeads];
  int misc[8];
  union {
    uint8_t page[4][Geometry<D, MX>::kPageBytes];
    SelectShared<256> sel;
  } u;
};

struct GroupDesc {
  int b;         // request
  int nrows;     // rows in the group
  int row0;      // output row of the first row (grid row or chunk row)
  int row_step;  // output row stride between the group's rows (1)
  int col0;      // logits column base (prefill ks)
  int Lmax;
};

// ---------------------------------------------------------------------------
// Group tables (built by every workgroup in LDS)
// ---------------------------------------------------------------------------

template <int RG>
__device__ __forceinline__ int groups_per_request(int next_n) {
  return (next_n + RG - 1) / RG;
}

// Rows of group g and their lengths.  L[rho] = 0 marks an empty row slot.
template <int RG>
__device__ __forceinline__ GroupDesc describe_group(const ScoreParams& p, const int (*req_tab)[kMaxReqPrefill + 1],
                                                    int g, int (&L)[RG], int (&qrow)[RG]) {
  GroupDesc d;
  const RowArgs& R = p.rows;
  if (R.kind == 0) {
    const int gpr = groups_per_request<RG>(R.next_n);
    const int b = g / gpr;
    const int j = g - b * gpr;
    int seq = R.seq_lens[b];
    seq = seq > R.max_len ? R.max_len : seq;
    const int dl = R.decode_lens ? R.decode_lens[b] : R.next_n;
    d.b = b;
    d.row0 = b * R.next_n + j * RG;
    d.row_step = 1;
    d.col0 = 0;
    d.nrows = 0;
    d.Lmax = 0;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int i = j * RG + r;
      const bool exists = i < R.next_n;
      L[r] = exists ? decode_row_len(seq, dl, i, R.max_len) : 0;
      qrow[r] = (exists && i < dl) ? (R.q_packed ? req_tab[0][b] + i : b * R.next_n + i) : -1;
      d.nrows += exists ? 1 : 0;
      d.Lmax = L[r] > d.Lmax ? L[r] : d.Lmax;
    }
  } else {
    // binary search: last b with groups_before[b] <= g
    int lo = 0, hi = R.num_req;  // invariant tab[lo] <= g < tab[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (req_tab[0][mid] <= g) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int gi = g - req_tab[0][b];
    const int rows_b = req_tab[1][b + 1] - req_tab[1][b];
    const int first_row = req_tab[1][b] + gi * RG;
    const int j0 = req_tab[3][b] + gi * RG;
    int seq = R.seq_lens[b];
    seq = seq > R.max_len ? R.max_len : seq;
    const int qlen = R.qsl[b + 1] - R.qsl[b];
    d.b = b;
    d.row0 = first_row;
    d.row_step = 1;
    d.col0 = req_tab[2][b];
    d.nrows = rows_b - gi * RG < RG ? rows_b - gi * RG : RG;
    d.Lmax = 0;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const bool exists = r < d.nrows;
      int Lr = seq - qlen + j0 + r + 1;
      Lr = Lr < 0 ? 0 : (Lr > seq ? seq : Lr);
      L[r] = exists ? Lr : 0;
      qrow[r] = exists ? first_row + r : -1;
      d.Lmax = L[r] > d.Lmax ? L[r] : d.Lmax;
    }
  }
  return d;
}

// Fills sm.gprefix[0..NG] (page prefix over groups) and the request tables;
// returns NG.  Called by all 256 threads.
template <int RG, bool kFused, class SM>
__device__ int build_group_tables(const ScoreParams& p, SM& sm) {
  const RowArgs& R = p.rows;
  const int tid = threadIdx.x;
  int NG;
  if (R.kind == 0) {
    NG = R.num_req * groups_per_request<RG>(R.next_n);
    if (R.q_packed) {
      // exclusive prefix of decode_lens -> packed token offsets
      int run = 0;
      for (int base = 0; base < R.num_req; base += 256) {
        const int b = base + tid;
        const int v = (b < R.num_req) ? (R.decode_lens ? R.decode_lens[b] : R.next_n) : 0;
        int tot;
        const int ex = block_exclusive_scan<256>(v, tot, sm.misc);
        if (b < R.num_req) sm.req_tab[0][b] = run + ex;
        run += tot;
      }
      __syncthreads();
    }
  } else {
    // per request: rows of the chunk slice, groups, column base, first query index
    const int q0 = R.qsl[0];
    int run_g = 0, run_r = 0, run_c = 0;
    for (int base = 0; base < R.num_req; base += 256) {
      const int b = base + tid;
      int rows_b = 0, cols_b = 0, first_j = 0;
      if (b < R.num_req) {
        const int s = R.qsl[b] - q0, e = R.qsl[b + 1] - q0;
        const int lo = s > R.q_begin ? s : R.q_begin;
        const int hi = e < R.q_end ? e : R.q_end;
        rows_b = hi > lo ? hi - lo : 0;
        first_j = lo - s;
        int seq = R.seq_lens[b];
        cols_b = seq > R.max_len ? R.max_len : (seq < 0 ? 0 : seq);
      }
      const int gr = (rows_b + RG - 1) / RG;
      int tg, tr, tc;
      const int eg = block_exclusive_scan<256>(gr, tg, sm.misc);
      const int er = block_exclusive_scan<256>(rows_b, tr, sm.misc);
      const int ec = block_exclusive_scan<256>(cols_b, tc, sm.misc);
      if (b < R.num_req) {
        sm.req_tab[0][b] = run_g + eg;
        sm.req_tab[1][b] = run_r + er;
        sm.req_tab[2][b] = run_c + ec;
        sm.req_tab[3][b] = first_j;
      }
      run_g += tg;
      run_r += tr;
      run_c += tc;
    }
    if (tid == 0) {
      sm.req_tab[0][R.num_req] = run_g;
      sm.req_tab[1][R.num_req] = run_r;
      sm.req_tab[2][R.num_req] = run_c;
    }
    __syncthreads();
    NG = run_g;
  }
  // page prefix over groups
  int run = 0;
  for (int base = 0; base < NG; base += 256) {
    const int g = base + tid;
    int np = 0;
    if (g < NG) {
      int L[RG], qr[RG];
      GroupDesc d = describe_group<RG>(p, sm.req_tab, g, L, qr);
      np = (d.Lmax + kPage - 1) / kPage;
      if (kFused && d.Lmax <= p.k) np = 0;  // causal fill only, nothing to score
    }
    int tot;
    const int ex = block_exclusive_scan<256>(np, tot, sm.misc);
    if (g < NG) sm.gprefix[g] = run + ex;
    run += tot;
  }
  if (tid == 0) sm.gprefix[NG] = run;
  __syncthreads();
  return NG;
}

// ---------------------------------------------------------------------------
// Query fragments (a wave loads the A operands of one group)
// ---------------------------------------------------------------------------

template <int D, int RG, int MT>
struct QFrag {
  v8bf a[RG][MT][D / 16];
};

template <int D, int RG, int MT>
__device__ __forceinline__ void prepare_query(const ScoreParams& p, const int (&qrow)[RG],
                                              QFrag<D, RG, MT>& f, float (*wbuf)[kMaxHeads]) {
  const int lane = lane_id();
  const int m = lane & 31;
  const int g = lane >> 5;
#pragma unroll
  for (int r = 0; r < RG; ++r) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = 32 * mt + m;
      const bool valid = qrow[r] >= 0 && h < p.heads;
      const uint4* src = reinterpret_cast<const uint4*>(
          p.q + (static_cast<int64_t>(valid ? qrow[r] : 0) * p.heads + (valid ? h : 0)) * D + g * (D / 2));
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const uint4 v = valid ? src[s] : make_uint4(0, 0, 0, 0);
        f.a[r][mt][s] = __builtin_bit_cast(v8bf, v);
      }
      if (g == 0) wbuf[r][h] = valid ? p.w[static_cast<int64_t>(qrow[r]) * p.heads + h] : 0.0f;
    }
    if (MT == 1 && lane < 32) wbuf[r][32 + lane] = 0.0f;
  }
}

// 2^(e - 127) as an fp32 (e = 0 is the subnormal 2^-127, e = 255 is NaN).
__device__ __forceinline__ float ue8m0_to_float(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : e << 23));
}

// B fragments of one key (this lane's half of its dims) decoded to bf16.
template <int D, bool MX>
__device__ __forceinline__ void key_fragments(const uint8_t* rowp, int g, v8bf (&b)[D / 16]) {
  if (MX) {
    // D = 128: packed bytes [32 g, 32 g + 32) = blocks 2g, 2g+1 (dims 64 g ..)
    const uint32_t* w32 = reinterpret_cast<const uint32_t*>(rowp + 32 * g);
    const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(rowp + D / 2 + 2 * g);
    const float sc[2] = {ue8m0_to_float(sc2 & 0xFFu), ue8m0_to_float(sc2 >> 8)};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint32_t x = w32[s];
      const float f = sc[s / 4];
      const v2bf e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, f, 0);
      const v2bf e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, f, 1);
      const v2bf e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, f, 2);
      const v2bf e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, f, 3);
      b[s] = v8bf{e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
    }
  } else {
    const uint32_t* w32 = reinterpret_cast<const uint32_t*>(rowp + g * (D / 2));
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint32_t x0 = w32[2 * s], x1 = w32[2 * s + 1];
      const v2bf e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, false);
      const v2bf e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, true);
      const v2bf e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, false);
      const v2bf e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, true);
      b[s] = v8bf{e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
    }
  }
}

// ---------------------------------------------------------------------------
// The scorer kernel
// ---------------------------------------------------------------------------

template <int D, bool MX, int RG, int MT, bool kFused>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
  using Geo = Geometry<D, MX>;
  constexpr int KS = Geo::kKSteps;
  constexpr int RB = Geo::kRowBytes;
  __shared__ ScoreShared<D, MX, RG> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  const int NG = build_group_tables<RG, kFused>(p, sm);
  const int P = sm.gprefix[NG];

  // Fused: rows of groups that need no scoring are written here.
  if (kFused) {
    for (int gg = blockIdx.x; gg < NG; gg += gridDim.x) {
      if (sm.gprefix[gg + 1] != sm.gprefix[gg]) continue;
      int L[RG], qr[RG];
      GroupDesc d = describe_group<RG>(p, sm.req_tab, gg, L, qr);
      for (int r = 0; r < d.nrows; ++r) {
        int32_t* o = p.out + static_cast<int64_t>(d.row0 + r) * p.k;
        for (int j = tid; j < p.k; j += 256) o[j] = (j < L[r]) ? j : -1;
      }
    }
  }

  const int64_t G = gridDim.x;
  const int r0 = static_cast<int>((static_cast<int64_t>(P) * blockIdx.x) / G);
  const int r1 = static_cast<int>((static_cast<int64_t>(P) * (blockIdx.x + 1)) / G);

  uint8_t* buf = sm.u.page[wave];
  float(*wbuf)[kMaxHeads] = sm.wbuf[wave];

  QFrag<D, RG, MT> qf;
  int L[RG], qrow[RG];
  GroupDesc gd;
  gd.b = -1;
  int cur_g = -1;

  // group containing page r0 + wave: last gi with gprefix[gi] <= page
  // (groups without pages share their prefix with the next group; the walk
  // below steps over them)
  int gi = 0;
  if (r0 + wave < r1) {
    int lo = 0, hi = NG;
    const int target = r0 + wave;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm.gprefix[mid] <= target) lo = mid; else hi = mid;
    }
    gi = lo;
  }

  uint4 stage[Geo::kChunks];

  // physical page of global page index `pgl` in group `grp` (descriptor d)
  auto issue_load = [&](int pgl, const GroupDesc& d, int grp) {
    const int pg = pgl - sm.gprefix[grp];
    const int phys = p.rows.block_table[static_cast<int64_t>(d.b) * p.rows.bt_stride + pg];
    const bool ok = phys >= 0 && static_cast<int64_t>(phys) < p.cache.num_pages;
    if (!ok && lane == 0) atomicOr(p.status, 1u);
    const uint4* src = reinterpret_cast<const uint4*>(p.cache.base + static_cast<int64_t>(ok ? phys : 0) * p.cache.page_bytes);
#pragma unroll
    for (int c = 0; c < Geo::kChunks; ++c) {
      const int idx16 = c * kWave + lane;
      stage[c] = (ok && idx16 < Geo::kPageBytes / 16) ? src[idx16] : make_uint4(0, 0, 0, 0);
    }
  };

  int pg_cur = r0 + wave;
  GroupDesc nd;
  int nd_g = -1;
  int ndL[RG], ndq[RG];
  if (pg_cur < r1) {
    while (pg_cur >= sm.gprefix[gi + 1]) ++gi;
    nd = describe_group<RG>(p, sm.req_tab, gi, ndL, ndq);
    nd_g = gi;
    issue_load(pg_cur, nd, gi);
  }

  for (; pg_cur < r1; pg_cur += 4) {
    // the group of the current page is (nd, nd_g)
    if (nd_g != cur_g) {
      cur_g = nd_g;
      gd = nd;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        L[r] = ndL[r];
        qrow[r] = ndq[r];
      }
      prepare_query<D, RG, MT>(p, qrow, qf, wbuf);
    }
    const int pg_in_group = pg_cur - sm.gprefix[cur_g];

    // stage -> LDS
#pragma unroll
    for (int c = 0; c < Geo::kChunks; ++c) {
      const int idx16 = c * kWave + lane;
      if (idx16 < Geo::kPageBytes / 16) reinterpret_cast<uint4*>(buf)[idx16] = stage[c];
    }
    __builtin_amdgcn_wave_barrier();

    // prefetch the next page of this wave
    const int pg_next = pg_cur + 4;
    if (pg_next < r1) {
      while (pg_next >= sm.gprefix[gi + 1]) ++gi;
      if (gi != nd_g) {
        nd = describe_group<RG>(p, sm.req_tab, gi, ndL, ndq);
        nd_g = gi;
      }
      issue_load(pg_next, nd, gi);
    }

#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int key = nt * 32 + n;
      const uint8_t* rowp = buf + key * RB;
      v8bf bfr[KS];
      key_fragments<D, MX>(rowp, g, bfr);
      float key_scale = 1.0f;
      if (!MX) key_scale = *reinterpret_cast<const float*>(rowp + D);

#pragma unroll
      for (int r = 0; r < RG; ++r) {
        float partial = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          v16f acc = {};
#pragma unroll
          for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf.a[r][mt][s], bfr[s], acc, 0, 0, 0);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const float4 wv = *reinterpret_cast<const float4*>(&wbuf[r][32 * mt + 8 * i4 + 4 * g]);
            partial += wv.x * fmaxf(acc[4 * i4 + 0], 0.0f);
            partial += wv.y * fmaxf(acc[4 * i4 + 1], 0.0f);
            partial += wv.z * fmaxf(acc[4 * i4 + 2], 0.0f);
            partial += wv.w * fmaxf(acc[4 * i4 + 3], 0.0f);
          }
        }
        const float total = (partial + __shfl_xor(partial, 32, kWave)) * key_scale;
        const int t = pg_in_group * kPage + key;
        if (g == 0 && r < gd.nrows && t < L[r]) {
          const int64_t row = gd.row0 + r;
          p.logits[row * p.logits_stride + gd.col0 + t] = total;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  if (!kFused) return;

  // ---- fused top-k: the workgroup that completes a group selects its rows
  __threadfence();
  __syncthreads();
  if (r0 >= r1) return;
  int glo, ghi;
  {
    int lo = 0, hi = NG;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm.gprefix[mid] <= r0) lo = mid; else hi = mid;
    }
    glo = lo;
    lo = 0;
    hi = NG;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm.gprefix[mid] <= r1 - 1) lo = mid; else hi = mid;
    }
    ghi = lo;
  }
  for (int gg = glo; gg <= ghi; ++gg) {
    const int a0 = sm.gprefix[gg], a1 = sm.gprefix[gg + 1];
    if (a1 == a0) continue;
    const int c = (r1 < a1 ? r1 : a1) - (r0 > a0 ? r0 : a0);
    if (c <= 0) continue;
    if (tid == 0) {
      const int old = atomicAdd(&p.counters[gg], c);
      const int last = (old + c == a1 - a0) ? 1 : 0;
      if (last) p.counters[gg] = 0;
      sm.misc[0] = last;
    }
    __syncthreads();
    const int last = sm.misc[0];
    __syncthreads();
    if (!last) continue;
    __threadfence();
    int Lg[RG], qg[RG];
    GroupDesc d = describe_group<RG>(p, sm.req_tab, gg, Lg, qg);
    for (int r = 0; r < d.nrows; ++r) {
      const int64_t row = d.row0 + r;
      select_row<256>(p.logits + row * p.logits_stride, Lg[r], p.k, p.out + row * p.k, sm.u.sel);
      __syncthreads();
    }
  }
}

}  // namespace idx
