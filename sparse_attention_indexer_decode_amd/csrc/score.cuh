// Paged indexer scorer for gfx950:
//   logit[r, t] = scale_t * sum_h w[r,h] * relu(q[r,h,:] . code_t)   (t < L_r)
//
// Two kernels share the helpers below: score_kernel for decode rows and
// score_block_kernel (at the end of this file) for prefill rows.
//
// Work decomposition.  Rows are bundled into "groups" that share one
// request: a decode group is one row (the next_n rows of a request are
// scored by different waves that run at the same time, so a page's second
// read mostly hits the caches), a prefill group is up to eight consecutive
// query rows that read the request's pages once.  Every workgroup (one per
// CU) builds the prefix of pages over groups in LDS from the device lengths
// (the host never reads them); the global page list is then cut into equal
// contiguous ranges, one per wave (decode) or one per workgroup (prefill).
//
// Decode memory pipeline.  Each wave streams its pages through a ring of NP
// (2-4) pages in LDS filled by direct global->LDS loads
// (global_load_lds_dwordx4, 1 KiB per instruction): while page j is scored
// from one buffer, pages j+1 .. j+NP-1 are already in flight, and page j+NP
// is requested as soon as page j's buffer is consumed.  No staging
// registers are used, and the waits are explicit vmcnt counts (loads retire
// in order; every wait leaves exactly the loads issued after the page it
// needs outstanding).
//
// Per page (64 keys) a wave decodes its B fragments (32 keys per 32x32x16
// MFMA) from LDS to bf16 and runs bf16 MFMAs against query fragments held in
// registers.
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
//
#pragma once

#include "device_common.cuh"

namespace idx {

// Waves per decode workgroup (one workgroup per CU); every wave scores one
// row at a time.
constexpr int kDecodeWaves = 8;

struct ScoreParams {
  CacheArgs cache;
  RowArgs rows;
  const uint16_t* q;
  const float* w;
  int32_t heads;
  float* logits;          // row r at logits + r * logits_stride (+ column base)
  int64_t logits_stride;
  int32_t* header;        // workspace header: status word
  int32_t num_groups;     // decode: groups (prefill: derived on the device)
};

template <int D, bool MX>
struct Geometry {
  static constexpr int kRowBytes = MX ? (D / 2 + D / 32) : (D + 4);
  static constexpr int kPageBytes = kPage * kRowBytes;
  // A page moves to LDS as kWide 1 KiB loads (16 B per lane) plus kNarrow
  // 256 B loads (4 B per lane), exactly its bytes.
  static constexpr int kWide = kPageBytes / 1024;
  static constexpr int kNarrow = (kPageBytes % 1024) / 256;
  static constexpr int kLoads = kWide + kNarrow;
  static constexpr int kKSteps = D / 16;  // 32x32x16 steps
  static_assert(kPageBytes % 256 == 0, "page must split into 256-byte loads");
  static_assert(kLoads <= 15, "loads per page must fit a vmcnt immediate");
};

// Bytes of a row's query block staged in LDS (full 32-head tiles of 128
// dims only; see load_query_staged).
template <int D, int MT>
constexpr int query_stage_bytes() { return D == 128 ? MT * 32 * D * 2 : 0; }

// Pages in each wave's ring: as many as its LDS area holds (at least two,
// at most four), the area being sized for two pages or for the first group's
// staged queries, whichever is larger.
template <int D, bool MX, int MT>
constexpr int ring_pages() {
  constexpr int pb = Geometry<D, MX>::kPageBytes;
  constexpr int area = 2 * pb > query_stage_bytes<D, MT>() ? 2 * pb : query_stage_bytes<D, MT>();
  return area / pb > 4 ? 4 : area / pb;
}

// Each wave's LDS area: its page ring, which also stages the first group's
// queries before the first page is requested.
template <int D, bool MX, int MT>
union WaveArea {
  uint8_t page[ring_pages<D, MX, MT>()][Geometry<D, MX>::kPageBytes];
  uint8_t stage[query_stage_bytes<D, MT>() > 0 ? query_stage_bytes<D, MT>() : 16];
};

template <int D, bool MX, int MT, int NWV>
struct ScoreShared {
  int page_prefix[kMaxGroups + 1];     // pages before each group
  int req_tab[4][kMaxReqPrefill + 1];  // prefill: groups, rows, columns, first query; decode: packed offsets
  float wbuf[NWV][kMaxHeads];          // each wave's head weights on their way to registers
  int misc[16];
  alignas(16) WaveArea<D, MX, MT> area[NWV];
};

struct GroupDesc {
  int b;      // request
  int nrows;  // rows in the group
  int row0;   // output row of the first row (grid row or chunk row)
  int col0;   // logits column base (prefill ks)
  int Lmax;
};

template <int RG>
__device__ __forceinline__ int groups_per_request(int next_n) {
  return (next_n + RG - 1) / RG;
}

// Request of group g (decode: arithmetic; prefill: search of the LDS table).
template <int RG>
__device__ __forceinline__ int group_request(const RowArgs& R, const int (*req_tab)[kMaxReqPrefill + 1], int g) {
  if (R.kind == 0) return g / groups_per_request<RG>(R.next_n);
  int lo = 0, hi = R.num_req;  // last b with groups_before[b] <= g
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (req_tab[0][mid] <= g) lo = mid; else hi = mid;
  }
  return lo;
}

// Rows of group g: their key counts L (0 = empty slot), the q/w row each
// reads (qload, -1 = none) and whether the row is real (w is zeroed for
// padded decode slots, whose q row exists but must not count).
template <int RG>
__device__ __forceinline__ GroupDesc describe_group(const RowArgs& R, const int (*req_tab)[kMaxReqPrefill + 1],
                                                    int g, int b, int (&L)[RG], int (&qload)[RG],
                                                    bool (&real)[RG]) {
  GroupDesc d;
  d.b = b;
  d.Lmax = 0;
  d.nrows = 0;
  if (R.kind == 0) {
    const int j = g - b * groups_per_request<RG>(R.next_n);
    int seq = R.seq_lens[b];
    seq = seq > R.max_len ? R.max_len : seq;
    const int dl = R.decode_lens ? R.decode_lens[b] : R.next_n;
    d.row0 = b * R.next_n + j * RG;
    d.col0 = 0;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int i = j * RG + r;
      const bool exists = i < R.next_n;
      real[r] = exists && i < dl;
      L[r] = exists ? decode_row_len(seq, dl, i, R.max_len, R.ratio) : 0;
      if (R.q_packed) qload[r] = real[r] ? req_tab[0][b] + i : -1;
      else qload[r] = exists ? b * R.next_n + i : -1;
      d.nrows += exists ? 1 : 0;
      d.Lmax = L[r] > d.Lmax ? L[r] : d.Lmax;
    }
  } else {
    const int gi = g - req_tab[0][b];
    const int rows_b = req_tab[1][b + 1] - req_tab[1][b];
    const int first_row = req_tab[1][b] + gi * RG;
    const int j0 = req_tab[3][b] + gi * RG;
    int seq = R.seq_lens[b];
    seq = seq > R.max_len ? R.max_len : seq;
    const int qlen = R.qsl[b + 1] - R.qsl[b];
    d.row0 = first_row;
    d.col0 = req_tab[2][b];
    d.nrows = rows_b - gi * RG < RG ? rows_b - gi * RG : RG;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const bool exists = r < d.nrows;
      int Lr = seq - qlen + j0 + r + 1;
      Lr = Lr < 0 ? 0 : (Lr > seq ? seq : Lr);
      Lr = R.ratio == 1 ? Lr : Lr / R.ratio;
      L[r] = exists ? Lr : 0;
      real[r] = exists;
      qload[r] = exists ? first_row + r : -1;
      d.Lmax = L[r] > d.Lmax ? L[r] : d.Lmax;
    }
  }
  return d;
}

// Request tables in LDS: packed decode offsets, or (prefill) per request the
// groups/rows/columns before it and its first query index in the slice.
// Returns the number of groups (decode: num_req * groups per request).
template <int RG, int NT, class SM>
__device__ int build_request_tables(const RowArgs& R, SM& sm) {
  const int tid = threadIdx.x;
  if (R.kind == 0) {
    if (R.q_packed) {
      int run = 0;
      for (int base = 0; base < R.num_req; base += NT) {
        const int b = base + tid;
        const int v = (b < R.num_req) ? (R.decode_lens ? R.decode_lens[b] : R.next_n) : 0;
        int tot;
        const int ex = block_exclusive_scan<NT>(v, tot, sm.misc);
        if (b < R.num_req) sm.req_tab[0][b] = run + ex;
        run += tot;
      }
      __syncthreads();
    }
    return R.num_req * groups_per_request<RG>(R.next_n);
  }
  const int q0 = R.qsl[0];
  int run_g = 0, run_r = 0, run_c = 0;
  for (int base = 0; base < R.num_req; base += NT) {
    const int b = base + tid;
    int rows_b = 0, cols_b = 0, first_j = 0;
    if (b < R.num_req) {
      const int s = R.qsl[b] - q0, e = R.qsl[b + 1] - q0;
      const int lo = s > R.q_begin ? s : R.q_begin;
      const int hi = e < R.q_end ? e : R.q_end;
      rows_b = hi > lo ? hi - lo : 0;
      first_j = lo - s;
      const int seq = R.seq_lens[b];
      cols_b = request_keys(seq, R.max_len, R.ratio);
    }
    int tg, tr, tc;
    const int eg = block_exclusive_scan<NT>((rows_b + RG - 1) / RG, tg, sm.misc);
    const int er = block_exclusive_scan<NT>(rows_b, tr, sm.misc);
    const int ec = block_exclusive_scan<NT>(cols_b, tc, sm.misc);
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
  return run_g;
}

// ---------------------------------------------------------------------------
// Operand fragments
// ---------------------------------------------------------------------------

template <int D, int MT>
struct QFrag {
  v8bf a[MT][D / 16];
};

// A fragments of query row `qrow` (this lane: head 32 mt + lane % 32, dims
// [g D/2, g D/2 + D/2)).  A row (-1) or heads that do not exist read row 0 /
// head 0 instead (loads stay unconditional); their head weights are zero, so
// they add nothing.
template <int D, int MT>
__device__ __forceinline__ void load_query(const ScoreParams& p, int qrow, QFrag<D, MT>& f) {
  const int lane = lane_id();
  const int m = lane & 31;
  const int g = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = 32 * mt + m;
    const bool valid = qrow >= 0 && h < p.heads;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        p.q + (static_cast<int64_t>(valid ? qrow : 0) * p.heads + (valid ? h : 0)) * D + g * (D / 2));
#pragma unroll
    for (int s = 0; s < D / 16; ++s) f.a[mt][s] = __builtin_bit_cast(v8bf, src[s]);
  }
}

// The same fragments for D = 128 and heads = 32 MT, read through the wave's
// idle LDS area.  Loaded directly, each 16-byte fragment load of a wave
// touches 64 different 128-byte lines (32 heads x 2 lane halves).  Here
// direct global->LDS loads copy the group's query block into the area, each
// instruction 1 KiB of contiguous query (4 heads), and the fragments are
// read back from LDS.  Chunk c of head h (dims 8c .. 8c + 7) sits at 16-byte
// slot 16 h + (c ^ (h % 16) ^ ((h / 16) % 2)): the
// XOR keeps the 16 (or 32) lanes of each b128 fragment read on distinct
// bank groups.  The load writes lane l's 16 bytes to slot 64 i + l, so lane
// l fetches the chunk that belongs there, a permutation within the same
// 1 KiB.  Waits for every outstanding load before reading; the caller must
// not reuse the area before the reads have returned.
template <int D, int MT>
__device__ __forceinline__ void load_query_staged(const ScoreParams& p, int qrow, uint8_t* area, QFrag<D, MT>& f) {
  static_assert(D == 128, "staging assumes 16 chunks of 16 bytes per head");
  constexpr int kHeads = 32 * MT;
  constexpr int kLoads = kHeads * D * 2 / 1024;  // 1 KiB per load instruction
  const int lane = lane_id();
  auto swz = [](int h) { return (h & 15) ^ ((h >> 4) & 1); };
  const uint32_t base = lds_addr(area);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(p.q) + static_cast<int64_t>(qrow >= 0 ? qrow : 0) * kHeads * D * 2;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int h = 4 * i + lane / 16;
    const int c = (lane % 16) ^ swz(h);
    lds_dma16(src + (16 * h + c) * 16, base + 1024 * i);
  }
  wait_all_loads();
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  const lds_u32x4* st = (const lds_u32x4*)area;  // LDS accesses, whatever the compiler infers
  const int m = lane & 31;
  const int g = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int h = 32 * mt + m;
      f.a[mt][s] = __builtin_bit_cast(v8bf, st[16 * h + ((8 * g + s) ^ swz(h))]);
    }
}

// max(x, 0) in one instruction: as signed integers, negative floats
// (including -0.0) are below 0 and non-negative floats keep their order, so
// an integer max with 0 is the float ReLU (fmaxf would add a canonicalizing
// max in front of the MFMA result).
__device__ __forceinline__ float relu(float x) {
  const int i = __float_as_int(x);
  return __int_as_float(i > 0 ? i : 0);
}

// K-step s of one key's B fragment (this lane's 8 dims of the step) decoded
// to bf16: fp8 codes exactly, or e2m1 values times their MX block scale.
template <int D, bool MX>
__device__ __forceinline__ v8bf key_step(const uint8_t* rowp, int g, int s) {
  if (MX) {
    // D = 128: packed bytes [32 g, 32 g + 32) = blocks 2g, 2g+1 (dims 64 g ..)
    const uint32_t x = reinterpret_cast<const uint32_t*>(rowp + 32 * g)[s];
    // The scaled conversion takes its power-of-two scale from the fp32
    // exponent field alone (sign and mantissa ignored; byte 0 gives the
    // 2^-127 of the MX format, byte 255 NaN), so each ue8m0 byte of the pair
    // only has to be shifted into bits 23..30: one instruction per scale.
    const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(rowp + D / 2 + 2 * g);
    const float f = __uint_as_float(s < 4 ? sc2 << 23 : sc2 << 15);
    const u32x4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, f, 0)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, f, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, f, 2)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, f, 3))};
    return __builtin_bit_cast(v8bf, r);
  } else {
    const uint32_t* w32 = reinterpret_cast<const uint32_t*>(rowp + g * (D / 2));
    const uint32_t x0 = w32[2 * s], x1 = w32[2 * s + 1];
    const u32x4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, true))};
    return __builtin_bit_cast(v8bf, r);
  }
}

// B fragments of one key (this lane's half of its dims) decoded to bf16.
template <int D, bool MX>
__device__ __forceinline__ void key_fragments(const uint8_t* rowp, int g, v8bf (&b)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) b[s] = key_step<D, MX>(rowp, g, s);
}

// ---------------------------------------------------------------------------
// Direct global -> LDS page loads
// ---------------------------------------------------------------------------

// Requests 64-key unit `phys` (see page_ids) into the LDS buffer at byte
// address `lds`: byte i of the unit lands at lds + i.  Always issues exactly
// kLoads loads.  ONCE: the unit is read once per launch (non-temporal hint).
template <int D, bool MX, bool ONCE = false>
__device__ __forceinline__ void dma_page(const ScoreParams& p, int phys, uint32_t lds) {
  using Geo = Geometry<D, MX>;
  const int lane = lane_id();
  const int sh = p.cache.page_shift;
  const uint8_t* src = p.cache.base + static_cast<int64_t>(phys >> sh) * p.cache.page_bytes +
                       (phys & ((1 << sh) - 1)) * Geo::kPageBytes;
#pragma unroll
  for (int c = 0; c < Geo::kWide; ++c) {
    if constexpr (ONCE) lds_dma16_s_nt(src + 1024 * c, 16 * lane, lds + 1024 * c);
    else lds_dma16_s(src + 1024 * c, 16 * lane, lds + 1024 * c);
  }
#pragma unroll
  for (int c = 0; c < Geo::kNarrow; ++c) {
    if constexpr (ONCE) lds_dma4_s_nt(src + 1024 * Geo::kWide + 256 * c, 4 * lane, lds + 1024 * Geo::kWide + 256 * c);
    else lds_dma4_s(src + 1024 * Geo::kWide + 256 * c, 4 * lane, lds + 1024 * Geo::kWide + 256 * c);
  }
}

// Waits until a page has landed in LDS, given how many pages were requested
// after it (each page is exactly kLoads requests, and vector memory
// operations complete in issue order).
template <int D, bool MX>
__device__ __forceinline__ void wait_page_with_later(int later) {
  constexpr int n = Geometry<D, MX>::kLoads;
  if (later >= 3) wait_vmcnt<3 * n>();
  else if (later == 2) wait_vmcnt<2 * n>();
  else if (later == 1) wait_vmcnt<n>();
  else wait_all_loads();
}

// Head weights of a row as the accumulator layout needs them: lane half g,
// M-tile mt, register v -> head 32 mt + 8 (v / 4) + 4 g + v % 4.
template <int MT>
struct WFrag {
  float v[MT][16];
};

// Output of one row: a raw buffer over its L logits, so that stores of keys
// at or past L (and of the lane half that does not store) fall outside the
// buffer and are dropped by the hardware, with no branch around the store.
typedef __amdgpu_buffer_rsrc_t RowOut;

__device__ __forceinline__ RowOut row_out(float* base, int L) {
  // the descriptor lives in scalar registers: make its (wave-uniform)
  // fields visibly uniform
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(L > 0 ? L * 4 : 0);
  float* u = reinterpret_cast<float*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, n, 0x00020000);
}

// Weighted ReLU head sum of one accumulator tile into four partial sums
// (independent chains, so the FMAs do not wait on each other).
template <int MT>
__device__ __forceinline__ void head_sum(const v16f& acc, const WFrag<MT>& wf, int mt, float (&ps)[4]) {
#pragma unroll
  for (int v = 0; v < 16; ++v) ps[v % 4] += wf.v[mt][v] * relu(acc[v]);
}

// Logit of this lane's key from its four partial sums: add the other lane
// half's heads (v_permlane32_swap leaves lo + hi in both halves), times the
// fp8 token scale; stored through the row's buffer descriptor.
__device__ __forceinline__ void finish_key(const float (&ps)[4], float key_scale, const RowOut& out, int off) {
  const float partial = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(partial), __float_as_uint(partial), false, false);
  const float total = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * key_scale;
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(total), out, off, 0, 0);
}

// Raw scores of one row against 32-key tile nt of a raw page in LDS.
template <int D, bool MX, int MT>
__device__ __forceinline__ void tile_mfma_raw(const uint8_t* buf, int nt, const QFrag<D, MT>& qf, v16f (&acc)[MT],
                                              float& key_scale) {
  using Geo = Geometry<D, MX>;
  const int lane = lane_id();
  const uint8_t* rowp = buf + (nt * 32 + (lane & 31)) * Geo::kRowBytes;
  v8bf bfr[Geo::kKSteps];
  key_fragments<D, MX>(rowp, lane >> 5, bfr);
  key_scale = MX ? 1.0f : *reinterpret_cast<const float*>(rowp + D);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v16f{};
#pragma unroll
  for (int s = 0; s < Geo::kKSteps; ++s)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf.a[mt][s], bfr[s], acc[mt], 0, 0, 0);
}

// Logits of one 32-key tile from its raw scores; `off` is the byte offset
// of this lane's key in the row (out of range: nothing stored).
template <int MT>
__device__ __forceinline__ void tile_logits(const v16f (&acc)[MT], float key_scale, const WFrag<MT>& wf,
                                            const RowOut& out, int off) {
  float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) head_sum<MT>(acc[mt], wf, mt, ps);
  finish_key(ps, key_scale, out, (lane_id() >> 5) == 0 ? off : 0x7FFFFFF0);
}

// Weighted ReLU head sum of one 32-key tile into one partial per lane (this
// lane half's heads of key lane % 32), in two independent chains.
template <int MT>
__device__ __forceinline__ float tile_partial(const v16f (&acc)[MT], const WFrag<MT>& wf) {
  float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) head_sum<MT>(acc[mt], wf, mt, ps);
  return (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

// Logits of a page's 64 keys from the partials of its two tiles: one swap of
// lane halves (v_permlane32_swap: lanes 32..63 of the first operand with
// lanes 0..31 of the second) leaves tile 0's totals in lanes 0..31 and tile
// 1's in lanes 32..63, i.e. key `lane` of the page in lane `lane`; times that
// key's fp8 scale, stored at byte offset off + 4 lane (off: the page's first
// key in the row; out of range: nothing stored).
__device__ __forceinline__ void page_logits(float p0, float p1, float key_scale, const RowOut& out, int off) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  const float total = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * key_scale;
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(total), out, off + 4 * lane_id(), 0, 0);
}

constexpr int kBlockRows = 8;  // rows per group = waves per workgroup
constexpr int kRing = 4;       // page buffers per workgroup
constexpr int kDecBufs = 3;    // decoded pages: the one scored, the next, the one being decoded

template <int D, bool MX>
struct BlockShared {
  int page_prefix[kMaxGroups + 1];
  int req_tab[4][kMaxReqPrefill + 1];
  float wbuf[kBlockRows][kMaxHeads];
  int misc[16];
  alignas(16) uint8_t ring[kRing][Geometry<D, MX>::kPageBytes];  // raw pages
  alignas(16) v8bf dec[kDecBufs][2 * (D / 16) * kWave];  // decoded pages, in B-fragment order
};

// ---------------------------------------------------------------------------
// The scorer kernel
// ---------------------------------------------------------------------------

// Pages per group -> exclusive prefix in sm.page_prefix[0 .. NG] (LDS).
template <int RG, int NT, class SM>
__device__ __forceinline__ void build_page_prefix(const RowArgs& R, SM& sm, int NG) {
  const int tid = threadIdx.x;
  int run = 0;
  for (int base = 0; base < NG; base += NT) {
    const int g = base + tid;
    int np = 0;
    if (g < NG) {
      int L[RG], ql[RG];
      bool rl[RG];
      const GroupDesc d = describe_group<RG>(R, sm.req_tab, g, group_request<RG>(R, sm.req_tab, g), L, ql, rl);
      np = (d.Lmax + kPage - 1) / kPage;
    }
    int tot;
    const int ex = block_exclusive_scan<NT>(np, tot, sm.misc);
    if (g < NG) sm.page_prefix[g] = run + ex;
    run += tot;
  }
  if (tid == 0) sm.page_prefix[NG] = run;
  __syncthreads();
}

// Page j of the global list -> (group, page within group) by walking the
// prefix from the previous group (pages of a wave are visited in order).
__device__ __forceinline__ int advance_group(const int* page_prefix, int g, int pgl) {
  while (pgl >= page_prefix[g + 1]) ++g;
  return g;
}

// Group holding global page j: the last group whose first page is <= j
// (groups without pages share their first page with the next group).
__device__ __forceinline__ int group_of_page(const int* page_prefix, int ng, int j) {
  int lo = 0, hi = ng;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (page_prefix[mid] <= j) lo = mid; else hi = mid;
  }
  return lo;
}

// Unit ids of global pages jb + lane (one per lane, 0 past j1): a cache
// page of 64 << page_shift keys is 1 << page_shift units of 64 keys, unit
// id = page << page_shift | unit within the page; -1 for a block-table
// entry outside the pool (reported where it is used).
template <int RG>
__device__ __forceinline__ int page_ids(const ScoreParams& p, const int* page_prefix,
                                        const int (*req_tab)[kMaxReqPrefill + 1], int ng, int jb, int j1) {
  const int j = jb + lane_id();
  if (j >= j1) return 0;
  const RowArgs& R = p.rows;
  const int g = group_of_page(page_prefix, ng, j);
  const int b = group_request<RG>(R, req_tab, g);
  const int u = j - page_prefix[g];  // 64-key unit of the request
  const int sh = p.cache.page_shift;
  const int e = R.block_table[static_cast<int64_t>(b) * R.bt_stride + (u >> sh)];
  const bool ok = e >= 0 && static_cast<int64_t>(e) < p.cache.num_pages;
  return ok ? (e << sh) | (u & ((1 << sh) - 1)) : -1;  // unit id, or -1 outside the pool
}

// ---------------------------------------------------------------------------
// Requests of two grid rows (next_n = 2): wave pairs
// ---------------------------------------------------------------------------
//
// With one row per wave over a list of rows, the two rows of a request read
// its pages on unrelated waves at unrelated times, and the second read goes
// past L2 (measured: 1.48x the key bytes fetched on the MTP decode batch).
// For next_n = 2 the list counts request units instead, and each pair of
// waves of a workgroup (waves 2m and 2m + 1: one CU, so one L2) walks one
// contiguous range of them.  A request with two real rows has one unit per
// 64-key unit of its longer row, and the pair scores rows 0 and 1 of the same
// unit side by side, so the second request for a page finds it in the L2
// the first one filled; a request with one real row has one unit per two of
// its 64-key units, one for each wave.

// (request keys clamped to max_len, real rows) of request b.
__device__ __forceinline__ void pair_request(const RowArgs& R, int b, int& seq, int& dl) {
  seq = R.seq_lens[b];
  seq = seq > R.max_len ? R.max_len : seq;
  dl = R.decode_lens ? R.decode_lens[b] : 2;
}

// 64-key units of row 0 of a one-row request.
__device__ __forceinline__ int pair_row0_units(const RowArgs& R, int seq) {
  return (decode_row_len(seq, 1, 0, R.max_len, R.ratio) + kPage - 1) / kPage;
}

// Units of request b in the pair list.
__device__ __forceinline__ int pair_units(const RowArgs& R, int b) {
  int seq, dl;
  pair_request(R, b, seq, dl);
  if (dl >= 2) return (decode_row_len(seq, dl, 1, R.max_len, R.ratio) + kPage - 1) / kPage;
  if (dl == 1) return (pair_row0_units(R, seq) + 1) / 2;
  return 0;
}

// 64-key unit that the wave of parity `par` scores at unit t of a request
// with `dl` real rows (`np0` units in row 0 when dl = 1), or -1.
__device__ __forceinline__ int pair_unit(int dl, int np0, int t, int par) {
  if (dl >= 2) return t;
  const int u = 2 * t + par;
  return u < np0 ? u : -1;
}

// Units per request -> exclusive prefix in sm.page_prefix[0 .. num_req].
template <int NT, class SM>
__device__ __forceinline__ void build_pair_prefix(const RowArgs& R, SM& sm) {
  const int tid = threadIdx.x;
  int run = 0;
  for (int base = 0; base < R.num_req; base += NT) {
    const int b = base + tid;
    const int n = b < R.num_req ? pair_units(R, b) : 0;
    int tot;
    const int ex = block_exclusive_scan<NT>(n, tot, sm.misc);
    if (b < R.num_req) sm.page_prefix[b] = run + ex;
    run += tot;
  }
  if (tid == 0) sm.page_prefix[R.num_req] = run;
  __syncthreads();
}

// page_ids for the pair list: unit ids of the pages of units jb + lane for
// the wave of parity par; -2 where this wave has no page (a one-row
// request's odd last unit), -1 outside the pool.
__device__ __forceinline__ int pair_page_ids(const ScoreParams& p, const int* page_prefix, int jb, int j1, int par) {
  const int j = jb + lane_id();
  if (j >= j1) return 0;
  const RowArgs& R = p.rows;
  const int b = group_of_page(page_prefix, R.num_req, j);
  int seq, dl;
  pair_request(R, b, seq, dl);
  const int u = pair_unit(dl, dl == 1 ? pair_row0_units(R, seq) : 0, j - page_prefix[b], par);
  if (u < 0) return -2;
  const int sh = p.cache.page_shift;
  const int e = R.block_table[static_cast<int64_t>(b) * R.bt_stride + (u >> sh)];
  const bool ok = e >= 0 && static_cast<int64_t>(e) < p.cache.num_pages;
  return ok ? (e << sh) | (u & ((1 << sh) - 1)) : -1;
}

// The row of group g (decode groups hold one row): its query fragments,
// head weights (through the wave's LDS staging row, into the accumulator
// layout) and output descriptor.  `stage` is the wave's idle LDS area for a
// staged query load, or null.  Returns the row's key count.
template <int D, int MT>
__device__ __forceinline__ int setup_row(const ScoreParams& p, const int (*req_tab)[kMaxReqPrefill + 1], int g,
                                         float* wrow, QFrag<D, MT>& qf, WFrag<MT>& wf, RowOut& out,
                                         uint8_t* stage) {
  const RowArgs& R = p.rows;
  const int lane = lane_id();
  int L[1], qr[1];
  bool rl[1];
  const GroupDesc gd = describe_group<1>(R, req_tab, g, group_request<1>(R, req_tab, g), L, qr, rl);
  const int Lr = gd.nrows > 0 ? L[0] : 0;
  const bool real = rl[0];
  // weights first: they land with (not after) the queries
  const float wv = p.w[static_cast<int64_t>(real ? qr[0] : 0) * p.heads + (lane < p.heads ? lane : 0)];
  if constexpr (query_stage_bytes<D, MT>() > 0) {
    if (stage != nullptr && p.heads == 32 * MT) load_query_staged<D, MT>(p, qr[0], stage, qf);
    else load_query<D, MT>(p, qr[0], qf);
  } else {
    load_query<D, MT>(p, qr[0], qf);
  }
  wrow[lane] = (!real || lane >= p.heads) ? 0.0f : wv;
  out = row_out(p.logits + static_cast<int64_t>(gd.row0) * p.logits_stride + gd.col0, Lr);
  __builtin_amdgcn_wave_barrier();
  const int hg = 4 * (lane >> 5);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const float4 x = *reinterpret_cast<const float4*>(&wrow[32 * mt + 8 * i4 + hg]);
      wf.v[mt][4 * i4 + 0] = x.x;
      wf.v[mt][4 * i4 + 1] = x.y;
      wf.v[mt][4 * i4 + 2] = x.z;
      wf.v[mt][4 * i4 + 3] = x.w;
    }
  __builtin_amdgcn_wave_barrier();
  return __builtin_amdgcn_readfirstlane(Lr);
}

// Decode scorer: every decode row is a group of its own and every wave walks
// a contiguous range of the list of rows' pages; with PAIRS (next_n = 2)
// the list counts request units and wave pairs walk it (see above).
template <int D, bool MX, int MT, bool PAIRS>
__global__ __launch_bounds__(kDecodeWaves * kWave, 1) void score_kernel(ScoreParams p) {
  constexpr int kThreads = kDecodeWaves * kWave;
  __shared__ ScoreShared<D, MX, MT, kDecodeWaves> sm;
  const RowArgs& R = p.rows;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const bool tables = R.kind != 0 || R.q_packed;
  const int NG = tables ? build_request_tables<1, kThreads>(R, sm) : p.num_groups;

  int NL;  // entries of the list: rows, or requests with PAIRS
  int j0, j1;
  if constexpr (PAIRS) {
    build_pair_prefix<kThreads>(R, sm);
    NL = R.num_req;
    // this wave pair's contiguous unit range
    even_split(sm.page_prefix[NL], gridDim.x * (kDecodeWaves / 2), blockIdx.x * (kDecodeWaves / 2) + (wave >> 1),
               j0, j1);
  } else {
    build_page_prefix<1, kThreads>(R, sm, NG);
    NL = NG;
    // this wave's contiguous page range
    even_split(sm.page_prefix[NL], gridDim.x * kDecodeWaves, blockIdx.x * kDecodeWaves + wave, j0, j1);
  }
  j0 = __builtin_amdgcn_readfirstlane(j0);
  j1 = __builtin_amdgcn_readfirstlane(j1);
  const int par = wave & 1;

  float* wrow = sm.wbuf[wave];
  WaveArea<D, MX, MT>& area = sm.area[wave];
  constexpr int NP = ring_pages<D, MX, MT>();
  static_assert(NP >= 2 && NP <= 4, "ring of two to four pages");
  const uint32_t ring_lds = lds_addr(area.page[0]);  // page i of the ring at ring_lds + i * kPageBytes

  bool bad_page = false;
  if (j0 < j1) {
    // Page ids come in batches of 64 (lane i: entry jb + i), so that no
    // compiler-visible load sits between page requests; a later batch costs
    // one drain of the requests in flight.
    auto batch = [&](int jb_) -> int {
      if constexpr (PAIRS) return pair_page_ids(p, sm.page_prefix, jb_, j1, par);
      else return page_ids<1>(p, sm.page_prefix, sm.req_tab, NG, jb_, j1);
    };
    int jb = j0;
    int ids = batch(jb);
    auto id_of = [&](int j) -> int {  // j < j1
      if (j - jb >= kWave) {
        jb = j;
        ids = batch(jb);
      }
      const int id = __builtin_amdgcn_readlane(ids, j - jb);
      bad_page |= id == -1;  // ids outside the pool read page 0 and are reported
      return id >= 0 ? id : 0;  // (-2: no page for this wave; page 0 keeps the ring moving)
    };

    // The row this wave scores in list entry g, and with PAIRS the request's
    // real rows and row-0 units.
    int dl_cur = 0, np0_cur = 0;
    auto entry_row = [&](int g) -> int {
      if constexpr (PAIRS) {
        int seq;
        pair_request(R, g, seq, dl_cur);
        np0_cur = dl_cur == 1 ? pair_row0_units(R, seq) : 0;
        return 2 * g + (dl_cur >= 2 ? par : 0);
      } else {
        return g;
      }
    };

    // The first entry's queries and weights are loaded together with the
    // ids and before any page is requested: waiting for them then never
    // waits for a page, and the first page can be scored as soon as it lands.
    QFrag<D, MT> qf;
    WFrag<MT> wf;
    RowOut out;
    int gs = group_of_page(sm.page_prefix, NL, j0);  // list entry of the page being scored
    int row_len = setup_row<D, MT>(p, sm.req_tab, entry_row(gs), wrow, qf, wf, out, area.stage);
    int g_first = sm.page_prefix[gs];  // the entry's first list index
    int cur_g = gs;

    // With one row per request every page is read once per launch: its
    // requests carry the non-temporal hint (rows of one request read their
    // pages again and keep the default).
    const bool once = !PAIRS && R.next_n == 1;
    auto request = [&](int id, uint32_t lds) {
      if (once) dma_page<D, MX, true>(p, id, lds);
      else dma_page<D, MX, false>(p, id, lds);
    };
    int first[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) first[i] = j0 + i < j1 ? id_of(j0 + i) : 0;
    wait_all_loads();  // nothing the compiler loaded before is still in flight
    wait_lds();        // the staged query reads have returned: the area is free
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (j0 + i < j1) request(first[i], ring_lds + i * Geometry<D, MX>::kPageBytes);

    int slot = 0;  // ring slot of page j
    // 32-key tiles are pipelined across pages: a tile's MFMAs are issued
    // next to the head sums of the tile before it.
    v16f acc0[MT], acc1[MT];
    float ks0 = 0.0f, ks1 = 0.0f;
    int off1 = 0x7FFFFFF0;  // byte offset of the pending tile (none yet)
    const int key_off = (lane & 31) * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc1[mt] = v16f{};

    for (int j = j0; j < j1; ++j) {
      gs = advance_group(sm.page_prefix, gs, j);
      if (gs != cur_g) {
        // a later entry (waiting for its loads drains the page requests in
        // flight; a wave's range crosses few entry boundaries)
        tile_logits<MT>(acc1, ks1, wf, out, off1);  // the old row's pending tile
        off1 = 0x7FFFFFF0;
        row_len = setup_row<D, MT>(p, sm.req_tab, entry_row(gs), wrow, qf, wf, out, nullptr);
        // Wait for the new row's loads here, on this path only.  Left to the
        // compiler, the waits for them land at their first uses in the
        // scoring below, which runs for every page, where they also count
        // the page requests in flight (the compiler does not see those).
        wait_all_loads();
        g_first = sm.page_prefix[gs];
        cur_g = gs;
      }
      // the row's 64-key unit at list index j (none for this wave: -1)
      int u = j - g_first;
      if constexpr (PAIRS) u = pair_unit(dl_cur, np0_cur, u, par);
      const int nxt = j + NP < j1 ? id_of(j + NP) : 0;
      // page j has landed once only the requests after it (pages up to
      // j + NP - 1) are outstanding
      wait_page_with_later<D, MX>((j + NP - 1 < j1 - 1 ? j + NP - 1 : j1 - 1) - j);
      if (row_len > 0 && u >= 0) {  // wave-uniform: a padded slot only keeps the ring moving
        const uint8_t* buf = area.page[slot];
        const int base = u * kPage * 4 + key_off;
        tile_mfma_raw<D, MX, MT>(buf, 0, qf, acc0, ks0);
        tile_logits<MT>(acc1, ks1, wf, out, off1);
        __builtin_amdgcn_sched_barrier(0);  // keep each stage's registers to itself
        tile_mfma_raw<D, MX, MT>(buf, 1, qf, acc1, ks1);
        tile_logits<MT>(acc0, ks0, wf, out, base);
        __builtin_amdgcn_sched_barrier(0);
        off1 = base + 32 * 4;
      }
      if (j + NP < j1) request(nxt, ring_lds + slot * Geometry<D, MX>::kPageBytes);  // into the freed slot
      slot = slot + 1 == NP ? 0 : slot + 1;
    }
    tile_logits<MT>(acc1, ks1, wf, out, off1);  // the last tile
  }
  wait_all_loads();  // no request may still be writing LDS when the wave ends
  if (bad_page && lane == 0) atomicOr(reinterpret_cast<uint32_t*>(p.header) + kHdrStatus, kStatusBadPage);
}

// ---------------------------------------------------------------------------
// The prefill scorer: one page ring per workgroup
// ---------------------------------------------------------------------------
//
// Prefill rows come in long runs of one request whose key ranges differ by
// one key per row, so here a group is kBlockRows consecutive query rows and
// each wave scores one of them: every page is read from memory once per
// group and shared by the eight waves through a ring of kRing page buffers
// in LDS.  Wave 0 requests pages four ahead of the one scored.  Each page
// is decoded to bf16 once, by all waves together (an eighth each), two pages
// ahead of scoring, into one of kDecBufs decoded-page buffers, so that the
// per-row VALU work is the head sums.

// Decodes this wave's share of a raw page into B-fragment order: fragment
// (tile nt, k-step s) of lane l goes to dec[(nt KS + s) 64 + l], so that a
// wave reads a fragment with one contiguous 1 KiB LDS access.  The 2 KS
// fragment blocks of a page are spread over the waves.
template <int D, bool MX>
__device__ __forceinline__ void decode_page_slice(const uint8_t* raw, v8bf* dec, int wave) {
  constexpr int KS = D / 16;
  const int lane = lane_id();
#pragma unroll
  for (int b0 = 0; b0 < 2 * KS; b0 += kBlockRows) {
    const int blk = b0 + wave;
    if ((2 * KS) % kBlockRows == 0 || blk < 2 * KS) {
      const int nt = blk / KS, s = blk % KS;
      dec[blk * kWave + lane] = key_step<D, MX>(raw + (nt * 32 + (lane & 31)) * Geometry<D, MX>::kRowBytes, lane >> 5, s);
    }
  }
}

// Raw scores of one row against 32-key tile nt of a decoded page.
template <int D, bool MX, int MT>
__device__ __forceinline__ void tile_mfma(const v8bf* dec, int nt, const QFrag<D, MT>& qf, v16f (&acc)[MT]) {
  constexpr int KS = D / 16;
  const int lane = lane_id();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v16f{};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const v8bf b = dec[(nt * KS + s) * kWave + lane];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf.a[mt][s], b, acc[mt], 0, 0, 0);
  }
}

// This wave's row (row `wave` of group g): query fragments, weights and
// output descriptor.
template <int D, int MT>
__device__ __forceinline__ void setup_block_row(const ScoreParams& p, const int (*req_tab)[kMaxReqPrefill + 1], int g,
                                                int wave, float* wrow, QFrag<D, MT>& qf, WFrag<MT>& wf,
                                                RowOut& out) {
  const RowArgs& R = p.rows;
  const int lane = lane_id();
  int L[kBlockRows], ql[kBlockRows];
  bool rl[kBlockRows];
  const GroupDesc gd =
      describe_group<kBlockRows>(R, req_tab, g, group_request<kBlockRows>(R, req_tab, g), L, ql, rl);
  const bool exists = wave < gd.nrows;
  const int qrow = exists ? ql[wave] : -1;
  load_query<D, MT>(p, qrow, qf);
  float wv = p.w[static_cast<int64_t>(exists ? qrow : 0) * p.heads + (lane < p.heads ? lane : 0)];
  if (!exists || lane >= p.heads) wv = 0.0f;
  wrow[lane] = wv;
  out = row_out(p.logits + static_cast<int64_t>(gd.row0 + wave) * p.logits_stride + gd.col0, exists ? L[wave] : 0);
  __builtin_amdgcn_wave_barrier();
  const int hg = 4 * (lane >> 5);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const float4 x = *reinterpret_cast<const float4*>(&wrow[32 * mt + 8 * i4 + hg]);
      wf.v[mt][4 * i4 + 0] = x.x;
      wf.v[mt][4 * i4 + 1] = x.y;
      wf.v[mt][4 * i4 + 2] = x.z;
      wf.v[mt][4 * i4 + 3] = x.w;
    }
  __builtin_amdgcn_wave_barrier();
}

// Waits (wave 0) until page j has landed, given how many pages were
// requested after it.
template <int D, bool MX>
__device__ __forceinline__ void wait_ring_page(int after) {
  constexpr int n = Geometry<D, MX>::kLoads;
  static_assert(kRing == 4, "the waits below cover up to kRing - 2 later pages");
  if (after >= 2) wait_vmcnt<2 * n>();
  else if (after == 1) wait_vmcnt<n>();
  else wait_all_loads();
}

// A tile's B fragments, read from a decoded page into registers.
template <int D>
__device__ __forceinline__ void tile_frags(const v8bf* dec, int nt, v8bf (&b)[D / 16]) {
  constexpr int KS = D / 16;
  const int lane = lane_id();
#pragma unroll
  for (int s = 0; s < KS; ++s) b[s] = dec[(nt * KS + s) * kWave + lane];
}

template <int D, int MT>
__device__ __forceinline__ void tile_mfma_regs(const v8bf (&b)[D / 16], const QFrag<D, MT>& qf, v16f (&acc)[MT]) {
  constexpr int KS = D / 16;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v16f{};
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf.a[mt][s], b[s], acc[mt], 0, 0, 0);
}

// Key scale of key `lane` of a raw page (fp8 rows carry one; MXFP4 block
// scales are applied while decoding).
template <int D, bool MX>
__device__ __forceinline__ float raw_key_scale(const uint8_t* raw) {
  return MX ? 1.0f : *reinterpret_cast<const float*>(raw + lane_id() * Geometry<D, MX>::kRowBytes + D);
}

template <int D, bool MX, int MT>
__global__ __launch_bounds__(kBlockRows * kWave, 1) void score_block_kernel(ScoreParams p) {
  constexpr int NT = kBlockRows * kWave;
  constexpr int KS = D / 16;
  __shared__ BlockShared<D, MX> sm;
  const RowArgs& R = p.rows;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int NG = build_request_tables<kBlockRows, NT>(R, sm);
  build_page_prefix<kBlockRows, NT>(R, sm, NG);
  const int P = sm.page_prefix[NG];

  // this workgroup's contiguous page range (the same for all its waves)
  int j0, j1;
  even_split(P, gridDim.x, blockIdx.x, j0, j1);
  j0 = __builtin_amdgcn_readfirstlane(j0);
  j1 = __builtin_amdgcn_readfirstlane(j1);
  if (j0 >= j1) return;

  const bool issuer = wave == 0;
  bool bad_page = false;
  int jb = j0;
  int ids = issuer ? page_ids<kBlockRows>(p, sm.page_prefix, sm.req_tab, NG, jb, j1) : 0;
  auto id_of = [&](int j) -> int {  // wave 0 only; j < j1
    if (j - jb >= kWave) {
      jb = j;
      ids = page_ids<kBlockRows>(p, sm.page_prefix, sm.req_tab, NG, jb, j1);
    }
    const int id = __builtin_amdgcn_readlane(ids, j - jb);
    const bool ok = id >= 0;
    bad_page |= !ok;  // ids outside the pool read page 0 and are reported
    return ok ? id : 0;
  };

  QFrag<D, MT> qf;
  WFrag<MT> wf;
  RowOut out;
  int gs = group_of_page(sm.page_prefix, NG, j0);
  setup_block_row<D, MT>(p, sm.req_tab, gs, wave, sm.wbuf[wave], qf, wf, out);
  int g_first = sm.page_prefix[gs];

  // Pipeline (page j0 + i: raw buffer i % kRing, decoded buffer i % kDecBufs):
  // in the iteration of page j the waves score page j, decode page j + 2
  // and read the first tile's fragments of page j + 1 (decoded two
  // iterations before), and wave 0 requests page j + 4; one barrier per
  // page, at the end, publishes decoded page j + 2 and raw page j + 3 and
  // retires every read of page j - 1's buffers.  The first tile's
  // fragments are thus in registers when the barrier opens, and the decode
  // runs under the MFMAs of page j.
  if (issuer) {
    int first[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) first[i] = j0 + i < j1 ? id_of(j0 + i) : 0;
    wait_all_loads();  // nothing the compiler loaded before is still in flight
#pragma unroll
    for (int i = 0; i < kRing; ++i)
      if (j0 + i < j1) dma_page<D, MX>(p, first[i], lds_addr(sm.ring[i]));
    // pages j0 and j0 + 1 have landed
    const int last = j0 + kRing - 1 < j1 - 1 ? j0 + kRing - 1 : j1 - 1;
    wait_ring_page<D, MX>(last - (j0 + 1) > 0 ? last - (j0 + 1) : 0);
  }
  __syncthreads();
  decode_page_slice<D, MX>(sm.ring[0], sm.dec[0], wave);
  float ks_cur = raw_key_scale<D, MX>(sm.ring[0]);
  float ks_nxt = 0.0f;
  if (j0 + 1 < j1) {
    decode_page_slice<D, MX>(sm.ring[1], sm.dec[1], wave);
    ks_nxt = raw_key_scale<D, MX>(sm.ring[1]);
  }
  if (issuer && j0 + 2 < j1) wait_ring_page<D, MX>(j0 + 3 < j1 ? 1 : 0);  // page j0 + 2 has landed
  __syncthreads();
  v8bf bt0[KS];
  tile_frags<D>(sm.dec[0], 0, bt0);

  constexpr int kNone = 0x7FFFFF00;  // an offset past any row: nothing stored
  v16f acc0[MT], acc1[MT];
  int j = j0;
  for (;;) {
    const int seg_end = sm.page_prefix[gs + 1] < j1 ? sm.page_prefix[gs + 1] : j1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc1[mt] = v16f{};
    float pend0 = 0.0f;     // tile 0 partial of the pending page
    float pend_ks = 0.0f;   // its key scales (key `lane` of the page)
    int pend_off = kNone;   // its first key's byte offset in the row (none yet)
    for (; j < seg_end; ++j) {
      const int i = j - j0;
      if (issuer && j + kRing < j1) {
        const int nxt = id_of(j + kRing);
        dma_page<D, MX>(p, nxt, lds_addr(sm.ring[i % kRing]));
      }
      const v8bf* dec = sm.dec[i % kDecBufs];
      float ks_new;
      {
        // past the range's end this decodes a stale buffer into a decoded
        // buffer that nothing reads again (branch-free, so that the decode
        // interleaves with the MFMAs)
        const uint8_t* raw2 = sm.ring[(i + 2) % kRing];
        decode_page_slice<D, MX>(raw2, sm.dec[(i + 2) % kDecBufs], wave);
        ks_new = raw_key_scale<D, MX>(raw2);
      }
      tile_mfma_regs<D, MT>(bt0, qf, acc0);
      page_logits(pend0, tile_partial<MT>(acc1, wf), pend_ks, out, pend_off);  // the previous page
      __builtin_amdgcn_sched_barrier(0);  // keep each stage's registers to itself
      tile_mfma<D, MX, MT>(dec, 1, qf, acc1);
      pend0 = tile_partial<MT>(acc0, wf);
      tile_frags<D>(sm.dec[(i + 1) % kDecBufs], 0, bt0);  // (stale past the end, unused)
      __asm__ volatile("" : : "v"(pend0), "v"(ks_new));  // computed here, not after the wait below
      __builtin_amdgcn_sched_barrier(0);
      pend_ks = ks_cur;
      ks_cur = ks_nxt;
      ks_nxt = ks_new;
      pend_off = (j - g_first) * kPage * 4;
      if (issuer && j + 3 < j1) wait_ring_page<D, MX>(j + kRing < j1 ? 1 : 0);  // raw page j + 3 has landed
      __syncthreads();
    }
    page_logits(pend0, tile_partial<MT>(acc1, wf), pend_ks, out, pend_off);  // the segment's last page
    if (j >= j1) break;
    gs = advance_group(sm.page_prefix, gs, j);
    setup_block_row<D, MT>(p, sm.req_tab, gs, wave, sm.wbuf[wave], qf, wf, out);
    g_first = sm.page_prefix[gs];
  }
  wait_all_loads();  // no request may still be writing LDS when the wave ends
  if (bad_page && lane == 0) atomicOr(reinterpret_cast<uint32_t*>(p.header) + kHdrStatus, kStatusBadPage);
}

}  // namespace idx
