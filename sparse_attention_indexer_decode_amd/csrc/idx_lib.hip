// Host side of the indexer library: argument checks, workspace sizing,
// kernel selection and launch.  See include/idx.h for the contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>

#include "../../include/idx.h"
#include "idx_internal.h"
#include "cache_write.cuh"
#include "pool.cuh"
#include "score.cuh"
#include "topk.cuh"

// Scratch of idx_decode_topk_noalloc: the row logits and long rows' chunk
// candidates of one decode batch, in place of a caller workspace.  Each GPU
// that runs the library holds its own copy until the process ends; calls on
// one GPU share it (and race if they overlap).
constexpr size_t kStaticScratchBytes = size_t{160} << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace idx {
namespace {

constexpr int kMaxDevices = 64;

thread_local const char* g_last_error = "";

// Records which check failed (for idx_last_error) and returns the status.
idx_status fail(idx_status st, const char* what) {
  g_last_error = what;
  return st;
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkThreadsLean = 512;

int row_bytes(int fmt, int d) { return fmt == IDX_FMT_FP8_E4M3 ? d + 4 : d / 2 + d / 32; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

idx_status check_cache(const idx_cache* c, CacheArgs& out) {
  if (!c || !c->base) return fail(IDX_EINVAL, "cache descriptor or its base pointer is null");
  if (c->num_pages <= 0 || c->page_bytes <= 0 || c->reserved != 0) return fail(IDX_EINVAL, "cache: num_pages and page_bytes must be positive, reserved 0");
  if (c->page_size != kPage && c->page_size != 4 * kPage) return fail(IDX_EUNSUPPORTED, "cache: page_size must be 64 or 256");
  if (c->fmt == IDX_FMT_FP8_E4M3) {
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return fail(IDX_EUNSUPPORTED, "cache: fp8 head_dim must be 32, 64 or 128");
  } else if (c->fmt == IDX_FMT_MXFP4) {
    if (c->head_dim != 128) return fail(IDX_EUNSUPPORTED, "cache: MXFP4 head_dim must be 128");
  } else {
    return fail(IDX_EUNSUPPORTED, "cache: unknown format");
  }
  const int rb = row_bytes(c->fmt, c->head_dim);
  if (c->page_bytes < static_cast<int64_t>(c->page_size) * rb) return fail(IDX_EINVAL, "cache: page_bytes smaller than page_size token rows");
  const int shift = c->page_size == kPage ? 0 : 2;
  if (c->num_pages > (INT32_MAX >> shift)) return fail(IDX_EUNSUPPORTED, "cache: more than 2^31 64-token units");
  if ((c->page_bytes & 15) != 0 || (reinterpret_cast<uintptr_t>(c->base) & 15) != 0) return fail(IDX_EINVAL, "cache: base and page_bytes must be 16-byte aligned");
  out.base = static_cast<const uint8_t*>(c->base);
  out.num_pages = c->num_pages;
  out.page_bytes = c->page_bytes;
  out.page_shift = shift;
  out.head_dim = c->head_dim;
  out.row_bytes = rb;
  out.fmt = c->fmt;
  return IDX_OK;
}

int64_t rows_count(const idx_rows* r) {
  if (!r) return -1;
  if (r->kind == IDX_ROWS_DECODE) {
    if (r->num_req < 0 || r->next_n < 1) return -1;
    return static_cast<int64_t>(r->num_req) * r->next_n;
  }
  if (r->kind == IDX_ROWS_PREFILL) {
    if (r->q_begin < 0 || r->q_end < r->q_begin) return -1;
    return static_cast<int64_t>(r->q_end) - r->q_begin;
  }
  return -1;
}

// `need_table`: the block table is read (scoring); top-k needs lengths only.
idx_status check_rows(const idx_rows* r, bool need_table, RowArgs& out) {
  const int64_t nrows = rows_count(r);
  if (nrows < 0) return fail(IDX_EINVAL, "rows: bad kind, next_n < 1 or q_end < q_begin");
  if (r->num_req < 0 || r->max_seq_len < 0) return fail(IDX_EINVAL, "rows: negative num_req or max_seq_len");
  if (r->num_req > 0 && !r->seq_lens) return fail(IDX_EINVAL, "rows: seq_lens is null");
  if (need_table) {
    if (r->num_req > 0 && !r->block_table) return fail(IDX_EINVAL, "rows: block_table is null");
    if (r->bt_width < 0 || r->bt_stride < r->bt_width) return fail(IDX_EINVAL, "rows: bt_stride < bt_width");
  }
  if (r->compress_ratio < 0) return fail(IDX_EINVAL, "rows: compress_ratio < 0");
  if (r->compress_ratio > kMaxRatio) return fail(IDX_EUNSUPPORTED, "rows: compress_ratio above 1024");
  if (nrows > (int64_t{1} << 30)) return fail(IDX_EUNSUPPORTED, "rows: more than 2^30 rows");
  if (r->kind == IDX_ROWS_DECODE) {
    if (r->q_packed != 0 && r->q_packed != 1) return fail(IDX_EINVAL, "rows: q_packed must be 0 or 1");
    if (r->q_packed && r->num_req > kMaxReqPrefill) return fail(IDX_EUNSUPPORTED, "rows: packed queries support at most 256 requests");
  } else {
    if (r->num_req > 0 && !r->query_start_loc) return fail(IDX_EINVAL, "rows: query_start_loc is null");
    if (r->num_req > kMaxReqPrefill) return fail(IDX_EUNSUPPORTED, "rows: a prefill chunk supports at most 256 requests");
    if (r->num_req == 0 && nrows > 0) return fail(IDX_EINVAL, "rows: prefill rows without requests");
  }
  out.kind = r->kind;
  out.num_req = r->num_req;
  out.block_table = r->block_table;
  out.bt_stride = r->bt_stride;
  out.max_len = r->max_seq_len;
  out.ratio = r->compress_ratio > 1 ? r->compress_ratio : 1;
  out.max_keys = out.max_len / out.ratio;
  out.seq_lens = r->seq_lens;
  out.decode_lens = r->decode_lens;
  out.next_n = r->kind == IDX_ROWS_DECODE ? r->next_n : 1;
  out.q_packed = r->kind == IDX_ROWS_DECODE ? r->q_packed : 0;
  out.qsl = r->query_start_loc;
  out.q_begin = r->q_begin;
  out.q_end = r->q_end;
  out.num_rows = static_cast<int32_t>(nrows);
  return IDX_OK;
}

// The block table covers every key of the longest row: ceil(max_keys /
// page_size) <= bt_width.
idx_status check_table(const idx_rows* r, const RowArgs& R, const CacheArgs& C) {
  const int64_t page = int64_t{kPage} << C.page_shift;
  if ((R.max_keys + page - 1) / page > r->bt_width) return fail(IDX_EINVAL, "rows: max_seq_len / compress_ratio exceeds bt_width * page_size");
  return IDX_OK;
}

// Rows per scorer group: prefill, kBlockRows consecutive query rows per
// workgroup; decode, one row (a wave's page range walks one row at a time).
int pick_rg(const RowArgs& R) { return R.kind != 0 ? kBlockRows : 1; }

// Upper bound of the scorer's row groups.
int64_t group_bound(const RowArgs& R, int rg) {
  if (R.kind == 0) return static_cast<int64_t>(R.num_req) * ceil_div(R.next_n, rg);
  return ceil_div(R.num_rows, rg) + R.num_req;
}

int64_t scratch_stride(const RowArgs& R) {
  const int64_t m = R.max_keys > 0 ? R.max_keys : 1;
  return ceil_div(m, 64) * 64;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Decode-topk workspace: [header 256 B][row logits, scratch_stride apart]
size_t scratch_offset() { return kStatusBytes; }
size_t decode_ws_bytes(const RowArgs& R) {
  return scratch_offset() + sizeof(float) * static_cast<size_t>(R.num_rows) * scratch_stride(R);
}

template <int D, bool MX, int MT>
hipError_t launch_score(const ScoreParams& p, int grid, hipStream_t s) {
  // next_n = 2: the two rows of a request on a wave pair
  if (p.rows.next_n == 2)
    hipLaunchKernelGGL((score_kernel<D, MX, MT, true>), dim3(grid), dim3(kDecodeWaves * kWave), 0, s, p);
  else
    hipLaunchKernelGGL((score_kernel<D, MX, MT, false>), dim3(grid), dim3(kDecodeWaves * kWave), 0, s, p);
  return hipGetLastError();
}

template <int D, bool MX, int MT>
hipError_t launch_block(const ScoreParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((score_block_kernel<D, MX, MT>), dim3(grid), dim3(kBlockRows * kWave), 0, s, p);
  return hipGetLastError();
}

hipError_t dispatch_score(const ScoreParams& p, int grid, hipStream_t s) {
  const int d = p.cache.head_dim;
  const bool mx = p.cache.fmt == IDX_FMT_MXFP4;
  const int mt = p.heads > 32 ? 2 : 1;
  if (p.rows.kind != 0) {
#define IDX_BLOCK_CASE(D_, MX_, MT_) \
  if (d == D_ && mx == MX_ && mt == MT_) return launch_block<D_, MX_, MT_>(p, grid, s);
    IDX_BLOCK_CASE(128, false, 1) IDX_BLOCK_CASE(128, false, 2)
    IDX_BLOCK_CASE(64, false, 1) IDX_BLOCK_CASE(64, false, 2)
    IDX_BLOCK_CASE(32, false, 1) IDX_BLOCK_CASE(32, false, 2)
    IDX_BLOCK_CASE(128, true, 1) IDX_BLOCK_CASE(128, true, 2)
#undef IDX_BLOCK_CASE
    return hipErrorInvalidValue;
  }
#define IDX_SCORE_CASE(D_, MX_, MT_) \
  if (d == D_ && mx == MX_ && mt == MT_) return launch_score<D_, MX_, MT_>(p, grid, s);
#define IDX_SCORE_RGMT(D_, MX_) IDX_SCORE_CASE(D_, MX_, 1) IDX_SCORE_CASE(D_, MX_, 2)
  IDX_SCORE_RGMT(128, false)
  IDX_SCORE_RGMT(64, false)
  IDX_SCORE_RGMT(32, false)
  IDX_SCORE_RGMT(128, true)
#undef IDX_SCORE_RGMT
#undef IDX_SCORE_CASE
  return hipErrorInvalidValue;
}

// One workgroup per CU (each wave streams a contiguous page range), fewer
// when the launch cannot hold a page per wave.
int score_grid(const RowArgs& R, int rg) {
  const int64_t pages = group_bound(R, rg) * ceil_div(R.max_keys, kPage);
  int64_t g = device_cu_count();
  const int64_t need = ceil_div(pages, 8);
  if (g > need) g = need;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

idx_status check_queries(const uint16_t* q, const float* w, int heads) {
  if (heads < 1) return fail(IDX_EINVAL, "heads must be >= 1");
  if (heads > kMaxHeads) return fail(IDX_EUNSUPPORTED, "heads must be <= 64");
  if (!q || !w) return fail(IDX_EINVAL, "q or w is null");
  if ((reinterpret_cast<uintptr_t>(q) & 15) != 0) return fail(IDX_EINVAL, "q must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(w) & 3) != 0) return fail(IDX_EINVAL, "w must be 4-byte aligned");
  return IDX_OK;
}

// Rows longer than the register path (kRowCap keys) are split into chunks
// of kRowCap keys, each chunk selected by its own workgroup, then merged per
// row, when all the chunks fit one workgroup per CU of the target part
// (kChunkWgMax); with more, a chunk's workgroup waits for a CU and one
// workgroup per row streaming its row is faster.  (A pure function of the
// rows and k, so that the workspace size does not depend on the device.)
constexpr int kChunkWgMax = 256;

int topk_chunks(const RowArgs& R) {
  if (R.max_keys <= kRowCap) return 0;
  const int64_t c = ceil_div(R.max_keys, kRowCap);
  if (c > kMaxTopkChunks || static_cast<int64_t>(R.num_rows) * c > kChunkWgMax) return 0;
  return static_cast<int>(c);
}

// Long rows are split with one shared threshold when k allows the one-read
// selection (topk_split_*: kCandCap candidates per chunk slot and a count
// per slot), otherwise by a top-k per chunk (topk_chunk_kernel /
// topk_merge_kernel: k per slot, contiguous per row).
bool topk_split_sampled(int k) { return k <= kSampleMaxK; }

// Workspace bytes of the chunk candidates (two [rows][chunks][cap] arrays,
// logits and row positions, then the [rows][chunks] counts when sampled).
size_t topk_chunk_bytes(const RowArgs& R, int k) {
  const int c = topk_chunks(R);
  if (!c) return 0;
  const size_t slots = static_cast<size_t>(R.num_rows) * c;
  const bool sampled = topk_split_sampled(k);
  const size_t cap = sampled ? kCandCap : static_cast<size_t>(k);
  return align_up(2 * sizeof(int32_t) * slots * cap + (sampled ? sizeof(int32_t) * slots : 0), 256);
}

idx_status launch_topk(const float* logits, int64_t stride, const RowArgs& R, int k, int32_t* out,
                       void* chunk_ws, hipStream_t s) {
  TopkParams p{};
  p.logits = logits;
  p.stride = stride;
  p.rows = R;
  p.k = k;
  p.out = out;
  const int nc = topk_chunks(R);
  if (nc > 0) {
    const bool sampled = topk_split_sampled(k);
    p.chunks = nc;
    p.cap = sampled ? kCandCap : k;
    const size_t n = static_cast<size_t>(R.num_rows) * nc * p.cap;
    p.cand_val = static_cast<float*>(chunk_ws);
    p.cand_pos = reinterpret_cast<int32_t*>(p.cand_val + n);
    p.cand_cnt = p.cand_pos + n;
    // dynamic LDS: the k selected positions of a chunk or a merge
    // (topk_chunk_kernel, topk_merge_kernel; the split kernels leave it
    // unused), sized so that two of these workgroups never share a CU (the
    // launch has at most a few hundred; doubling up would halve their speed)
    constexpr unsigned kOneWgPerCu = 48 * 1024;
    static_assert(kOneWgPerCu >= sizeof(int32_t) * kMaxK, "k positions must fit the dynamic LDS");
    if (sampled) {
      hipLaunchKernelGGL(topk_split_collect_kernel<kTopkThreads>, dim3(R.num_rows * nc), dim3(kTopkThreads),
                         kOneWgPerCu, s, p);
      hipLaunchKernelGGL(topk_split_merge_kernel<kTopkThreads>, dim3(R.num_rows), dim3(kTopkThreads), kOneWgPerCu,
                         s, p);
    } else {
      hipLaunchKernelGGL(topk_chunk_kernel<kTopkThreads>, dim3(R.num_rows * nc), dim3(kTopkThreads), kOneWgPerCu, s,
                         p);
      hipLaunchKernelGGL(topk_merge_kernel<kTopkThreads>, dim3(R.num_rows), dim3(kTopkThreads), kOneWgPerCu, s, p);
    }
    return hipGetLastError() == hipSuccess ? IDX_OK : fail(IDX_EHIP, "kernel launch failed");
  }
  // Batches whose rows may exceed the register path and that have at least
  // two rows per CU run a streaming-only 512-thread kernel, several rows per
  // CU at once; otherwise one 1024-thread workgroup per row.
  if (R.max_keys > kRowCap && R.num_rows >= 2 * device_cu_count())
    hipLaunchKernelGGL((topk_kernel<kTopkThreadsLean, false>), dim3(R.num_rows), dim3(kTopkThreadsLean), 0, s, p);
  else
    hipLaunchKernelGGL(topk_kernel<kTopkThreads>, dim3(R.num_rows), dim3(kTopkThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? IDX_OK : fail(IDX_EHIP, "kernel launch failed");
}

idx_status check_ws(void* ws, size_t have, size_t need) {
  if (!ws) return fail(IDX_EINVAL, "workspace is null");
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(IDX_EINVAL, "workspace must be 256-byte aligned");
  if (have < need) return fail(IDX_ENOSPC, "workspace too small (see idx_workspace_bytes)");
  return IDX_OK;
}

// Pool selection arguments, against the rows' longest row.
idx_status check_pools(const idx_pools* pl, const RowArgs& R, int& lg) {
  if (!pl) return fail(IDX_EINVAL, "pools descriptor is null");
  lg = pl->pool_size == 16 ? 4 : pl->pool_size == 32 ? 5 : pl->pool_size == 64 ? 6 : pl->pool_size == 128 ? 7 : -1;
  if (lg < 0) return fail(IDX_EUNSUPPORTED, "pool_size must be 16, 32, 64 or 128");
  if (pl->topk_pools < 1) return fail(IDX_EINVAL, "topk_pools must be >= 1");
  if (pl->topk_pools > kMaxPoolTopk) return fail(IDX_EUNSUPPORTED, "topk_pools must be <= 512");
  if (pl->init_pools < 0 || pl->local_pools < 0 ||
      static_cast<int64_t>(pl->init_pools) + pl->local_pools > pl->topk_pools)
    return fail(IDX_EINVAL, "init_pools and local_pools must be >= 0 with a sum <= topk_pools");
  if ((static_cast<int64_t>(R.max_keys) >> lg) > kMaxPools)
    return fail(IDX_EUNSUPPORTED, "rows of more than 8192 complete pools");
  return IDX_OK;
}

idx_status launch_pool_topk(const float* logits, int64_t stride, const RowArgs& R, const idx_pools* pl, int lg,
                            int32_t* out_tokens, int32_t* out_pools, hipStream_t s) {
  PoolParams p{};
  p.logits = logits;
  p.stride = stride;
  p.rows = R;
  p.pool_log2 = lg;
  p.topk = pl->topk_pools;
  p.init_pools = pl->init_pools;
  p.local_pools = pl->local_pools;
  p.out_tokens = out_tokens;
  p.out_pools = out_pools;
  hipLaunchKernelGGL(pool_topk_kernel<kPoolThreads>, dim3(R.num_rows), dim3(kPoolThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? IDX_OK : fail(IDX_EHIP, "kernel launch failed");
}

// Argument checks shared by the two decode top-k entry points.
idx_status check_decode_topk(const idx_cache* cache, const idx_rows* rows, const uint16_t* q, const float* w,
                             int heads, int k, const int32_t* out, CacheArgs& C, RowArgs& R) {
  idx_status st = check_cache(cache, C);
  if (st != IDX_OK) return st;
  if ((st = check_rows(rows, true, R)) != IDX_OK) return st;
  if (R.kind != IDX_ROWS_DECODE) return fail(IDX_EINVAL, "idx_decode_topk takes DECODE rows");
  if ((st = check_table(rows, R, C)) != IDX_OK) return st;
  if ((st = check_queries(q, w, heads)) != IDX_OK) return st;
  if (!out) return fail(IDX_EINVAL, "out is null");
  if (k < 1) return fail(IDX_EINVAL, "k must be >= 1");
  if (k > kMaxK) return fail(IDX_EUNSUPPORTED, "k must be <= 4096");
  if (group_bound(R, pick_rg(R)) > kMaxGroups) return fail(IDX_EUNSUPPORTED, "too many row groups in one launch (limit 2048)");
  return IDX_OK;
}

// Decode scorer into row logits scratch_stride(R) apart.
idx_status launch_decode_scorer(const CacheArgs& C, const RowArgs& R, const uint16_t* q, const float* w,
                                int heads, float* logits, int32_t* header, hipStream_t s) {
  const int rg = pick_rg(R);
  ScoreParams p{};
  p.cache = C;
  p.rows = R;
  p.q = q;
  p.w = w;
  p.heads = heads;
  p.logits = logits;
  p.logits_stride = scratch_stride(R);
  p.header = header;
  p.num_groups = static_cast<int32_t>(group_bound(R, rg));
  if (dispatch_score(p, score_grid(R, rg), s) != hipSuccess) return fail(IDX_EHIP, "kernel launch failed");
  return IDX_OK;
}

// Scorer into the scratch's row logits (after its 256-byte header), then
// top-k of each row (the kernel boundary orders the two); long rows' chunk
// candidates follow the row logits.
idx_status run_decode_topk(const CacheArgs& C, const RowArgs& R, const uint16_t* q, const float* w, int heads,
                           int k, int32_t* out, uint8_t* ws, int32_t* header, hipStream_t s) {
  float* logits = reinterpret_cast<float*>(ws + scratch_offset());
  idx_status st = IDX_OK;
  if (R.max_keys > 0 && (st = launch_decode_scorer(C, R, q, w, heads, logits, header, s)) != IDX_OK) return st;
  return launch_topk(logits, scratch_stride(R), R, k, out, ws + decode_ws_bytes(R), s);
}

// This device's address of the static scratch (looked up once per device,
// with that device current; the array's host-side name is not a device
// address).
idx_status static_scratch(uint8_t*& out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(IDX_EHIP, "hipGetDevice failed");
  if (dev >= kMaxDevices) return fail(IDX_EUNSUPPORTED, "device ordinal above 63");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return fail(IDX_EHIP, "hipGetSymbolAddress of the static scratch failed");
    addr[dev] = p;
  }
  out = static_cast<uint8_t*>(addr[dev]);
  return IDX_OK;
}

}  // namespace
}  // namespace idx

using namespace idx;

extern "C" {

int64_t idx_num_rows(const idx_rows* rows) { return rows_count(rows); }

size_t idx_workspace_bytes(int32_t op, const idx_cache* cache, const idx_rows* rows, int32_t heads,
                           int32_t k) {
  RowArgs R;
  if (op == IDX_OP_CACHE_WRITE) {
    CacheArgs C;
    return check_cache(cache, C) == IDX_OK ? kStatusBytes : 0;
  }
  if (op == IDX_OP_TOPK) {
    if (check_rows(rows, false, R) != IDX_OK) return 0;
    if (k < 1 || k > kMaxK) return 0;
    return kStatusBytes + topk_chunk_bytes(R, k);
  }
  if (op == IDX_OP_POOL_TOPK) return check_rows(rows, false, R) == IDX_OK ? kStatusBytes : 0;
  CacheArgs C;
  if (check_cache(cache, C) != IDX_OK || check_rows(rows, true, R) != IDX_OK) return 0;
  if (heads < 1 || heads > kMaxHeads) return 0;
  if (op == IDX_OP_LOGITS) return kStatusBytes;
  if (op == IDX_OP_DECODE_TOPK) {
    if (R.kind != IDX_ROWS_DECODE || k < 1 || k > kMaxK) return 0;
    return decode_ws_bytes(R) + topk_chunk_bytes(R, k);
  }
  if (op == IDX_OP_DECODE_POOL_TOPK) return R.kind == IDX_ROWS_DECODE ? decode_ws_bytes(R) : 0;
  return 0;
}

idx_status idx_logits_paged(const idx_cache* cache, const idx_rows* rows, const uint16_t* q,
                            const float* w, int32_t heads, float* logits, int64_t logits_stride,
                            void* workspace, size_t workspace_bytes, void* stream) {
  CacheArgs C;
  RowArgs R;
  idx_status st = check_cache(cache, C);
  if (st != IDX_OK) return st;
  if ((st = check_rows(rows, true, R)) != IDX_OK) return st;
  if ((st = check_table(rows, R, C)) != IDX_OK) return st;
  if ((st = check_queries(q, w, heads)) != IDX_OK) return st;
  if (!logits || logits_stride < 0) return fail(IDX_EINVAL, "logits is null or logits_stride < 0");
  if (R.kind == IDX_ROWS_DECODE && logits_stride < R.max_keys) return fail(IDX_EINVAL, "logits_stride < max_seq_len / compress_ratio");
  if ((st = check_ws(workspace, workspace_bytes, kStatusBytes)) != IDX_OK) return st;
  const int rg = pick_rg(R);
  if (group_bound(R, rg) > kMaxGroups) return fail(IDX_EUNSUPPORTED, "too many row groups in one launch (limit 2048)");
  if (R.num_rows == 0 || R.max_keys == 0) return IDX_OK;
  ScoreParams p{};
  p.cache = C;
  p.rows = R;
  p.q = q;
  p.w = w;
  p.heads = heads;
  p.logits = logits;
  p.logits_stride = logits_stride;
  p.header = static_cast<int32_t*>(workspace);
  p.num_groups = static_cast<int32_t>(group_bound(R, rg));
  const hipError_t e = dispatch_score(p, score_grid(R, rg), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? IDX_OK : fail(IDX_EHIP, "kernel launch failed");
}

idx_status idx_cache_write(const idx_cache* cache, const uint16_t* k, int64_t k_stride,
                           const int64_t* slot_mapping, int64_t num_tokens, void* workspace,
                           size_t workspace_bytes, void* stream) {
  CacheArgs C;
  idx_status st = check_cache(cache, C);
  if (st != IDX_OK) return st;
  if (!k || !slot_mapping) return fail(IDX_EINVAL, "k or slot_mapping is null");
  if ((reinterpret_cast<uintptr_t>(k) & 15) != 0) return fail(IDX_EINVAL, "k must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7) != 0) return fail(IDX_EINVAL, "slot_mapping must be 8-byte aligned");
  if (k_stride < C.head_dim || (k_stride & 7) != 0) return fail(IDX_EINVAL, "k_stride must be >= head_dim and a multiple of 8");
  if (num_tokens < 0) return fail(IDX_EINVAL, "num_tokens < 0");
  if ((st = check_ws(workspace, workspace_bytes, kStatusBytes)) != IDX_OK) return st;
  if (num_tokens == 0) return IDX_OK;
  CacheWriteParams p{};
  p.base = const_cast<uint8_t*>(C.base);
  p.num_pages = C.num_pages;
  p.page_bytes = C.page_bytes;
  p.page_shift = C.page_shift;
  p.k = k;
  p.k_stride = k_stride;
  p.slots = slot_mapping;
  p.num_tokens = num_tokens;
  p.header = static_cast<int32_t*>(workspace);
  const int64_t per_block = (kWriteThreads / kWave) * kWriteGroups * (kWave / (C.head_dim / 8));  // tokens per workgroup
  const int64_t grid = ceil_div(num_tokens, per_block);
  if (grid > 0x7FFFFFFF) return fail(IDX_EUNSUPPORTED, "num_tokens too large for one launch");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool mx = C.fmt == IDX_FMT_MXFP4;
  if (mx) hipLaunchKernelGGL((cache_write_kernel<128, true>), dim3(grid), dim3(kWriteThreads), 0, s, p);
  else if (C.head_dim == 128) hipLaunchKernelGGL((cache_write_kernel<128, false>), dim3(grid), dim3(kWriteThreads), 0, s, p);
  else if (C.head_dim == 64) hipLaunchKernelGGL((cache_write_kernel<64, false>), dim3(grid), dim3(kWriteThreads), 0, s, p);
  else hipLaunchKernelGGL((cache_write_kernel<32, false>), dim3(grid), dim3(kWriteThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? IDX_OK : fail(IDX_EHIP, "kernel launch failed");
}

idx_status idx_topk(const float* logits, int64_t logits_stride, const idx_rows* rows, int32_t k,
                    int32_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  RowArgs R;
  idx_status st = check_rows(rows, false, R);
  if (st != IDX_OK) return st;
  if (!logits || !out || logits_stride < 0) return fail(IDX_EINVAL, "logits or out is null, or logits_stride < 0");
  if (k < 1) return fail(IDX_EINVAL, "k must be >= 1");
  if (k > kMaxK) return fail(IDX_EUNSUPPORTED, "k must be <= 4096");
  if (R.kind == IDX_ROWS_DECODE && logits_stride < R.max_keys) return fail(IDX_EINVAL, "logits_stride < max_seq_len / compress_ratio");
  if ((st = check_ws(workspace, workspace_bytes, kStatusBytes + topk_chunk_bytes(R, k))) != IDX_OK) return st;
  if (R.num_rows == 0) return IDX_OK;
  return launch_topk(logits, logits_stride, R, k, out, static_cast<uint8_t*>(workspace) + kStatusBytes,
                     static_cast<hipStream_t>(stream));
}

idx_status idx_decode_topk(const idx_cache* cache, const idx_rows* rows, const uint16_t* q,
                           const float* w, int32_t heads, int32_t k, int32_t* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  CacheArgs C;
  RowArgs R;
  idx_status st = check_decode_topk(cache, rows, q, w, heads, k, out, C, R);
  if (st != IDX_OK) return st;
  if ((st = check_ws(workspace, workspace_bytes, decode_ws_bytes(R) + topk_chunk_bytes(R, k))) != IDX_OK) return st;
  if (R.num_rows == 0) return IDX_OK;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return run_decode_topk(C, R, q, w, heads, k, out, ws, reinterpret_cast<int32_t*>(ws),
                         static_cast<hipStream_t>(stream));
}

idx_status idx_decode_topk_noalloc(const idx_cache* cache, const idx_rows* rows, const uint16_t* q,
                                   const float* w, int32_t heads, int32_t k, int32_t* out, uint32_t* status,
                                   void* stream) {
  CacheArgs C;
  RowArgs R;
  idx_status st = check_decode_topk(cache, rows, q, w, heads, k, out, C, R);
  if (st != IDX_OK) return st;
  if ((reinterpret_cast<uintptr_t>(status) & 3) != 0) return fail(IDX_EINVAL, "status must be 4-byte aligned");
  if (decode_ws_bytes(R) + topk_chunk_bytes(R, k) > kStaticScratchBytes)
    return fail(IDX_ENOSPC, "rows need more than the 160 MiB static scratch (use idx_decode_topk with a workspace)");
  if (R.num_rows == 0) return IDX_OK;
  uint8_t* ws = nullptr;
  if ((st = static_scratch(ws)) != IDX_OK) return st;
  // the status bits go to the caller's word, or to the scratch header when
  // there is none (nobody reads that one, so it needs no clearing)
  int32_t* header = status ? reinterpret_cast<int32_t*>(status) : reinterpret_cast<int32_t*>(ws);
  return run_decode_topk(C, R, q, w, heads, k, out, ws, header, static_cast<hipStream_t>(stream));
}

idx_status idx_pool_topk(const float* logits, int64_t logits_stride, const idx_rows* rows, const idx_pools* pools,
                         int32_t* out_tokens, int32_t* out_pools, void* workspace, size_t workspace_bytes,
                         void* stream) {
  RowArgs R;
  idx_status st = check_rows(rows, false, R);
  if (st != IDX_OK) return st;
  if (!logits || !out_tokens || logits_stride < 0) return fail(IDX_EINVAL, "logits or out_tokens is null, or logits_stride < 0");
  int lg = 0;
  if ((st = check_pools(pools, R, lg)) != IDX_OK) return st;
  if (R.kind == IDX_ROWS_DECODE && logits_stride < R.max_keys) return fail(IDX_EINVAL, "logits_stride < max_seq_len / compress_ratio");
  if ((st = check_ws(workspace, workspace_bytes, kStatusBytes)) != IDX_OK) return st;
  if (R.num_rows == 0) return IDX_OK;
  return launch_pool_topk(logits, logits_stride, R, pools, lg, out_tokens, out_pools, static_cast<hipStream_t>(stream));
}

idx_status idx_decode_pool_topk(const idx_cache* cache, const idx_rows* rows, const uint16_t* q, const float* w,
                                int32_t heads, const idx_pools* pools, int32_t* out_tokens, int32_t* out_pools,
                                void* workspace, size_t workspace_bytes, void* stream) {
  CacheArgs C;
  RowArgs R;
  // the token top-k's checks with a placeholder k (the pools replace it)
  idx_status st = check_decode_topk(cache, rows, q, w, heads, 1, out_tokens, C, R);
  if (st != IDX_OK) return st;
  int lg = 0;
  if ((st = check_pools(pools, R, lg)) != IDX_OK) return st;
  if ((st = check_ws(workspace, workspace_bytes, decode_ws_bytes(R))) != IDX_OK) return st;
  if (R.num_rows == 0) return IDX_OK;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* logits = reinterpret_cast<float*>(ws + scratch_offset());
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (R.max_keys > 0 && (st = launch_decode_scorer(C, R, q, w, heads, logits, reinterpret_cast<int32_t*>(ws), s)) != IDX_OK)
    return st;
  return launch_pool_topk(logits, scratch_stride(R), R, pools, lg, out_tokens, out_pools, s);
}

idx_status idx_read_device_status(void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags) return fail(IDX_EINVAL, "workspace or flags is null");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return fail(IDX_EHIP, "reading the status word failed");
  if (hipStreamSynchronize(s) != hipSuccess) return fail(IDX_EHIP, "stream synchronisation failed");
  *flags = v;
  const uint32_t zero = 0;
  if (hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess) return fail(IDX_EHIP, "clearing the status word failed");
  if (hipStreamSynchronize(s) != hipSuccess) return fail(IDX_EHIP, "stream synchronisation failed");
  return IDX_OK;
}

const char* idx_status_string(idx_status s) {
  switch (s) {
    case IDX_OK: return "ok";
    case IDX_EINVAL: return "invalid argument";
    case IDX_EUNSUPPORTED: return "unsupported shape or format";
    case IDX_ENOSPC: return "workspace or output capacity too small";
    case IDX_EHIP: return "HIP runtime or launch failure";
    default: return "unknown status";
  }
}

const char* idx_version(void) { return "0.1.0"; }

const char* idx_last_error(void) { return g_last_error; }

}  // extern "C"
