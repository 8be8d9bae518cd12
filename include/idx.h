/*
 * idx.h -- C ABI of the sparse-attention lightning-indexer library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library scores every key of a query row's sequence, read from a
 * paged fp8 (or MXFP4) index cache through a block table,
 *
 *     logit[t] = scale_t * sum_h w_h * relu(q_h . k_t),   t < L(row)
 *
 * and selects the top-k key positions per row.  The data layout, the
 * per-token causal lengths, padded decode rows, the exact causal fill and
 * the prefill chunking rules follow the vLLM DeepSeek-V3.2 indexer backend
 * page (indexer.py: DeepSeekV32IndexerDecodeMetadata,
 * _prepare_decode_tensors, split_indexer_prefill_chunks,
 * build_prefill_chunk_metadata) and the vLLM glm5next sparse_indexer helper
 * page (_decode_topk_seq_lens, _fill_short_decode_causal_indices,
 * _gather_workspace_shapes, kv_cache_as_quant_view).
 *
 * Conventions for every entry point:
 *   - Pointers documented "device" must be HIP device memory of the current
 *     device; "host" pointers are ordinary CPU memory.  The library never
 *     allocates device memory and keeps no pointer across calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every GPU entry point only enqueues work on it: no host
 *     synchronisation, no device-to-host reads.
 *   - All argument checks are made on host scalars before anything is
 *     enqueued; on error nothing is enqueued and the status says why.
 *     Values that live in device memory (lengths, page ids) cannot be
 *     checked on the host: lengths are clamped into [0, max_seq_len], a
 *     page id outside [0, num_pages) is never dereferenced (page 0 is read
 *     in its place, so the logits of those 64 positions are unspecified)
 *     and sets bit IDX_DEV_BAD_PAGE of the workspace status word.
 *   - Nothing is thread-safe across calls that share a workspace: such calls
 *     must be ordered on one stream.
 */
#ifndef IDX_H_
#define IDX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t idx_status;

#define IDX_OK 0            /* success */
#define IDX_EINVAL 1        /* null pointer, negative size, bad stride */
#define IDX_EUNSUPPORTED 2  /* valid request outside what the kernels cover */
#define IDX_ENOSPC 3        /* workspace or output capacity too small */
#define IDX_EHIP 4          /* a HIP runtime call or kernel launch failed */

/* Index-cache element formats. */
#define IDX_FMT_FP8_E4M3 0  /* D e4m3fn codes + fp32 per-token scale (4 B, LE) */
#define IDX_FMT_MXFP4 1     /* D/2 packed e2m1 (element 2j = low nibble of byte j)
                               + D/32 ue8m0 block scales */

/* Row kinds. */
#define IDX_ROWS_DECODE 0   /* padded [num_req, next_n] grid of decode tokens */
#define IDX_ROWS_PREFILL 1  /* the query tokens of one prefill chunk */

/* Bits of the device status word (first 4 bytes of a workspace). */
#define IDX_DEV_BAD_PAGE 1u
#define IDX_DEV_BAD_SLOT 2u  /* idx_cache_write: a slot at or past num_pages * page_size */

/*
 * Paged index cache (the `(num_blocks, block_size, head_size)` allocation of
 * the DeepSeek-V3.2 indexer backend).  Token `slot` of page `p` is the row of
 * `row_bytes` bytes at base + p * page_bytes + slot * row_bytes, where
 * row_bytes = head_dim + 4 (fp8) or head_dim/2 + head_dim/32 (MXFP4).
 * page_size is 64, or 256 for the compressed cache of the DeepSeek-V4
 * indexer backend on the same page (its only supported block size).
 */
typedef struct idx_cache {
  const void* base;    /* device, 16-byte aligned, num_pages * page_bytes bytes */
  int64_t num_pages;   /* > 0 */
  int64_t page_bytes;  /* >= page_size * row_bytes, multiple of 16 */
  int32_t page_size;   /* tokens per page: 64 or 256 */
  int32_t head_dim;    /* D: fp8 32, 64 or 128; MXFP4 128 */
  int32_t fmt;         /* IDX_FMT_* */
  int32_t reserved;    /* must be 0 */
} idx_cache;

/*
 * Query rows and where their keys are.
 *
 * DECODE: rows form the padded grid r = b * next_n + i (b < num_req,
 * i < next_n).  Request b has decode_lens[b] real tokens (next_n when
 * decode_lens is NULL) and seq_lens[b] keys, its own tokens included.  Row
 * (b, i) sees L = seq_lens[b] - decode_lens[b] + i + 1 keys (its position
 * + 1, the glm5next page's token-granular length, equal to the
 * DeepSeek-V3.2 page's `L - next_n + j + 1` for full requests); rows with
 * i >= decode_lens[b] are padding (L = 0, empty output).  With q_packed = 0
 * the q/w rows follow the grid; with q_packed = 1 they are the packed decode
 * tokens and grid row (b, i) reads token offset_b + i, offset_b being the
 * sum of decode_lens before b.
 *
 * PREFILL: the chunk covers num_req requests whose query tokens are
 * concatenated (query_start_loc[b] .. query_start_loc[b+1], relative to
 * query_start_loc[0]); rows are the slice [q_begin, q_end) of those tokens,
 * row r reading q/w row r (pass q/w already offset to the chunk's first
 * token).  Query token j of request b sees L = seq_lens[b] -
 * query_len[b] + j + 1 keys and writes logits columns ks + t, ks being the
 * sum of seq_lens before b (the page's cu_seqlen_ks / cu_seqlen_ke window).
 *
 * block_table[b * bt_stride + p] is the physical page of keys
 * [page_size p, page_size (p + 1)) of request b; only the first
 * ceil(L/page_size) entries of a row are read (bt_width * page_size must
 * cover max_seq_len / compress_ratio keys).  max_seq_len is a host upper
 * bound of every seq_lens[b] (no device read), used for sizing; seq_lens
 * beyond it are clamped.
 */
typedef struct idx_rows {
  int32_t kind;                   /* IDX_ROWS_* */
  int32_t num_req;                /* >= 0 */
  const int32_t* block_table;     /* device int32 [num_req * bt_stride] */
  int64_t bt_stride;              /* elements, >= bt_width */
  int32_t bt_width;               /* >= ceil(max_seq_len / compress_ratio / page_size) */
  int32_t max_seq_len;            /* host bound of seq_lens, >= 0 */
  const int32_t* seq_lens;        /* device int32 [num_req] */
  /* DECODE */
  const int32_t* decode_lens;     /* device int32 [num_req] or NULL */
  int32_t next_n;                 /* grid width, >= 1 */
  int32_t q_packed;               /* 0 or 1 */
  /* PREFILL */
  const int32_t* query_start_loc; /* device int32 [num_req + 1] */
  int32_t q_begin;                /* chunk query slice, 0 <= q_begin <= q_end */
  int32_t q_end;
  /* Compressed index cache: 0 or 1 = none; r > 1 (at most 1024) = every
   * cached key stands for r tokens.  seq_lens (and max_seq_len) stay token
   * counts; request b holds seq_lens[b] / r keys, and every row's key count
   * above is divided by r, rounded down (the DeepSeek-V3.2 indexer page
   * divides its decode per-token lengths by compress_ratio and gives a
   * prefill token (start_pos + 1 + offset) // COMPRESS_RATIO keys, its
   * columns starting at the sum of the earlier requests' seq_lens / r). */
  int32_t compress_ratio;
} idx_rows;

/* One prefill chunk, as planned by idx_prefill_chunks. */
typedef struct idx_chunk {
  int32_t req_begin, req_end;     /* requests [req_begin, req_end) (+ request_offset) */
  int32_t q_begin, q_end;         /* slice of the chunk's concatenated query tokens */
  int64_t total_seq_lens;         /* N: logits columns / gathered keys of the chunk */
  int64_t token_begin, token_end; /* the slice in the caller's query-token numbering */
  int32_t skip_kv_gather;         /* 1 when an earlier slice of this chunk gathered its keys */
  int32_t over_budget;            /* 1 when a lone request breaks a budget anyway */
} idx_chunk;

/*
 * Number of grid rows described by `rows`: num_req * next_n (DECODE) or
 * q_end - q_begin (PREFILL); -1 when `rows` is invalid.
 */
int64_t idx_num_rows(const idx_rows* rows);

/* Operation codes for idx_workspace_bytes. */
#define IDX_OP_LOGITS 0
#define IDX_OP_TOPK 1
#define IDX_OP_DECODE_TOPK 2
#define IDX_OP_CACHE_WRITE 3
#define IDX_OP_POOL_TOPK 4         /* k is ignored */
#define IDX_OP_DECODE_POOL_TOPK 5  /* k is ignored */

/*
 * Pool-level selection (the pool_topk / expand_pools_and_append_tail variant
 * of the glm5next sparse_indexer page; the topk_blocks, init_blocks and
 * local_blocks of the MiniMax-M3 mono runner page's indexer).  The pages do
 * not define how a pool is scored; this library's reading: pool p of a row
 * is the pool_size keys [p * pool_size, (p + 1) * pool_size); a row of L keys
 * has n = L / pool_size complete pools and a tail of the last L % pool_size
 * keys; a pool's score is the largest logit of its keys; the first
 * init_pools and the last local_pools complete pools are always kept and
 * count toward topk_pools; the other places go to the highest-scoring
 * complete pools, ties to the lower pool index (-0.0 equal to +0.0); every
 * complete pool is kept when n <= topk_pools.
 */
typedef struct idx_pools {
  int32_t pool_size;    /* keys per pool: 16, 32, 64 or 128 */
  int32_t topk_pools;   /* pools kept per row, 1..512 */
  int32_t init_pools;   /* >= 0 */
  int32_t local_pools;  /* >= 0, init_pools + local_pools <= topk_pools */
} idx_pools;

/*
 * Bytes of device workspace `op` needs for these arguments.  The caller
 * allocates it (256-byte aligned) once and passes it to every call, the way
 * the DeepSeek-V3.2 indexer page's metadata builder preallocates its
 * persistent buffers at fixed addresses so that captured CUDA graphs
 * (UNIFORM_BATCH) can replay over them, and sizes its prefill gather
 * workspace from the model's maximum length (get_max_prefill_buffer_size).
 * Its first 256 bytes hold the device status word (see
 * idx_read_device_status), which must be zero before the first use; nothing
 * else needs clearing, so a workspace can be reused and calls on it
 * captured in a HIP graph.  Calls that share a workspace must not overlap.
 * Returns 0 when the arguments are invalid (for IDX_OP_TOPK and
 * IDX_OP_DECODE_TOPK this includes k outside 1..4096).
 */
size_t idx_workspace_bytes(int32_t op, const idx_cache* cache, const idx_rows* rows,
                           int32_t heads, int32_t k);
/* (IDX_OP_CACHE_WRITE needs only `cache`; rows may be NULL.) */

/*
 * Logits of every row (the scorer the DeepSeek-V3.2 page calls
 * fp8_fp4_paged_mqa_logits).
 *   q      device bf16 bits [rows, heads, head_dim] (row stride heads*head_dim)
 *   w      device fp32 [rows, heads]
 *   heads  1..64
 *   logits device fp32; row r, column c at logits[r * logits_stride + c].
 *          DECODE writes columns [0, L); PREFILL writes [ks, ks + L).
 *          Other columns are left untouched.
 *   logits_stride >= max_seq_len / compress_ratio (DECODE) or >= the chunk's
 *          sum of seq_lens / compress_ratio
 *          (PREFILL, the caller's N), in elements.
 */
idx_status idx_logits_paged(const idx_cache* cache, const idx_rows* rows, const uint16_t* q,
                            const float* w, int32_t heads, float* logits, int64_t logits_stride,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k of rows of logits (the top-k kernels of the DeepSeek-V3.2 indexer
 * page, which take the per-token lengths of DeepSeekV32IndexerDecodeMetadata
 * -- one per row, 1-D or the 2-D next_n grid -- and the exact causal fill of
 * _fill_short_decode_causal_indices on the glm5next sparse_indexer page,
 * applied per row): out[r * k .. r * k + k) receives, in ascending
 * order, the k key positions t < L(r) with the largest logits[r, col0 + t]
 * (col0 = 0 for DECODE, ks for PREFILL), ties going to the lower position,
 * -1 padded.  Rows with L <= k get 0..L-1 (exact causal fill); padded rows
 * (L = 0) get all -1.  -0.0 and +0.0 are equal; NaN inputs are outside the
 * contract.
 *   logits device fp32, same layout as idx_logits_paged's output
 *   k      1..4096
 *   out    device int32 [rows, k]
 * Workspace: idx_workspace_bytes(IDX_OP_TOPK, NULL, rows, 0, k) -- the
 * status word, plus the chunk candidates when rows longer than 32768 keys are
 * split over workgroups (at most 131072 keys per row, and rows x chunks at
 * most 256, chunks = ceil(max keys / 32768)): 2 x rows x chunks x 4096 4-byte
 * values and rows x chunks counts for k <= 2048, 2 x rows x chunks x k 4-byte
 * values above.
 */
idx_status idx_topk(const float* logits, int64_t logits_stride, const idx_rows* rows, int32_t k,
                    int32_t* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode scoring and top-k of every DECODE row (the decode branch of the
 * indexer's forward on the DeepSeek-V3.2 page: paged MQA logits, then top-k
 * per row): two launches on `stream`, the scorer writing each row's logits
 * into the workspace and the selector reading them.  Keys of a request are
 * read once for all its rows; rows with L <= k are causal filled; padded
 * rows get -1.  Output as idx_topk.  The workspace
 * (idx_workspace_bytes(IDX_OP_DECODE_TOPK, ...)) holds the status word,
 * the per-row logits and, for long rows, idx_topk's chunk candidates.
 */
idx_status idx_decode_topk(const idx_cache* cache, const idx_rows* rows, const uint16_t* q,
                           const float* w, int32_t heads, int32_t k, int32_t* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Pool-level top-k of rows of logits (same rows and logits layout as
 * idx_topk).  Per row:
 *   out_tokens[r * W .. r * W + W), W = (topk_pools + 1) * pool_size: the
 *       kept pools' key positions in ascending order, then the tail keys
 *       n * pool_size .. L - 1 (appended whatever their logits), -1 padded;
 *       padded rows (L = 0) are all -1;
 *   out_pools[r * topk_pools ..] (optional, may be NULL): the kept pool
 *       indices, ascending, -1 padded.
 * Rows may hold at most 8192 complete pools (max_seq_len / compress_ratio /
 * pool_size <= 8192, checked on the host).  Workspace:
 * idx_workspace_bytes(IDX_OP_POOL_TOPK, NULL, rows, 0, 0) (the status word).
 */
idx_status idx_pool_topk(const float* logits, int64_t logits_stride, const idx_rows* rows, const idx_pools* pools,
                         int32_t* out_tokens, int32_t* out_pools, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Decode scoring followed by the pool-level selection of every DECODE row
 * (the decode path of the glm5next page's pool indexer: logits on the padded
 * grid, then pool_topk and the expansion): the scorer writes each row's
 * logits into the workspace, the pool selection reads them.  Output as
 * idx_pool_topk.  Workspace: idx_workspace_bytes(IDX_OP_DECODE_POOL_TOPK,
 * cache, rows, heads, 0) (the status word and the row logits).
 */
idx_status idx_decode_pool_topk(const idx_cache* cache, const idx_rows* rows, const uint16_t* q, const float* w,
                                int32_t heads, const idx_pools* pools, int32_t* out_tokens, int32_t* out_pools,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * idx_decode_topk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same output, with the row logits and chunk
 * candidates kept in a static device array of the library instead of a
 * caller workspace.  That array is 160 MiB (enough for 256 grid rows of
 * 131072 keys at k = 2048); arguments that would need more
 * (idx_workspace_bytes(IDX_OP_DECODE_TOPK, ...) > 160 MiB) return
 * IDX_ENOSPC before anything is enqueued.  Each GPU the library runs on
 * holds its own copy from the first call on it until the process ends, and
 * every call on that GPU shares it: calls that overlap on one GPU (two
 * streams, two threads) race.  Nothing is allocated and nothing needs
 * clearing between calls.
 *   status  optional device uint32 (4-byte aligned) that receives the
 *           IDX_DEV_* bits of this call OR-ed in (the caller zeroes it);
 *           NULL: the bits are dropped
 * Other arguments and the output as idx_decode_topk.
 */
idx_status idx_decode_topk_noalloc(const idx_cache* cache, const idx_rows* rows, const uint16_t* q,
                                   const float* w, int32_t heads, int32_t k, int32_t* out, uint32_t* status,
                                   void* stream);

/*
 * Index-cache write: quantise new key tokens and store each token's row in
 * the paged cache at its slot, the step that fills the cache the scorer
 * reads.  The int64 per-token slot mapping is the one the DeepSeek-V3.2
 * indexer page's metadata carries (slot_mapping and its compressed variant)
 * and the MiniMax-M3 mono runner page documents for its page slots: token t
 * goes to row slot % page_size of page slot / page_size (64-token pages, or
 * 256-token pages of the compressed cache); a negative slot (a padding
 * token) is skipped.  The row layouts are those of idx_cache (the glm5next page's
 * _gather_workspace_shapes).  The pages do not print the quantiser; this one
 * follows the per-token absmax / OCP MX block-scale reading:
 *   FP8_E4M3  scale = amax/448 as an fp32 division (1 for an all-zero row),
 *             code_d = e4m3fn(k_d / scale): fp32 division, clamped to +-448,
 *             round to nearest even.
 *   MXFP4     per 32-element block e = floor(log2 amax) - 2, at least -127
 *             (an all-zero block gets -127), ue8m0 byte e + 127, elements
 *             k_d * 2^-e rounded to the nearest e2m1 value (ties to the even
 *             code), saturating at +-6.
 *   Every code keeps the key's sign bit.
 * Arguments:
 *   cache         its base must be writable device memory
 *   k             device bf16 bits [num_tokens, k_stride], the first head_dim
 *                 elements of each row used; 16-byte aligned, k_stride a
 *                 multiple of 8 and >= head_dim
 *   slot_mapping  device int64 [num_tokens], 8-byte aligned; slots must be
 *                 distinct (two tokens on one slot race)
 *   num_tokens    >= 0 (0 enqueues nothing)
 * A slot at or past num_pages * page_size is skipped and sets
 * IDX_DEV_BAD_SLOT in the workspace status word.  Workspace: idx_workspace_bytes(
 * IDX_OP_CACHE_WRITE, cache, NULL, 0, 0) bytes (the status word only).
 */
idx_status idx_cache_write(const idx_cache* cache, const uint16_t* k, int64_t k_stride,
                           const int64_t* slot_mapping, int64_t num_tokens, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Host-only prefill planner (split_indexer_prefill_chunks and
 * build_prefill_chunk_metadata of the DeepSeek-V3.2 indexer page): greedy
 * request chunks with sum(seq_lens) <= workspace_tokens and
 * M * N * 4 <= max_logits_bytes, a lone request taken even when over budget,
 * then M split into max(1, max_logits_bytes/4 / N) slices.  Chunks without
 * keys are dropped.  token_begin/end count from the first request given.
 *   seq_lens, query_lens  host int32 [num_req]
 *   out                   host array of out_cap records; *n_out receives the
 *                         number of chunks (also when IDX_ENOSPC is returned).
 */
idx_status idx_prefill_chunks(const int32_t* seq_lens, const int32_t* query_lens, int32_t num_req,
                              int64_t workspace_tokens, int64_t max_logits_bytes,
                              int32_t request_offset, idx_chunk* out, int32_t out_cap,
                              int32_t* n_out);

/*
 * Copies the workspace's device status word (IDX_DEV_* bits accumulated by
 * the calls that used it) to *flags and clears it.  This call synchronises
 * `stream`; it is meant for tests and diagnostics, not the hot path.
 */
idx_status idx_read_device_status(void* workspace, uint32_t* flags, void* stream);

/*
 * Static description of a status code.  The codes follow how the pages'
 * callers refuse work: the MiniMax-M3 mono runner page raises
 * MonoUnsupported for a configuration its kernels were not built for (here
 * IDX_EUNSUPPORTED), and the DeepSeek-V3.2 indexer backend asserts its
 * supported head sizes, block sizes and single KV head before building
 * metadata (here IDX_EINVAL / IDX_EUNSUPPORTED, returned before anything is
 * enqueued).  Unknown codes give "unknown status".
 */
const char* idx_status_string(idx_status s);

/*
 * Which check the calling thread's most recent failing call tripped (a
 * static string; "" before any failure).  Not reset by successful calls.
 */
const char* idx_last_error(void);

/* Library version, "major.minor.patch". */
const char* idx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H_ */
