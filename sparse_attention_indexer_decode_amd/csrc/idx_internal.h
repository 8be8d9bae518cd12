// Internal parameter blocks passed by value to the kernels.
#pragma once

#include <stdint.h>

namespace idx {

// Limits of this build (checked on the host before any launch).
constexpr int kMaxHeads = 64;
constexpr int kMaxGroups = 2048;   // row groups per scorer launch (LDS table)
constexpr int kMaxK = 4096;        // top-k
constexpr int kMaxTopkChunks = 4;  // chunks of a long row split over workgroups
constexpr int kMaxReqPrefill = 256;  // requests per prefill chunk / packed decode batch
constexpr int kStatusBytes = 256;  // workspace header: status word + pad
constexpr int kMaxRatio = 1024;    // compress ratio of a compressed index cache

// Workspace header layout (int32 slots).
constexpr int kHdrStatus = 0;
constexpr uint32_t kStatusBadPage = 1u;  // a block-table entry outside the pool (IDX_DEV_BAD_PAGE)
constexpr uint32_t kStatusBadSlot = 2u;  // a cache-write slot past the pool (IDX_DEV_BAD_SLOT)

struct CacheArgs {
  const uint8_t* base;
  int64_t num_pages;
  int64_t page_bytes;
  int32_t page_shift;  // log2(page_size / 64): a page holds 1 << page_shift 64-key units
  int32_t head_dim;
  int32_t row_bytes;
  int32_t fmt;  // 0 fp8, 1 mxfp4
};

struct RowArgs {
  int32_t kind;  // 0 decode, 1 prefill
  int32_t num_req;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t max_len;   // clamp of seq_lens (uncompressed tokens)
  int32_t ratio;     // compress ratio >= 1: a row of L tokens sees L / ratio keys
  int32_t max_keys;  // max_len / ratio
  const int32_t* seq_lens;
  const int32_t* decode_lens;
  int32_t next_n;
  int32_t q_packed;
  const int32_t* qsl;
  int32_t q_begin;
  int32_t q_end;
  int32_t num_rows;
};

}  // namespace idx
