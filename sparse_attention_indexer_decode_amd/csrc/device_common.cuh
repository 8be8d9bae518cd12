// Device helpers shared by the indexer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "idx_internal.h"

namespace idx {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16-byte load/store unit
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kPage = 64;  // tokens per cache page

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Order-preserving map from float to uint32: larger float -> larger key.
// -0.0 is first folded onto +0.0 so that both compare equal.
__device__ __forceinline__ uint32_t ordered_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Wave-wide inclusive prefix sum (DPP: shifts within 16-lane rows, then
// row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Block-wide exclusive prefix sum over NT threads (NT a multiple of 64).
// `sm` holds NT/64 ints.  Returns the exclusive prefix; `total` receives the
// block sum.  Contains two __syncthreads().
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int& total, int* sm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int x = wave_inclusive_scan(v);
  if (lane == kWave - 1) sm[wid] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    int s = sm[w];
    before += (w < wid) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

__device__ __forceinline__ int block_sum_int(int v, int* sm, int nt) {
  // generic block sum for any multiple-of-64 block size
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  if (lane == 0) sm[wid] = v;
  __syncthreads();
  int tot = 0;
  for (int w = 0; w < nt / kWave; ++w) tot += sm[w];
  __syncthreads();
  return tot;
}

// Key count of grid row (b, i) of a decode batch: position + 1 for real
// tokens, 0 for padded slots; clamped to [0, max_len].
__device__ __forceinline__ int decode_row_len(int seq, int dl, int i, int max_len) {
  if (i >= dl) return 0;
  int L = seq - dl + i + 1;
  L = L < 0 ? 0 : L;
  return L > max_len ? max_len : L;
}

}  // namespace idx
