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

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (global_load_lds) with counted waits
// ---------------------------------------------------------------------------

// One direct global -> LDS load: lane i's `size` bytes at gptr land at LDS
// byte address lds + size * i.  Written as inline assembly so that the
// compiler's own wait-count tracking, which cannot tell LDS buffers
// apart and would wait for every request before any LDS read, stays out of
// it; the waits below count these loads instead.  (An asm load also makes any
// wait the compiler computes for its own loads stricter, never weaker.)
// Each load sets m0, which nothing else in this library keeps live.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is named as clobbered on purpose
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds) : "memory", "m0");
}
// The same with a wave-uniform base in scalar registers and a per-lane byte
// offset (global address sbase + voff; no immediate offset), so that a
// page's address arithmetic runs on the scalar unit.
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
// The same two with the non-temporal hint (data read once: the caches need
// not keep it).
__device__ __forceinline__ void lds_dma16_s_nt(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_s_nt(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef const __attribute__((address_space(3))) uint8_t* lds_ptr;
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)p)));
}

// s_waitcnt for vector memory only (vmcnt <= n; the gfx9 encoding keeps
// vmcnt in bits [3:0] and [15:14] and leaves expcnt and lgkmcnt at their
// maxima).  The builtin keeps the compiler's wait-count model in step (it
// learns that its own older loads are complete); the empty asm keeps LDS
// reads of the DMA'd data from moving above the wait.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_all_loads() { wait_vmcnt<0>(); }

// s_waitcnt lgkmcnt(0): every LDS (and scalar memory) access of the wave has
// completed, e.g. before a direct load overwrites LDS the wave was reading.
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  asm volatile("" ::: "memory");
}

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

// Block-wide min and max of a float over NT threads (NaNs are ignored, as
// by fminf / fmaxf) with one barrier: DPP within 16-lane rows, lane reads
// across the rows, one LDS slot per wave.  `sm` holds 2 NT/64 ints that no
// thread may write again before the caller's next barrier.
template <int NT>
__device__ __forceinline__ void block_min_max(float& lo, float& hi, int* sm) {
  auto dpp = [](float v, int ctrl) -> float {
    const int i = __float_as_int(v);
    switch (ctrl) {
      case 0xB1: return __int_as_float(__builtin_amdgcn_update_dpp(i, i, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
      case 0x4E: return __int_as_float(__builtin_amdgcn_update_dpp(i, i, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
      case 0x141: return __int_as_float(__builtin_amdgcn_update_dpp(i, i, 0x141, 0xF, 0xF, false));  // row_half_mirror
      default: return __int_as_float(__builtin_amdgcn_update_dpp(i, i, 0x140, 0xF, 0xF, false));  // row_mirror
    }
  };
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ctrl = c == 0 ? 0xB1 : c == 1 ? 0x4E : c == 2 ? 0x141 : 0x140;
    lo = fminf(lo, dpp(lo, ctrl));
    hi = fmaxf(hi, dpp(hi, ctrl));
  }
  auto lane_f = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  lo = fminf(fminf(lane_f(lo, 0), lane_f(lo, 16)), fminf(lane_f(lo, 32), lane_f(lo, 48)));
  hi = fmaxf(fmaxf(lane_f(hi, 0), lane_f(hi, 16)), fmaxf(lane_f(hi, 32), lane_f(hi, 48)));
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sm[wid] = __float_as_int(lo);
    sm[NT / kWave + wid] = __float_as_int(hi);
  }
  __syncthreads();
  lo = __int_as_float(sm[0]);
  hi = __int_as_float(sm[NT / kWave]);
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) {
    lo = fminf(lo, __int_as_float(sm[w]));
    hi = fmaxf(hi, __int_as_float(sm[NT / kWave + w]));
  }
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

// Range [begin, end) of part `i` when `total` items are split into `parts`
// contiguous ranges of floor or ceil(total / parts) items (the first
// total % parts get one more).  32-bit arithmetic: one unsigned division.
__device__ __forceinline__ void even_split(uint32_t total, uint32_t parts, uint32_t i, int& begin, int& end) {
  const uint32_t q = total / parts;
  const uint32_t r = total - q * parts;
  begin = static_cast<int>(q * i + (i < r ? i : r));
  end = begin + static_cast<int>(q) + (i < r ? 1 : 0);
}

// Key count of grid row (b, i) of a decode batch: position + 1 for real
// tokens, 0 for padded slots; clamped to [0, max_len], then divided by the
// compress ratio (rounded down) for a compressed index cache.
__device__ __forceinline__ int decode_row_len(int seq, int dl, int i, int max_len, int ratio) {
  if (i >= dl) return 0;
  int L = seq - dl + i + 1;
  L = L < 0 ? 0 : L;
  L = L > max_len ? max_len : L;
  return ratio == 1 ? L : L / ratio;
}

// Stored keys of a request of `seq` tokens (clamped to [0, max_len]).
__device__ __forceinline__ int request_keys(int seq, int max_len, int ratio) {
  seq = seq > max_len ? max_len : (seq < 0 ? 0 : seq);
  return ratio == 1 ? seq : seq / ratio;
}

}  // namespace idx
