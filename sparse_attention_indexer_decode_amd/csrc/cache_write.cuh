// Index-cache write for gfx950: quantise new bf16 key tokens and store each
// token's row at its int64 page slot (page = slot / page_size, row = slot %
// page_size, page_size 64 or 256) of the paged cache; negative slots are
// skipped.
//
// Row formats (the ones the scorer reads):
//   fp8    D e4m3fn codes, then the fp32 per-token scale.  scale = amax / 448
//          (1 for an all-zero row), code = e4m3(k / scale) with the quotient
//          an IEEE fp32 division clamped to +-448 and converted to nearest
//          even by the hardware conversion.
//   MXFP4  D/2 bytes of e2m1 pairs (even element in the low nibble), then one
//          ue8m0 byte per 32-element block: e = floor(log2 amax) - 2 (at
//          least -127), byte e + 127, elements k * 2^-e rounded to the
//          nearest e2m1 value (ties to the even code), saturating at 6.
//   The sign bit of every code is the key's.
//
// Work decomposition.  HBM-bound streaming: each lane owns 8 consecutive
// elements of one token (one 16-byte load), D/8 lanes a token, so a token
// group of 64/(D/8) tokens uses every lane's 16-byte load; a wave covers
// kWriteGroups groups with all loads in flight at once.  The per-token (fp8)
// or per-block (MXFP4) absmax is a butterfly over the token's lanes.
#pragma once

#include "device_common.cuh"

namespace idx {

struct CacheWriteParams {
  uint8_t* base;
  int64_t num_pages;
  int64_t page_bytes;
  int32_t page_shift;  // log2(page_size / 64)
  const uint16_t* k;
  int64_t k_stride;  // elements between tokens
  const int64_t* slots;
  int64_t num_tokens;
  int32_t* header;  // workspace status word
};

constexpr int kWriteThreads = 256;
constexpr int kWriteGroups = 4;  // token groups per wave

// Maximum over the `width` lanes of an aligned lane group (width a power of
// two <= 64).
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// e2m1 code magnitude (0..7) of |x| <= 6 and beyond (saturating): the
// thresholds are the midpoints between the values 0, .5, 1, 1.5, 2, 3, 4, 6,
// a midpoint itself going to the even code.
__device__ __forceinline__ uint32_t e2m1_magnitude(float a) {
  return (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
}

// One token group of a wave (64 / (D/8) tokens) from its loaded bf16 bits:
// quantise and store.  Returns whether a live token had a slot past the pool.
template <int D, bool MX>
__device__ __forceinline__ bool write_tokens(const CacheWriteParams& p, bool live, int64_t slot, const u32x4& raw) {
  constexpr int kLanes = D / 8;
  constexpr int kRowBytes = MX ? D / 2 + D / 32 : D + 4;
  const int lane = lane_id();
  const int sub = lane % kLanes;  // this lane's 8 elements: 8 sub .. 8 sub + 7
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(raw[i] << 16);
    f[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));

  const int rows_log2 = 6 + p.page_shift;  // token rows per page: 64 or 256
  const int64_t capacity = p.num_pages << rows_log2;
  const bool bad = live && slot >= capacity;
  const bool store = live && slot >= 0 && slot < capacity;
  uint8_t* row = p.base + (store ? (slot >> rows_log2) * p.page_bytes +
                                       (slot & ((int64_t{1} << rows_log2) - 1)) * kRowBytes
                                 : 0);

  if constexpr (!MX) {
    amax = group_max<kLanes>(amax);
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = fminf(fmaxf(f[4 * h + i] / scale, -448.0f), 448.0f);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], v, true);
      w[h] = static_cast<uint32_t>(v);
    }
    if (store) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(row + 8 * sub);
      dst[0] = w[0];
      dst[1] = w[1];
      if (sub == 0) *reinterpret_cast<float*>(row + D) = scale;
    }
  } else {
    amax = group_max<4>(amax);  // the four lanes of a 32-element block
    const uint32_t E = (__float_as_uint(amax) >> 23) & 0xFFu;
    const int e = E == 0 ? -127 : max(static_cast<int>(E) - 129, -127);
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);  // 2^-e
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t sign = (__float_as_uint(f[i]) >> 31) << 3;
      word |= (e2m1_magnitude(fabsf(f[i] * inv)) | sign) << (4 * i);
    }
    // the four block scales gathered by the token's first lane
    const uint32_t sb = static_cast<uint32_t>(e + 127);
    const int base_lane = lane - sub;
    const uint32_t s1 = __shfl(sb, base_lane + 4, 64);
    const uint32_t s2 = __shfl(sb, base_lane + 8, 64);
    const uint32_t s3 = __shfl(sb, base_lane + 12, 64);
    if (store) {
      *reinterpret_cast<uint32_t*>(row + 4 * sub) = word;
      if (sub == 0) *reinterpret_cast<uint32_t*>(row + D / 2) = sb | (s1 << 8) | (s2 << 16) | (s3 << 24);
    }
  }
  return bad;
}

// Each wave covers kWriteGroups consecutive token groups and issues all of
// their loads before quantising any, so that 4 KiB per wave are in flight.
template <int D, bool MX>
__global__ __launch_bounds__(kWriteThreads) void cache_write_kernel(CacheWriteParams p) {
  constexpr int kLanes = D / 8;             // lanes per token
  constexpr int kTokensPerWave = kWave / kLanes;
  static_assert(!MX || D == 128, "MXFP4 rows hold 128 dims");
  const int lane = lane_id();
  const int sub = lane % kLanes;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kWriteThreads / kWave) + (threadIdx.x >> 6);
  int64_t slot[kWriteGroups];
  u32x4 raw[kWriteGroups];
  bool live[kWriteGroups];
#pragma unroll
  for (int u = 0; u < kWriteGroups; ++u) {
    const int64_t t = (wave * kWriteGroups + u) * kTokensPerWave + lane / kLanes;
    live[u] = t < p.num_tokens;
    slot[u] = -1;
    raw[u] = u32x4{0u, 0u, 0u, 0u};
    if (live[u]) {
      slot[u] = p.slots[t];
      raw[u] = *reinterpret_cast<const u32x4*>(p.k + t * p.k_stride + 8 * sub);
    }
  }
  bool bad = false;
#pragma unroll
  for (int u = 0; u < kWriteGroups; ++u) bad |= write_tokens<D, MX>(p, live[u], slot[u], raw[u]);
  // every lane of the wave is here (no early exit): one report per wave
  if (__any(bad) && lane == 0) atomicOr(reinterpret_cast<uint32_t*>(p.header) + kHdrStatus, kStatusBadSlot);
}

}  // namespace idx
