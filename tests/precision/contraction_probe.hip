// Test-only probe of the contraction's precision on gfx950 (not part of the
// library): logits of dense fp8 e4m3 keys (codes + fp32 per-token scale)
// against bf16 queries, logit[t] = scale_t * sum_h w_h * relu(q_h . code_t),
// with the q . code products summed by one of three MFMA forms:
//   mode 0: v_mfma_f32_32x32x16_bf16, keys decoded exactly to bf16, q as
//           given (what the library's scorers do);
//   mode 1: v_mfma_scale_f32_32x32x64_f8f6f4 with fp8 x fp8 operands, q as
//           one e4m3 term per element (a per-head power-of-two scale folded
//           into w by the caller);
//   mode 2: the same MFMA with q split into two e4m3 terms q = hi + lo / 16
//           (per-head power-of-two scale, folded into w), the lo term riding
//           the instruction's e8m0 A scale of 2^-4 into the same accumulator.
// One wave per (row, 32-key tile).  Lane l works on key l % 32 of the tile
// and, in each k-step, on the dims of lane half l / 32; A (heads) and B
// (keys) use the same dims per lane, so the contraction covers all 128.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kH = 64;

struct ProbeArgs {
  const uint8_t* codes;     // [L][128] e4m3 key codes
  const float* kscale;      // [L] per-token scales
  const uint16_t* q;        // [R][64][128] bf16 bits   (mode 0)
  const uint8_t* q_hi;      // [R][64][128] e4m3 codes  (modes 1, 2)
  const uint8_t* q_lo;      // [R][64][128] e4m3 codes  (mode 2)
  const float* w;           // [R][64] head weights (times the q scale in modes 1, 2)
  float* out;               // [R][L]
  int L;                    // multiple of 32
  int mode;
};

__global__ __launch_bounds__(64) void probe_kernel(ProbeArgs p) {
  const int tiles = p.L / 32;
  const int r = blockIdx.x / tiles;
  const int t0 = (blockIdx.x % tiles) * 32;
  const int lane = threadIdx.x;
  const int m = lane & 31;
  const int g = lane >> 5;
  const int key = t0 + m;
  v16f acc[2] = {v16f{}, v16f{}};
  if (p.mode == 0) {
    const uint8_t* kc = p.codes + static_cast<int64_t>(key) * kD;
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) {
      const int d0 = 16 * s + 8 * g;
      const uint32_t x0 = *reinterpret_cast<const uint32_t*>(kc + d0);
      const uint32_t x1 = *reinterpret_cast<const uint32_t*>(kc + d0 + 4);
      const u32x4 kb = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x0, 1.0f, true)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x1, 1.0f, true))};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int h = 32 * mt + m;
        const u32x4 qa = *reinterpret_cast<const u32x4*>(p.q + (static_cast<int64_t>(r) * kH + h) * kD + d0);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, qa), __builtin_bit_cast(v8bf, kb),
                                                          acc[mt], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < kD / 64; ++s) {
      const int d0 = 64 * s + 32 * g;
      const v8i kb = *reinterpret_cast<const v8i*>(p.codes + static_cast<int64_t>(key) * kD + d0);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int64_t qo = (static_cast<int64_t>(r) * kH + 32 * mt + m) * kD + d0;
        const v8i hi = *reinterpret_cast<const v8i*>(p.q_hi + qo);
        acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(hi, kb, acc[mt], 0, 0, 0, 127, 0, 127);
        if (p.mode == 2) {
          const v8i lo = *reinterpret_cast<const v8i*>(p.q_lo + qo);
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(lo, kb, acc[mt], 0, 0, 0, 127 - 4, 0, 127);
        }
      }
    }
  }
  // accumulator lane l, register v: key l % 32, head 32 mt + 8 (v / 4) + 4 g + v % 4
  float part = 0.0f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int h = 32 * mt + 8 * (v / 4) + 4 * g + v % 4;
      part += p.w[static_cast<int64_t>(r) * kH + h] * fmaxf(acc[mt][v], 0.0f);
    }
  part += __shfl_xor(part, 32, 64);
  if (g == 0) p.out[static_cast<int64_t>(r) * p.L + key] = part * p.kscale[key];
}

}  // namespace

// Returns 0 on success, 1 for bad arguments, 2 for a launch failure.
extern "C" int probe_logits(const uint8_t* codes, const float* kscale, const uint16_t* q, const uint8_t* q_hi,
                            const uint8_t* q_lo, const float* w, float* out, int rows, int L, int mode,
                            void* stream) {
  if (rows < 1 || L < 32 || L % 32 != 0 || mode < 0 || mode > 2) return 1;
  if (!codes || !kscale || !w || !out) return 1;
  if (mode == 0 && !q) return 1;
  if (mode >= 1 && !q_hi) return 1;
  if (mode == 2 && !q_lo) return 1;
  ProbeArgs a{codes, kscale, q, q_hi, q_lo, w, out, L, mode};
  const int64_t grid = static_cast<int64_t>(rows) * (L / 32);
  if (grid > 0x7FFFFFFF) return 1;
  hipLaunchKernelGGL(probe_kernel, dim3(static_cast<unsigned>(grid)), dim3(64), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
