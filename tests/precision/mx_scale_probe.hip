// Test-only probe (not part of the library): how gfx950's scaled fp4 -> bf16
// conversion reads its fp32 scale operand.  For each 16-bit word holding two
// ue8m0 block-scale bytes (low byte, high byte), lane t converts two words
// that hold all 16 e2m1 codes with the scale operand given as the word
// shifted left by 23 (the low byte lands in the fp32 exponent field, bit 0
// of the high byte in the sign) and by 15 (the high byte in the exponent
// field, the low byte in the mantissa), each at the four nibble-pair
// selectors: 16 bf16 pairs per word.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(64) void mx_scale_kernel(const uint16_t* words, uint32_t* out, int n) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  if (t >= n) return;
  const uint32_t w = words[t];
  const uint32_t codes[2] = {0x76543210u, 0xFEDCBA98u};
  const float f[2] = {__uint_as_float(w << 23), __uint_as_float(w << 15)};
  uint32_t* o = out + static_cast<int64_t>(t) * 16;
#pragma unroll
  for (int form = 0; form < 2; ++form) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      o[form * 8 + c * 4 + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[c], f[form], 0));
      o[form * 8 + c * 4 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[c], f[form], 1));
      o[form * 8 + c * 4 + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[c], f[form], 2));
      o[form * 8 + c * 4 + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[c], f[form], 3));
    }
  }
}

}  // namespace

// words: device uint16 [n]; out: device uint32 [n][2 forms][2 code words][4
// selectors].  Returns 0 on success, 1 for bad arguments, 2 for a launch
// failure.
extern "C" int probe_mx_scale(const uint16_t* words, uint32_t* out, int n, void* stream) {
  if (!words || !out || n < 1 || n > (1 << 20)) return 1;
  hipLaunchKernelGGL(mx_scale_kernel, dim3((n + 63) / 64), dim3(64), 0, static_cast<hipStream_t>(stream), words,
                     out, n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
