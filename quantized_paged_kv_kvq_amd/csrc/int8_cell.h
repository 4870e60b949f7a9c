// INT8_G64 cell encoder shared by quantize-on-write (append) and the decode kernel's fused
// append, so both write identical bytes.
//
// strata PR #2698, "What it does": int8 codes with one fp16 scale = absmax / 127 per 64 values;
// strata PR #120, "Tests": rounding ties to even.  Every binary32 operation rounds on its own
// (no contraction); the division is the correctly rounded HIP default.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct Int8x4 {
  uint32_t packed;      // codes of the 4 values, value e in byte e
  uint16_t scale_bits;  // fp16 scale of the 64-group (+0 for an all-zero group)
};

// 4 consecutive values of one lane; the 16 lanes of a 64-group are 16 consecutive lanes
// (lanes 16k .. 16k+15), so the group max-abs is an xor-shuffle reduction (max is exact).
static __device__ __forceinline__ Int8x4 int8_encode_x4(const float v[4]) {
#pragma clang fp contract(off)
  float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  am = fmaxf(am, __shfl_xor(am, 8));
  am = fmaxf(am, __shfl_xor(am, 4));
  am = fmaxf(am, __shfl_xor(am, 2));
  am = fmaxf(am, __shfl_xor(am, 1));
  const float s = am / 127.0f;                     // binary32 scale; fp16 is only its storage
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    int q = 0;
    if (am > 0.0f) q = (int)fminf(fmaxf(rintf(v[e] / s), -127.0f), 127.0f);
    packed |= (uint32_t)(q & 0xff) << (8 * e);
  }
  return Int8x4{packed, __builtin_bit_cast(uint16_t, static_cast<_Float16>(am > 0.0f ? s : 0.0f))};
}

}  // namespace kvq
