// Q4_0_H256 cell encoder shared by quantize-on-write (append) and the decode kernel's fused append,
// so both write identical bytes.
//
// strata PR #120, "What"/"How" and strata PR #2698, "Not in this PR": the 256 values are rotated by
// the orthonormal Walsh-Hadamard transform H_256 / 16, then stored as q4_0 blocks of 32 with
// d = (the block's first value of largest magnitude) / -8 and code = clamp(rint(z / d) + 8, 0, 15).
// One wave per cell; lane l holds values 4l .. 4l+3.  Every binary32 operation rounds on its own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// FWHT butterflies in the order of spans 1, 2, 4, ..., 128: spans 1 and 2 inside a lane, spans
// 4..128 between lanes l and l ^ (span / 4).  Each butterfly maps (a, b) -> (a + b, a - b) for the
// pair (i, i + span), exactly as the definition, so the result is bit-identical to any other
// evaluation of the same sequence of stages.
static __device__ __forceinline__ void fwht256_lane(float y[4], int lane) {
#pragma clang fp contract(off)
  float a0 = y[0] + y[1], a1 = y[0] - y[1], a2 = y[2] + y[3], a3 = y[2] - y[3];   // span 1
  y[0] = a0 + a2; y[2] = a0 - a2; y[1] = a1 + a3; y[3] = a1 - a3;                   // span 2
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {                                                // spans 4..128
    const bool upper = (lane & o) != 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float other = __shfl_xor(y[e], o);
      y[e] = upper ? (other - y[e]) : (y[e] + other);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = y[e] * 0.0625f;
}

struct Q4x4 {
  uint8_t b0, b1;       // code bytes of values 4l, 4l+1 and 4l+2, 4l+3 (low nibble first)
  uint16_t d_bits;      // fp16 d of the lane's 32-block (+0 for an all-zero block)
};

// The lane's 4 values (before the rotation) -> their codes and the block's d.
static __device__ __forceinline__ Q4x4 q4h_encode_x4(float y[4], int lane) {
#pragma clang fp contract(off)
  fwht256_lane(y, lane);
  // signed max-abs of each block of 32 (= 8 lanes): the first index with the largest magnitude
  float best = y[0];
  int bidx = 4 * lane;
#pragma unroll
  for (int e = 1; e < 4; ++e)
    if (fabsf(y[e]) > fabsf(best)) { best = y[e]; bidx = 4 * lane + e; }
#pragma unroll
  for (int o = 4; o >= 1; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(bidx, o);
    if (fabsf(ob) > fabsf(best) || (fabsf(ob) == fabsf(best) && oi < bidx)) { best = ob; bidx = oi; }
  }
  const float d = best / -8.0f;
  uint32_t q[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    q[e] = 8;
    if (best != 0.0f) q[e] = (uint32_t)fminf(fmaxf(rintf(y[e] / d) + 8.0f, 0.0f), 15.0f);
  }
  return Q4x4{(uint8_t)(q[0] | (q[1] << 4)), (uint8_t)(q[2] | (q[3] << 4)),
              __builtin_bit_cast(uint16_t, static_cast<_Float16>(best != 0.0f ? d : 0.0f))};
}

}  // namespace kvq
