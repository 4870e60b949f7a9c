// ISO3 constants shared by the encoder, the gather and the attention kernels.
//
// FreeToken PR #398, "What": the eight levels are those of the optimal 3-bit Lloyd-Max quantiser
// of a standard normal variable, scaled by 1/sqrt(128) because a unit 128-vector has per-value
// variance 1/128.  Code k (0..7) selects level k in ascending order.
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

constexpr double kIsoSqrt128 = 11.3137084989847603904135327140;

// binary32 level values: the fp64 quotient rounded once
static __constant__ float kIsoLevels[8] = {
    (float)(-2.1520 / kIsoSqrt128), (float)(-1.3440 / kIsoSqrt128), (float)(-0.7560 / kIsoSqrt128),
    (float)(-0.2451 / kIsoSqrt128), (float)(0.2451 / kIsoSqrt128),  (float)(0.7560 / kIsoSqrt128),
    (float)(1.3440 / kIsoSqrt128),  (float)(2.1520 / kIsoSqrt128)};

// S: the attention kernels feed the levels to fp16 MFMAs as S * level rounded to fp16; with this S
// every one of the eight products lies within 2^-15.9 (relative) of its fp16 rounding, where plain
// fp16 rounding of the levels would cost up to 2^-12.
constexpr float kIsoLevelScale = 1.2495174407958984f;

}  // namespace kvq
