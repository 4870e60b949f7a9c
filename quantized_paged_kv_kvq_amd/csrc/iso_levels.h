// ISO3 / ISO4 constants shared by the encoders, the gathers and the attention kernels.
//
// FreeToken PR #398, "What": the eight ISO3 levels are those of the optimal 3-bit Lloyd-Max
// quantiser of a standard normal variable, scaled by 1/sqrt(128) because a unit 128-vector has
// per-value variance 1/128.  Code k selects level k in ascending order.  ISO4, the 4-bit sibling
// ("What": 4.25 bits per value), takes the sixteen levels of the 16-level Lloyd-Max quantiser of
// a standard normal variable to 4 decimals (the page does not list them).
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

static __constant__ float kIso4Levels[16] = {
    (float)(-2.7326 / kIsoSqrt128), (float)(-2.0690 / kIsoSqrt128), (float)(-1.6180 / kIsoSqrt128),
    (float)(-1.2562 / kIsoSqrt128), (float)(-0.9423 / kIsoSqrt128), (float)(-0.6568 / kIsoSqrt128),
    (float)(-0.3880 / kIsoSqrt128), (float)(-0.1284 / kIsoSqrt128), (float)(0.1284 / kIsoSqrt128),
    (float)(0.3880 / kIsoSqrt128),  (float)(0.6568 / kIsoSqrt128),  (float)(0.9423 / kIsoSqrt128),
    (float)(1.2562 / kIsoSqrt128),  (float)(1.6180 / kIsoSqrt128),  (float)(2.0690 / kIsoSqrt128),
    (float)(2.7326 / kIsoSqrt128)};

// The ISO4 counterpart of kIsoLevelScale: all sixteen products lie within 2^-13.4 (relative) of
// their fp16 roundings (plain fp16 rounding of the levels: 2^-11.4).
constexpr float kIso4LevelScale = 1.1301089525222778f;

}  // namespace kvq
