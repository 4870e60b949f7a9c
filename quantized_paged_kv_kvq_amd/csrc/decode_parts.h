// Device pieces shared by the decode kernels: exact MFMA operands of int8 codes (fp16 values; bf16
// values biased by 128), the hi / lo split of the softmax weights into bf16 MFMA operands, and, for
// Hadamard-rotated q4_0 stores (strata PR #120, "What"/"How": V rotated by H = H_256/16 and stored in
// q4_0; the attention output is rotated back), the biased bf16 operand of 4 tokens' 4-bit codes and
// the back-rotation of a partial output row.
#pragma once

#include "device_util.h"

namespace kvq {

// 8 int8 codes (two dwords, code e in byte e) -> 8 exact fp16 values.
__device__ __forceinline__ f16x8 codes_to_f16(uint32_t w0, uint32_t w1) {
  const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;     // biased: code + 128
  const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2 p0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u0, 0x05010400u)) - off;
  const f16x2 p1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u0, 0x05030402u)) - off;
  const f16x2 p2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u1, 0x05010400u)) - off;
  const f16x2 p3 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u1, 0x05030402u)) - off;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 4 int8 codes (code e in byte e) -> 4 exact fp16 values.
__device__ __forceinline__ f16x4 codes_to_f16x4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;                                 // biased: code + 128
  const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2 p0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u)) - off;
  const f16x2 p1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u)) - off;
  return f16x4{p0[0], p0[1], p1[0], p1[1]};
}

// 4 q4_0 codes (code e, 0..15, in byte e) -> 4 exact fp16 values code - 8.
__device__ __forceinline__ f16x4 nibbles_to_f16x4(uint32_t nib) {
  const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};              // 0x64nn reads 1024 + nn
  const f16x2 p0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, nib, 0x05010400u)) - off;
  const f16x2 p1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, nib, 0x05030402u)) - off;
  return f16x4{p0[0], p0[1], p1[0], p1[1]};
}

// fp16 parts of the products x0 * d0 and x1 * d1 (x fp32; d the fp16 in half H of its word when S
// is 1, the fp32 word itself when S is 0): .x = [hi0 | hi1] with hi the product rounded to fp16, .y =
// [lo0 | lo1] with lo the product minus hi rounded to fp16, each from one v_fma_mix (its fma is exact
// before the one rounding), so hi + lo keeps about 22 significant bits.  The leading wait state
// covers an x written by a transcendental instruction just before: the compiler pads that hazard
// for its own instructions but not for inline assembly.
template <int S0, int H0, int S1, int H1>
__device__ __forceinline__ uint2 mix_parts2(float x0, uint32_t d0, float x1, uint32_t d1) {
  uint32_t h, l;
  asm("s_nop 0\n\t"
      "v_fma_mixlo_f16 %0, %2, %3, 0 op_sel:[0,%c6,0] op_sel_hi:[0,%c7,0]\n\t"
      "v_fma_mixhi_f16 %0, %4, %5, 0 op_sel:[0,%c8,0] op_sel_hi:[0,%c9,0]\n\t"
      "v_fma_mixlo_f16 %1, %2, %3, -%0 op_sel:[0,%c6,0] op_sel_hi:[0,%c7,1]\n\t"
      "v_fma_mixhi_f16 %1, %4, %5, -%0 op_sel:[0,%c8,1] op_sel_hi:[0,%c9,1]"
      : "=&v"(h), "=&v"(l)
      : "v"(x0), "v"(d0), "v"(x1), "v"(d1), "n"(S0 ? H0 : 0), "n"(S0), "n"(S1 ? H1 : 0), "n"(S1));
  return make_uint2(h, l);
}

// 4 int8 codes -> bf16 (code + 128), exact (integers below 256 have 8 significant bits).
__device__ __forceinline__ s16x4 codes_to_bf16_biased(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const float f0 = (float)(u & 0xffu), f1 = (float)((u >> 8) & 0xffu), f2 = (float)((u >> 16) & 0xffu),
              f3 = (float)(u >> 24);
  const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  return __builtin_bit_cast(s16x4, make_uint2(lo, hi));
}

// Split x into bf16 hi (truncated) + bf16 lo (rounded): hi + lo carries 16 significant bits.
__device__ __forceinline__ void split_bf16(const float x[4], s16x4& hi, s16x4& lo) {
  uint32_t hb[4];
  float lf[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hb[e] = __float_as_uint(x[e]) & 0xffff0000u;
    lf[e] = x[e] - __uint_as_float(hb[e]);
  }
  hi = __builtin_bit_cast(s16x4, make_uint2(__builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u),
                                            __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u)));
  const uint32_t l0 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lf[0]) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lf[1]) << 16);
  const uint32_t l1 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lf[2]) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lf[3]) << 16);
  lo = __builtin_bit_cast(s16x4, make_uint2(l0, l1));
}

// 4-bit codes of 4 tokens (one byte each; nibble picked by the caller) -> bf16 (128 + code), exact.
__device__ __forceinline__ s16x4 nibbles_to_bf16_biased(uint32_t nib) {   // nib: 4 bytes, each 0..15
  const uint32_t lo = __builtin_amdgcn_perm(0x43434343u, nib, 0x05010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x43434343u, nib, 0x05030402u);
  return __builtin_bit_cast(s16x4, make_uint2(lo, hi));
}

__device__ __forceinline__ uint32_t word_of(const uint4& q, int k) {
  return k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w;
}

// One part of the hi/lo split, as the bf16 B operand and as the fp32 values it represents: the
// truncated bf16 hi part (lo_mask == 0) or the truncated bf16 part of the remainder x - hi
// (lo_mask == ~0).  hi + lo keeps 16 significant bits of x.
__device__ __forceinline__ void split_bf16_select(const float x[4], uint32_t lo_mask, s16x4& part, float used[4]) {
  uint32_t b[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t xb = __float_as_uint(x[e]);
    b[e] = __float_as_uint(x[e] - __uint_as_float(xb & 0xffff0000u & lo_mask)) & 0xffff0000u;
    used[e] = __uint_as_float(b[e]);
  }
  part = __builtin_bit_cast(s16x4, make_uint2(__builtin_amdgcn_perm(b[1], b[0], 0x07060302u),
                                              __builtin_amdgcn_perm(b[3], b[2], 0x07060302u)));
}

// y <- sum over butterflies of the rotated-basis row held as 64 values by the 4 lanes of a row
// (k8v4): value (t, k) of O is head_dim 32*(t/2) + 8*j4 + 2*k + (t&1).  Applies H = H_256/16.
template <int RT>
__device__ __forceinline__ void hadamard_rows(f32x4 (&O)[RT][16], int lane) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    // bit 0 of head_dim: tile parity
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float e = O[rt][2 * b][k], o = O[rt][2 * b + 1][k];
        O[rt][2 * b][k] = e + o; O[rt][2 * b + 1][k] = e - o;
      }
    // bits 1, 2: k
#pragma unroll
    for (int kb = 1; kb <= 2; kb <<= 1)
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (!(k & kb)) {
            const float x = O[rt][t][k], y = O[rt][t][k | kb];
            O[rt][t][k] = x + y; O[rt][t][k | kb] = x - y;
          }
    // bits 3, 4: lane groups (xor 16, 32)
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const bool upper = (lane & o) != 0;
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float other = o == 16 ? partner16(O[rt][t][k], lane) : partner32(O[rt][t][k], lane);
          O[rt][t][k] = upper ? (other - O[rt][t][k]) : (O[rt][t][k] + other);
        }
    }
    // bits 5..7: block index b = t/2
#pragma unroll
    for (int bb = 1; bb <= 4; bb <<= 1)
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if (!(b & bb))
#pragma unroll
          for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float x = O[rt][2 * b + par][k], y = O[rt][2 * (b | bb) + par][k];
              O[rt][2 * b + par][k] = x + y; O[rt][2 * (b | bb) + par][k] = x - y;
            }
#pragma unroll
    for (int t = 0; t < 16; ++t) O[rt][t] *= 0.0625f;
  }
}

}  // namespace kvq
