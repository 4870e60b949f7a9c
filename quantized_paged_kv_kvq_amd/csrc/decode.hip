// Split-K decode / MTP-verify attention over the packed paged cache.
//
// strata PR #2698, "What it does": decode and verify windows dequantise K and V on the fly inside
// the attention kernels, which split the context into parts whose partial results are combined.
// strata PR #120, "How": k8v4 keeps K int8 and unrotated (q is never rotated) and accumulates V
// in the Hadamard-rotated basis, rotating only the output back; "Tests": verify rows carry their
// own causal lengths (per-query step arrays).
//
// Work decomposition (one workgroup = one (sequence, KV head, split) triple):
//   * The query rows of a KV head are its (query token, query head) pairs: n_q * G <= 32 rows,
//     laid out as 16-wide MFMA column tiles (RT = 1 or 2).
//   * Each wave streams every NW-th page of the split: K codes token-major (16 B per lane per
//     64-group: the lane's token is lane % 16), V codes d-major (4 tokens of one head_dim
//     position per 32-bit load), both with 256-byte-coalesced wave accesses.
//   * QK: S^T[token][row] with v_mfma_f32_16x16x32_f16.  int8 codes become fp16 exactly through
//     a byte permute into 0x64xx (= 1024 + byte) and one packed fp16 subtract; q is pre-scaled
//     by a power of two per row so that its bf16 values convert to fp16 exactly.  Each 64-group
//     accumulates separately and is weighted by its (token, group) scale in fp32.
//   * Online softmax in base 2 per row; the row max is shared by the 4 lanes holding a row's 16
//     tokens of a page; the running sum stays per lane until the end.
//   * PV: O^T[d][row] with v_mfma_f32_16x16x16bf16_1k.  The B operand is the S^T accumulator
//     layout itself (lane: 4 tokens x 1 row) after exp2 and multiplication by the (token, group)
//     V scale, split into bf16 hi + lo parts (16 significant bits); the A operand is 4 tokens'
//     codes at one head_dim position converted exactly to bf16 as (code + 128) -- int8 -- or
//     (code + 128) -- 4-bit q4_0 code, value code - 8 -- with the offset removed at the end from
//     the per-group sums of the weights.  Every MFMA tile of 16 head_dim rows lies inside one
//     scale group, so one weight vector per group serves all its tiles.
//   * The NW waves of a workgroup merge (m, l, O) through LDS; the workgroup writes one
//     unnormalised partial.  A second kernel merges the splits with a log-sum-exp combine,
//     normalises, applies H to k8v4 outputs and writes fp32 rows.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }
__device__ __forceinline__ float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float h2f(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }

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

// 4 int8 codes -> bf16 (code + 128), exact (integers below 256 have 8 significant bits).
__device__ __forceinline__ s16x4 codes_to_bf16_biased(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const float f0 = (float)(u & 0xffu), f1 = (float)((u >> 8) & 0xffu), f2 = (float)((u >> 16) & 0xffu),
              f3 = (float)(u >> 24);
  const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  return __builtin_bit_cast(s16x4, make_uint2(lo, hi));
}

// 4-bit codes of 4 tokens (one byte each; nibble picked by the caller) -> bf16 (128 + code), exact.
__device__ __forceinline__ s16x4 nibbles_to_bf16_biased(uint32_t nib) {   // nib: 4 bytes, each 0..15
  const uint32_t lo = __builtin_amdgcn_perm(0x43434343u, nib, 0x05010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x43434343u, nib, 0x05030402u);
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

template <int N>
__device__ __forceinline__ void load_words(uint32_t (&dst)[N], const uint32_t* src) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const uint4 t = reinterpret_cast<const uint4*>(src)[c];
      dst[4 * c] = t.x; dst[4 * c + 1] = t.y; dst[4 * c + 2] = t.z; dst[4 * c + 3] = t.w;
    }
  } else {
    static_assert(N == 2, "scale words come in pairs or multiples of 4");
    const uint2 t = *reinterpret_cast<const uint2*>(src);
    dst[0] = t.x; dst[1] = t.y;
  }
}

template <int D, int VF>
struct PageBuf {
  static constexpr int NG = D / 64;                      // K scale groups
  static constexpr int NVG = VF == 1 ? D / 64 : D / 32;  // V scale groups
  static constexpr int NVW = VF == 1 ? D / 16 : D / 32;  // V dwords per lane
  uint4 k[NG];                // K codes: token lane%16, bytes 64g + 16*(lane/16) .. +15
  uint32_t v[NVW];            // V codes: 4 tokens 4*(lane/16).. at one head_dim position (or pair)
  uint32_t ks[2 * NG];        // fp16 pairs: K scale of token 4*(lane/16) + k, group g is half k*NG + g
  uint32_t vs[2 * NVG];       // V scales likewise
  __device__ __forceinline__ float kscale(int k, int g) const { return half_at(ks, k * NG + g); }
  __device__ __forceinline__ float vscale(int k, int g) const { return half_at(vs, k * NVG + g); }
  static __device__ __forceinline__ float half_at(const uint32_t* w, int i) {
    const uint32_t x = w[i >> 1];
    return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (x >> 16) : (x & 0xffffu))));
  }
};

template <int D, int VF>
__device__ __forceinline__ void load_page(PageBuf<D, VF>& pb, const DecodeArgs& a, int page, int kvh, int lane) {
  constexpr int NG = PageBuf<D, VF>::NG, NVG = PageBuf<D, VF>::NVG;
  const int i16 = lane & 15, j4 = lane >> 4;
  const size_t tile = (size_t)page * a.hkv + kvh;
  const uint8_t* kb = a.k_codes + tile * (16 * D) + (size_t)i16 * D + 16 * j4;
#pragma unroll
  for (int g = 0; g < NG; ++g) pb.k[g] = *reinterpret_cast<const uint4*>(kb + 64 * g);
  const uint8_t* vb = a.v_codes + tile * (16 * (VF == 1 ? D : D / 2)) + (size_t)i16 * 16 + 4 * j4;
#pragma unroll
  for (int t = 0; t < PageBuf<D, VF>::NVW; ++t) pb.v[t] = *reinterpret_cast<const uint32_t*>(vb + 256 * t);
  // scales of this lane's 4 tokens: 4*NG (resp. 4*NVG) consecutive fp16 values
  const uint32_t* ksb = reinterpret_cast<const uint32_t*>(a.k_scales + (tile * 16 + 4 * j4) * NG);
  const uint32_t* vsb = reinterpret_cast<const uint32_t*>(a.v_scales + (tile * 16 + 4 * j4) * NVG);
  load_words<2 * NG>(pb.ks, ksb);
  load_words<2 * NVG>(pb.vs, vsb);
}

template <int D, int RT, int VF>
__device__ __forceinline__ void page_step(const PageBuf<D, VF>& pb, int p, int j4, const int (&Lrow)[RT],
                                          const f16x8 (&qf)[RT][D / 64][2], const float (&qmul)[RT],
                                          float (&m_run)[RT], float (&l_run)[RT],
                                          float (&ls)[RT][VF == 1 ? D / 64 : D / 32], f32x4 (&O)[RT][D / 16]) {
  constexpr int NG = D / 64;
  constexpr int NVG = VF == 1 ? D / 64 : D / 32;
  constexpr int NT = D / 16;

    // ---- QK: S^T[token 4*j4 + k][row] per 64-group
    f32x4 acc[RT][NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const f16x8 a0 = codes_to_f16(pb.k[g].x, pb.k[g].y);
      const f16x8 a1 = codes_to_f16(pb.k[g].z, pb.k[g].w);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        acc[rt][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qf[rt][g][0], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        acc[rt][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qf[rt][g][1], acc[rt][g], 0, 0, 0);
      }
    }
    const int tok0 = p * KVQ_PAGE_SIZE + 4 * j4;

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float s[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float v = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) v += acc[rt][g][k] * pb.kscale(k, g);
        s[k] = (tok0 + k < Lrow[rt]) ? v * qmul[rt] : kNegInf;
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[rt], mx);
      const float m_use = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_use);
      m_run[rt] = m_new;
      float pk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pk[k] = __builtin_amdgcn_exp2f(s[k] - m_use);
      l_run[rt] = l_run[rt] * alpha + ((pk[0] + pk[1]) + (pk[2] + pk[3]));
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < NT; ++t) O[rt][t] *= alpha;
#pragma unroll
        for (int g = 0; g < NVG; ++g) ls[rt][g] *= alpha;
      }

      // ---- PV per V scale group
#pragma unroll
      for (int g = 0; g < NVG; ++g) {
        float pw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pw[k] = (tok0 + k < Lrow[rt]) ? pk[k] * pb.vscale(k, g) : 0.0f;
        ls[rt][g] += (pw[0] + pw[1]) + (pw[2] + pw[3]);
        s16x4 bhi, blo;
        split_bf16(pw, bhi, blo);
        if constexpr (VF == 1) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {              // tiles 4g .. 4g+3 (head_dim 64g .. 64g+63)
            const int t = 4 * g + tt;
            const s16x4 av = codes_to_bf16_biased(pb.v[t]);
            O[rt][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bhi, O[rt][t], 0, 0, 0);
            O[rt][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, blo, O[rt][t], 0, 0, 0);
          }
        } else {
          const uint32_t w = pb.v[g];                  // pair rows 16g + i16: d = 32g + 2*i16 (+1)
          const s16x4 alo = nibbles_to_bf16_biased(w & 0x0f0f0f0fu);
          const s16x4 ahi = nibbles_to_bf16_biased((w >> 4) & 0x0f0f0f0fu);
          O[rt][2 * g] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, bhi, O[rt][2 * g], 0, 0, 0);
          O[rt][2 * g] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, blo, O[rt][2 * g], 0, 0, 0);
          O[rt][2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bhi, O[rt][2 * g + 1], 0, 0, 0);
          O[rt][2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, blo, O[rt][2 * g + 1], 0, 0, 0);
        }
      }
    }

}

template <int D, int RT, int VF, int NW>
__global__ __launch_bounds__(NW * 64, RT == 1 ? 2 : 1) void k_decode_split(const DecodeArgs a) {
  constexpr int NG = D / 64;
  constexpr int NVG = VF == 1 ? D / 64 : D / 32;
  constexpr int NT = D / 16;                                // PV tiles of 16 head_dim rows
  constexpr int RA = 16 * RT;                               // allocated rows
  constexpr float kOff = VF == 1 ? 128.0f : 136.0f;         // bias carried by the V A-operand

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i16 = lane & 15, j4 = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;

  const int h0 = a.head_off[kvh];
  const int G = a.head_off[kvh + 1] - h0;
  const int R = a.n_q * G;
  const int cap = a.max_pages * KVQ_PAGE_SIZE;
  const int seq_len = clampi(a.seq_lens[b], 0, cap);
  int Lmax = 0;
  for (int t = 0; t < a.n_q; ++t)
    Lmax = max(Lmax, a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + t], 0, cap) : seq_len);
  const int npages = (Lmax + KVQ_PAGE_SIZE - 1) / KVQ_PAGE_SIZE;
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(p_begin + a.pages_per_split, npages);
  float* part = a.part + ((size_t)(b * a.hkv + kvh) * a.n_splits + split) * (RA * (D + 2));
  if (R == 0) return;
  if (p_begin >= p_end) {                                   // nothing visible in this split
    if (threadIdx.x < RA) { part[2 * threadIdx.x] = kNegInf; part[2 * threadIdx.x + 1] = 0.0f; }
    return;
  }

  // ---- per-row state; lane's column is row r = 16*rt + i16
  int Lrow[RT];
  f16x8 qf[RT][NG][2];
  float qmul[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 16 * rt + i16;
    const bool valid = r < R;
    const int t = valid ? r / G : 0;
    const int hq = a.head_list[h0 + (valid ? r % G : 0)];
    Lrow[rt] = valid ? (a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + t], 0, cap) : seq_len) : 0;
    const uint16_t* qp = a.q + (((size_t)b * a.n_q + t) * a.n_q_heads + hq) * D + 16 * j4;
    float mx = 0.0f;
    uint4 raw[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      raw[g][0] = *reinterpret_cast<const uint4*>(qp + 64 * g);
      raw[g][1] = *reinterpret_cast<const uint4*>(qp + 64 * g + 8);
      if (!valid) { raw[g][0] = make_uint4(0, 0, 0, 0); raw[g][1] = make_uint4(0, 0, 0, 0); }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w[4] = {raw[g][h].x, raw[g][h].y, raw[g][h].z, raw[g][h].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mx = fmaxf(mx, fmaxf(fabsf(bf16f(w[e] & 0xffffu)), fabsf(bf16f(w[e] >> 16))));
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    int ex = 0;
    if (mx > 0.0f) { frexpf(mx, &ex); ex = 15 - ex; }        // max * 2^ex in [2^14, 2^15)
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w[4] = {raw[g][h].x, raw[g][h].y, raw[g][h].z, raw[g][h].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[rt][g][h][2 * e] = (_Float16)ldexpf(bf16f(w[e] & 0xffffu), ex);
          qf[rt][g][h][2 * e + 1] = (_Float16)ldexpf(bf16f(w[e] >> 16), ex);
        }
      }
    qmul[rt] = ldexpf(a.scale_log2, -ex);
  }

  float m_run[RT], l_run[RT], ls[RT][NVG];
  f32x4 O[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.0f;
#pragma unroll
    for (int g = 0; g < NVG; ++g) ls[rt][g] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) O[rt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int* bt_row = a.bt + (size_t)b * a.max_pages;
  PageBuf<D, VF> b0, b1;
  int p = p_begin + wv;
  if (p < p_end) load_page<D, VF>(b0, a, clampi(bt_row[p], 0, a.num_pages - 1), kvh, lane);
  while (p < p_end) {
    if (p + NW < p_end) load_page<D, VF>(b1, a, clampi(bt_row[p + NW], 0, a.num_pages - 1), kvh, lane);
    page_step<D, RT, VF>(b0, p, j4, Lrow, qf, qmul, m_run, l_run, ls, O);
    p += NW;
    if (p >= p_end) break;
    if (p + NW < p_end) load_page<D, VF>(b0, a, clampi(bt_row[p + NW], 0, a.num_pages - 1), kvh, lane);
    page_step<D, RT, VF>(b1, p, j4, Lrow, qf, qmul, m_run, l_run, ls, O);
    p += NW;
  }

  // ---- per-wave totals: row sums over the 4 lane groups; remove the V operand bias
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] += __shfl_xor(l_run[rt], 16);
    l_run[rt] += __shfl_xor(l_run[rt], 32);
#pragma unroll
    for (int g = 0; g < NVG; ++g) {
      ls[rt][g] += __shfl_xor(ls[rt][g], 16);
      ls[rt][g] += __shfl_xor(ls[rt][g], 32);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int g = VF == 1 ? t / 4 : t / 2;
      O[rt][t] -= kOff * ls[rt][g];
    }
  }

  // ---- merge the NW waves through LDS (halving rounds)
  if constexpr (NW > 1) {
    __shared__ float lds_o[(NW / 2) * RT * NT * 4 * 64];
    __shared__ float lds_ml[(NW / 2) * RT * 2 * 64];
#pragma unroll
    for (int half = NW / 2; half >= 1; half >>= 1) {
      if (wv >= half && wv < 2 * half) {
        const int slot = wv - half;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int k = 0; k < 4; ++k) lds_o[(((slot * RT + rt) * NT + t) * 4 + k) * 64 + lane] = O[rt][t][k];
          lds_ml[((slot * RT + rt) * 2 + 0) * 64 + lane] = m_run[rt];
          lds_ml[((slot * RT + rt) * 2 + 1) * 64 + lane] = l_run[rt];
        }
      }
      __syncthreads();
      if (wv < half) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float mo = lds_ml[((wv * RT + rt) * 2 + 0) * 64 + lane];
          const float lo = lds_ml[((wv * RT + rt) * 2 + 1) * 64 + lane];
          const float M = fmaxf(m_run[rt], mo);
          const float Mu = M == kNegInf ? 0.0f : M;
          const float c1 = __builtin_amdgcn_exp2f(m_run[rt] - Mu), c2 = __builtin_amdgcn_exp2f(mo - Mu);
          m_run[rt] = M;
          l_run[rt] = l_run[rt] * c1 + lo * c2;
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int k = 0; k < 4; ++k)
              O[rt][t][k] = O[rt][t][k] * c1 + lds_o[(((wv * RT + rt) * NT + t) * 4 + k) * 64 + lane] * c2;
        }
      }
      __syncthreads();
    }
  }
  if (wv != 0) return;

  // ---- write the workgroup's partial: rows r < R, layout [RA][2] (m, l) then [RA][D]
  float* po = part + 2 * RA;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 16 * rt + i16;
    if (r >= R) continue;
    if (j4 == 0) { part[2 * r] = m_run[rt]; part[2 * r + 1] = l_run[rt]; }
    float* row = po + (size_t)r * D;
    if constexpr (VF == 1) {
#pragma unroll
      for (int t = 0; t < NT; ++t)   // lane holds d = 16t + 4*j4 + k
        *reinterpret_cast<float4*>(row + 16 * t + 4 * j4) = make_float4(O[rt][t][0], O[rt][t][1], O[rt][t][2], O[rt][t][3]);
    } else {
#pragma unroll
      for (int g = 0; g < NVG; ++g) {  // tiles 2g (even d) / 2g+1 (odd d): d = 32g + 8*j4 + 2k (+1)
        const f32x4 e = O[rt][2 * g], o = O[rt][2 * g + 1];
        *reinterpret_cast<float4*>(row + 32 * g + 8 * j4) = make_float4(e[0], o[0], e[1], o[1]);
        *reinterpret_cast<float4*>(row + 32 * g + 8 * j4 + 4) = make_float4(e[2], o[2], e[3], o[3]);
      }
    }
  }
}

// Log-sum-exp combine of the split partials of one row; k8v4 rows are rotated back by H.
template <int D, bool ROT>
__global__ __launch_bounds__(256) void k_decode_combine(const DecodeArgs a, int row_alloc) {
  __shared__ float w_s[1024];
  __shared__ float red[256];
  __shared__ float acc_s[1024];
  const int r = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int h0 = a.head_off[kvh];
  const int G = a.head_off[kvh + 1] - h0;
  if (r >= a.n_q * G) return;
  const int t = r / G, hq = a.head_list[h0 + r % G];
  const size_t stride = (size_t)row_alloc * (D + 2);
  const float* base = a.part + (size_t)(b * a.hkv + kvh) * a.n_splits * stride;
  const int S = a.n_splits;

  float mx = kNegInf;
  for (int s = tid; s < S; s += 256) {
    const float l = base[s * stride + 2 * r + 1];
    if (l > 0.0f) mx = fmaxf(mx, base[s * stride + 2 * r]);
  }
  red[tid] = mx;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float den = 0.0f;
  for (int s = tid; s < S; s += 256) {
    const float l = base[s * stride + 2 * r + 1];
    const float w = l > 0.0f ? __builtin_amdgcn_exp2f(base[s * stride + 2 * r] - M) : 0.0f;
    w_s[s] = w;
    den += w * l;
  }
  red[tid] = den;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float total = red[0];
  constexpr int TPR = D / 4;                   // threads per row (float4 each)
  constexpr int SG = 256 / TPR;                // split groups
  const int c4 = tid % TPR, sg = tid / TPR;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s = sg; s < S; s += SG) {
    const float w = w_s[s];
    if (w == 0.0f) continue;
    const float4 v = *reinterpret_cast<const float4*>(base + s * stride + 2 * row_alloc + (size_t)r * D + 4 * c4);
    acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
  }
  acc_s[sg * D + 4 * c4 + 0] = acc.x; acc_s[sg * D + 4 * c4 + 1] = acc.y;
  acc_s[sg * D + 4 * c4 + 2] = acc.z; acc_s[sg * D + 4 * c4 + 3] = acc.w;
  __syncthreads();
  const float inv = total > 0.0f ? 1.0f / total : 0.0f;
  for (int d = tid; d < D; d += 256) {
    float v = 0.0f;
    for (int g = 0; g < SG; ++g) v += acc_s[g * D + d];
    acc_s[d] = v * inv;
  }
  __syncthreads();
  if constexpr (ROT) {                         // y <- H y with H = H_256 / 16, spans 1 .. 128
    for (int h = 1; h < D; h <<= 1) {
      float nv = 0.0f;
      const int d = tid;
      if (d < D) {
        const float me = acc_s[d], other = acc_s[d ^ h];
        nv = (d & h) ? (other - me) : (me + other);
      }
      __syncthreads();
      if (d < D) acc_s[d] = nv;
      __syncthreads();
    }
  }
  float* out = a.out + (((size_t)b * a.n_q + t) * a.n_q_heads + hq) * D;
  for (int d = tid; d < D; d += 256) out[d] = ROT ? acc_s[d] * 0.0625f : acc_s[d];
}

template <int D, int RT, int VF, int NW>
hipError_t launch_t(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  dim3 grid(plan.n_splits, a.hkv, a.batch);
  k_decode_split<D, RT, VF, NW><<<grid, dim3(NW * 64), 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid(16 * RT, a.hkv, a.batch);
  k_decode_combine<D, VF == 2><<<cgrid, dim3(256), 0, s>>>(a, 16 * RT);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int head_dim, int hkv, int batch, int max_pages, int max_rows) {
  DecodePlan p{};
  p.row_tiles = max_rows <= 16 ? 1 : 2;
  p.waves = 4;
  const long total = (long)batch * hkv * max_pages;
  const long target = 2L * device_cu_count();
  long pps = (total + target - 1) / target;
  if (const char* env = getenv("KVQ_DECODE_PPS")) pps = atol(env);
  if (pps < 4) pps = 4;
  long ns = (max_pages + pps - 1) / pps;
  if (ns > 1024) { pps = (max_pages + 1023) / 1024; ns = (max_pages + pps - 1) / pps; }
  if (ns < 1) ns = 1;
  p.pages_per_split = (int)pps;
  p.n_splits = (int)ns;
  p.part_bytes = (size_t)batch * hkv * ns * (16 * p.row_tiles) * (head_dim + 2) * sizeof(float);
  return p;
}

hipError_t launch_decode(int v_fmt, int D, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  const bool q4 = v_fmt == KVQ_FMT_Q4_0_H256;
  const int rt = plan.row_tiles;
  if (q4) return rt == 1 ? launch_t<256, 1, 2, 4>(plan, a, s) : launch_t<256, 2, 2, 4>(plan, a, s);
  switch (D) {
    case 64: return rt == 1 ? launch_t<64, 1, 1, 4>(plan, a, s) : launch_t<64, 2, 1, 4>(plan, a, s);
    case 128: return rt == 1 ? launch_t<128, 1, 1, 4>(plan, a, s) : launch_t<128, 2, 1, 4>(plan, a, s);
    case 256: return rt == 1 ? launch_t<256, 1, 1, 4>(plan, a, s) : launch_t<256, 2, 1, 4>(plan, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
