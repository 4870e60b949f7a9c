// Split-K decode / verify attention over ISO3 (or ISO4) K and V stores.
//
// FreeToken PR #398, section What: the ISO attention backend runs its own kernels over the packed
// cells (its file table lists the ISO attention source), and a decode step stores each new token
// already quantised; section Correctness checks that attention against attention over the
// dequantised cells.  "What": an ISO3 cell holds, per 128-value block, the 3-bit codes of the block's
// unit vector after every 4-value group was rotated by one unit quaternion r, and the block's norm
// n.  A key block is k = n * conj(r) (x) c group by group (c: the level values of its codes), so its
// score is <q, k> = n * <r (x) q, c>: the query is rotated once per workgroup and the codes enter
// the product as they are.  Values likewise: sum_j p_j v_j = conj(r) (x) sum_j (p_j n_j) c_j, so the
// weighted sums accumulate in the rotated basis and each split's partial is rotated back once.
//
// Work decomposition: one workgroup = one (sequence, KV head, split of NW * PPW pages); wave w takes
// pages w, w + NW, ... of the split.  The query rows of a KV head (query token, query head) are at
// most 16, one MFMA column each.
//   * The levels enter fp16 MFMAs as S * level rounded to fp16 (within 2^-15.9 of exact for all
//     eight), through a 64-entry LDS table indexed by two adjacent codes: entry p holds the fp16
//     pair (S * level[p & 7], S * level[p >> 3]), so 6 bits of the code stream give two operand
//     values in one LDS read.
//   * QK: S^T[token][row] on v_mfma_f32_16x16x32_f16.  Lane (g = lane / 16, n = lane % 16) holds
//     token n and the 32 codes 32g .. 32g+31 of each block (12 contiguous bytes); the B operand is
//     r (x) q in the same order, scaled per row by a power of two and split into fp16 hi + lo parts.
//     With at most 8 rows the hi parts take MFMA columns 0-7 and the lo parts columns 8-15 and one
//     DPP add per accumulator joins them; with more, each part has its own MFMA.  Every block
//     accumulates separately and is weighted by its token's norm in fp32.
//   * PV: O^T[d][row] on v_mfma_f32_16x16x16_f16.  Lane (g, n) holds tokens 4g .. 4g+3 at head_dim
//     8n .. 8n+7 of each block (3 bytes of each token's cell, inside one 8-byte load); the pair
//     table gives, per token, dims (2k, 2k+1), and byte permutes regroup them into the (token,
//     token) pairs of the A operand.  The B operand is the S^T accumulator layout itself: softmax
//     weight x the token's V block norm, in fp16 hi + lo parts like q.
//   * Online softmax in base 2 with a lazily moved reference max; the waves merge (m, l, O) through
//     LDS; the partial is rotated back by conj(r) and goes to the log-sum-exp combine shared with the
//     other decode kernels.
//
// ISO4 (FreeToken PR #398, "What": the 4-bit sibling, 68 B per 128-value block) runs through the same
// kernel with BITS = 4: sixteen levels, a 256-entry pair table indexed by one code byte (two
// nibbles), 16 code bytes per lane and block for QK and one code word per token for PV, and binary32
// norms.
#include <type_traits>

#include "kvq_internal.h"
#include "device_util.h"
#include "decode_parts.h"
#include "iso_levels.h"

namespace kvq {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

template <int BITS>
constexpr int kBlockBytes = BITS == 3 ? 48 : 64;   // codes of one 128-value block
template <int BITS>
constexpr float kLevelScale = BITS == 3 ? kIsoLevelScale : kIso4LevelScale;
constexpr float kLazy = 8.0f;                   // weights stay below 2^8 between rescalings
// weight x V norm enters fp16 as 2^-9 * p * n / S: with p < 2^8 and n <= 65504 it stays finite
constexpr float kPScale = 1.0f / 512.0f;
constexpr int kBufFlags = 0x00020000;           // buffer resource word 3 (raw 32-bit data)
constexpr int kNonTemporal = 2;                 // streaming loads: each cell is read once

// Launch shapes: waves per workgroup, pages per wave per split, pages each wave keeps in flight
// with head_dim 128 (half as many with head_dim 256, whose pages are twice as large), waves per SIMD
// the registers allow.  Measured on 32 sequences of 4K-32K tokens (head_dim 128): 2 pages in flight
// at 4 waves per SIMD beat 4, 6 or 8 pages at 2-3 waves per SIMD (the kernel is bound by its VALU
// work per page, not by memory latency).
struct IsoShape { int nw, ppw, pd, occ, pps; };   // pps: pages per split (the waves take pages w, w + nw, ...)
constexpr IsoShape kIsoShapes[] = {{4, 16, 2, 2, 64}, {8, 8, 1, 2, 64}, {8, 4, 1, 2, 32}};
constexpr int kNumIsoShapes = (int)(sizeof(kIsoShapes) / sizeof(kIsoShapes[0]));

// KVQ_ISO3_DECODE_SHAPE overrides the choice (for tuning); -1 when unset
int iso_shape_override() {
  static int idx = -2;
  if (idx == -2) {
    idx = -1;
    if (const char* e = getenv("KVQ_ISO3_DECODE_SHAPE")) {
      const int v = atoi(e);
      if (v >= 0 && v < kNumIsoShapes) idx = v;
    }
  }
  return idx;
}

// Hamilton product a (x) u of quaternions (w, x, y, z).
__device__ __forceinline__ void quat_mul(const float a[4], const float u[4], float o[4]) {
  o[0] = a[0] * u[0] - a[1] * u[1] - a[2] * u[2] - a[3] * u[3];
  o[1] = a[0] * u[1] + a[1] * u[0] + a[2] * u[3] - a[3] * u[2];
  o[2] = a[0] * u[2] - a[1] * u[3] + a[2] * u[0] + a[3] * u[1];
  o[3] = a[0] * u[3] + a[1] * u[2] - a[2] * u[1] + a[3] * u[0];
}

// One page of one KV head as a lane holds it (NB = head_dim / 128 blocks per cell).
template <int BITS, int NB>
struct IsoPage {
  static constexpr int NW = BITS == 3 ? 2 * NB : 4 * NB;
  std::conditional_t<BITS == 3, u32x3, u32x4> k[NB];   // K: token lane % 16, codes 32 * (lane / 16) .. +31 of block b
  // V: token 4 * (lane / 16) + j: ISO3 the 8 bytes holding codes 8 * (lane % 16) .. +7, ISO4 the word of them
  std::conditional_t<BITS == 3, u32x2, uint32_t> v[NB][4];
  uint32_t kn[NW];       // norms of tokens 4 * (lane / 16) + j, block b: ISO3 fp16 half j * NB + b, ISO4 word
  uint32_t vn[NW];
  __device__ __forceinline__ float knorm(int j, int b) const {
    return BITS == 3 ? half_at(kn, j * NB + b) : __uint_as_float(kn[j * NB + b]);
  }
  __device__ __forceinline__ float vnorm(int j, int b) const {
    return BITS == 3 ? half_at(vn, j * NB + b) : __uint_as_float(vn[j * NB + b]);
  }
  static __device__ __forceinline__ float half_at(const uint32_t* w, int i) {
    const uint32_t x = w[i >> 1];
    return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (x >> 16) : (x & 0xffffu))));
  }
};

// Loads of one (page, KV head) tile through buffer resources spanning just that tile, so that no
// lane can read outside it.  v_off: byte offset, inside a block's code bytes, of the two words (ISO3)
// or the word (ISO4) that hold this lane's V code bits.
template <int BITS, int NB>
__device__ __forceinline__ void load_iso_page(IsoPage<BITS, NB>& pb, const DecodeArgs& a, int page, int kvh, int g,
                                              int n, int v_off) {
  constexpr int BB = kBlockBytes<BITS>;
  constexpr int CB = NB * BB;
  constexpr int NS = BITS == 3 ? NB : 2 * NB;       // 16-bit norm slots per (token, KV head)
  const size_t tile = (size_t)page * a.hkv + kvh;
  const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.k_codes + tile * (16 * CB)), (short)0,
                                                    16 * CB, kBufFlags);
  const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.v_codes + tile * (16 * CB)), (short)0,
                                                    16 * CB, kBufFlags);
  const auto rkn = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.k_scales + tile * (16 * NS)), (short)0,
                                                     32 * NS, kBufFlags);
  const auto rvn = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.v_scales + tile * (16 * NS)), (short)0,
                                                     32 * NS, kBufFlags);
  if constexpr (BITS == 3) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      pb.k[b] = __builtin_amdgcn_raw_buffer_load_b96(rk, n * CB + BB * b + 12 * g, 0, kNonTemporal);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pb.v[b][j] = __builtin_amdgcn_raw_buffer_load_b64(rv, (4 * g + j) * CB + BB * b + v_off, 0, kNonTemporal);
    if constexpr (NB == 1) {
      const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rkn, 8 * g, 0, kNonTemporal);
      const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(rvn, 8 * g, 0, kNonTemporal);
      pb.kn[0] = x[0]; pb.kn[1] = x[1];
      pb.vn[0] = y[0]; pb.vn[1] = y[1];
    } else {
      static_assert(NB == 2, "head_dim 128 or 256");
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rkn, 16 * g, 0, kNonTemporal);
      const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(rvn, 16 * g, 0, kNonTemporal);
#pragma unroll
      for (int e = 0; e < 4; ++e) { pb.kn[e] = x[e]; pb.vn[e] = y[e]; }
    }
  } else {                          // ISO4: 16 code bytes per lane and block, binary32 norms
#pragma unroll
    for (int b = 0; b < NB; ++b)
      pb.k[b] = __builtin_amdgcn_raw_buffer_load_b128(rk, n * CB + BB * b + 16 * g, 0, kNonTemporal);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pb.v[b][j] = __builtin_amdgcn_raw_buffer_load_b32(rv, (4 * g + j) * CB + BB * b + v_off, 0, kNonTemporal);
#pragma unroll
    for (int h = 0; h < NB; ++h) {  // words j * NB + b of tokens 4g .. 4g+3: 16 NB contiguous bytes
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rkn, 16 * NB * g + 16 * h, 0, kNonTemporal);
      const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(rvn, 16 * NB * g + 16 * h, 0, kNonTemporal);
#pragma unroll
      for (int e = 0; e < 4; ++e) { pb.kn[4 * h + e] = x[e]; pb.vn[4 * h + e] = y[e]; }
    }
  }
}

// fp16 hi + lo parts of 4 values: hi = RNE(x), lo = RNE(x - hi); hi + lo keeps 22 significant bits.
__device__ __forceinline__ void split_f16(const float x[4], f16x4& hi, f16x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = (_Float16)x[e];
    lo[e] = (_Float16)(x[e] - (float)hi[e]);
  }
}

// One page of one wave: QK on MFMA, online softmax, PV on MFMA.
template <int BITS, int D, bool DUP>
__device__ __forceinline__ void iso_page_step(const IsoPage<BITS, D / 128>& pb, int p, int g, bool lo_col, int Lrow,
                                              const f16x8* qb, float qmul, int v_shift,
                                              const uint32_t* lut, float& m_run, float& l_run, f32x4 (&O)[D / 16]) {
  constexpr int NB = D / 128;
  // ---- QK: S^T[token 4g + k][row] per block
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const auto w = pb.k[b];
    // the 32 codes as four groups of 8: ISO3 24-bit groups (code i of the group in bits 3i .. 3i+2),
    // ISO4 words (code i in bits 4i .. 4i+3)
    uint32_t x[4];
    if constexpr (BITS == 3) {
      x[0] = w[0]; x[1] = __builtin_amdgcn_alignbit(w[1], w[0], 24); x[2] = __builtin_amdgcn_alignbit(w[2], w[1], 16);
      x[3] = w[2] >> 8;
    } else {
      x[0] = w[0]; x[1] = w[1]; x[2] = w[2]; x[3] = w[3];
    }
    acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      constexpr int PB = 2 * BITS;                // bits of a code pair = the table index
      constexpr uint32_t PM = (1u << PB) - 1;
      const u32x4 pairs = {lut[x[c] & PM], lut[(x[c] >> PB) & PM], lut[(x[c] >> (2 * PB)) & PM],
                           lut[(x[c] >> (3 * PB)) & PM]};
      const f16x8 av = __builtin_bit_cast(f16x8, pairs);
      constexpr int NP = DUP ? 1 : 2;
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qb[((b * 4 + c) * NP) * 64], acc[b], 0, 0, 0);
      if constexpr (!DUP)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qb[((b * 4 + c) * NP + 1) * 64], acc[b], 0, 0, 0);
    }
    if constexpr (DUP) {          // columns r (hi part of q) and r + 8 (lo part): both get the sum
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[b][k] += dpp_ror8(acc[b][k]);
    }
  }
  const int tok0 = p * KVQ_PAGE_SIZE + 4 * g;
  float s[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float v = acc[0][k] * pb.knorm(k, 0);
#pragma unroll
    for (int b = 1; b < NB; ++b) v = fmaf(acc[b][k], pb.knorm(k, b), v);
    s[k] = (tok0 + k < Lrow) ? v * qmul : kNegInf;
  }
  // Lazy rescaling: the reference max moves only when a score exceeds it by more than 2^kLazy, and
  // O and l are rescaled only then (never while they are still zero).
  const float mx = max_over_row_lanes(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
  const bool move = mx > m_run + kLazy;
  const float m_new = move ? mx : m_run;
  const float m_use = m_new == kNegInf ? 0.0f : m_new;
  const bool rescale = move && m_run != kNegInf;
  const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
  m_run = m_new;
  float pk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) pk[k] = __builtin_amdgcn_exp2f(s[k] - m_use);
  l_run = l_run * alpha + ((pk[0] + pk[1]) + (pk[2] + pk[3]));
  if (__any(rescale)) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) O[t] *= alpha;
  }

  // ---- PV per block: tiles 8b + t' hold head_dim 128b + 8 * (A row) + t'
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    f16x4 bh, bl, bp;
    if constexpr (DUP) {
      // one part per column: a token pair's hi and lo parts of x * norm from four mixed-precision fmas,
      // one packed select per pair (norm (k, b): ISO3 fp16 half (k NB + b) & 1 of word (k NB + b) / 2,
      // ISO4 fp32 word k NB + b)
      constexpr float C = kPScale / kLevelScale<BITS>;
      const float x0 = pk[0] * C, x1 = pk[1] * C, x2 = pk[2] * C, x3 = pk[3] * C;
      uint2 p01, p23;
      if constexpr (BITS == 4) {
        p01 = mix_parts2<0, 0, 0, 0>(x0, pb.vn[b], x1, pb.vn[NB + b]);
        p23 = mix_parts2<0, 0, 0, 0>(x2, pb.vn[2 * NB + b], x3, pb.vn[3 * NB + b]);
      } else if constexpr (NB == 1) {
        p01 = mix_parts2<1, 0, 1, 1>(x0, pb.vn[0], x1, pb.vn[0]);
        p23 = mix_parts2<1, 0, 1, 1>(x2, pb.vn[1], x3, pb.vn[1]);
      } else {
        static_assert(NB == 2, "head_dim 128 or 256");
        p01 = b ? mix_parts2<1, 1, 1, 1>(x0, pb.vn[0], x1, pb.vn[1]) : mix_parts2<1, 0, 1, 0>(x0, pb.vn[0], x1, pb.vn[1]);
        p23 = b ? mix_parts2<1, 1, 1, 1>(x2, pb.vn[2], x3, pb.vn[3]) : mix_parts2<1, 0, 1, 0>(x2, pb.vn[2], x3, pb.vn[3]);
      }
      bp = __builtin_bit_cast(f16x4, lo_col ? make_uint2(p01.y, p23.y) : make_uint2(p01.x, p23.x));
    } else {
      float w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = pk[k] * (pb.vnorm(k, b) * (kPScale / kLevelScale<BITS>));
      split_f16(w, bh, bl);
    }
    uint32_t xv[4];               // code bits of token 4g + j: head_dim 8n .. 8n+7 of block b
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (BITS == 3) {
        const uint64_t pair = ((uint64_t)pb.v[b][j][1] << 32) | pb.v[b][j][0];
        xv[j] = (uint32_t)(pair >> v_shift);
      } else {
        xv[j] = pb.v[b][j];
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {   // dims 8n + 2kk (tile 2kk) and 8n + 2kk + 1 (tile 2kk + 1)
      constexpr int PB = 2 * BITS;
      constexpr uint32_t PM = (1u << PB) - 1;
      uint32_t L[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) L[j] = lut[(xv[j] >> (PB * kk)) & PM];
      const f16x4 a0 = __builtin_bit_cast(f16x4, u32x2{__builtin_amdgcn_perm(L[1], L[0], 0x05040100u),
                                                       __builtin_amdgcn_perm(L[3], L[2], 0x05040100u)});
      const f16x4 a1 = __builtin_bit_cast(f16x4, u32x2{__builtin_amdgcn_perm(L[1], L[0], 0x07060302u),
                                                       __builtin_amdgcn_perm(L[3], L[2], 0x07060302u)});
      f32x4& o0 = O[8 * b + 2 * kk];
      f32x4& o1 = O[8 * b + 2 * kk + 1];
      if constexpr (DUP) {
        o0 = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, bp, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, bp, o1, 0, 0, 0);
      } else {
        o0 = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, bh, o0, 0, 0, 0);
        o0 = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, bl, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, bh, o1, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, bl, o1, 0, 0, 0);
      }
    }
  }
}

template <int BITS, int D, bool DUP, int NW, int PPW, int PD, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void k_decode_iso(const DecodeArgs a) {
  constexpr int NB = D / 128;
  constexpr int NT = D / 16;                        // PV tiles of 16 head_dim rows
  constexpr int NTG = NT / 4;                       // groups of 4 tiles: 4 consecutive head_dim per lane
  constexpr int NL = 1 << (2 * BITS);               // pair-table entries
  // one LDS allocation with the pair table at its start: table addresses then fit the 16-bit offset
  // of the LDS loads, so a lookup's address is the shifted, masked code pair alone (two separate
  // arrays put the table after the merge buffers, past that range, with one more add per lookup).
  // Then the query fragments (B operands of QK, [block][group][part][lane], written by wave 0) and
  // each row's score multiplier, then the merge buffers (half of the tiles at a time).
  constexpr int NP = DUP ? 1 : 2;
  constexpr int kQWords = NB * 4 * NP * 64 * 4;
  __shared__ __align__(16) uint32_t lds[NL + kQWords + 64 + NW * ((NT / 2) * 64 * 4 + 2 * 64)];
  uint32_t* const lut = lds;
  f16x8* const qlds = reinterpret_cast<f16x8*>(lds + NL);
  float* const qmul_lds = reinterpret_cast<float*>(lds + NL + kQWords);
  float* const mrg = reinterpret_cast<float*>(lds + NL + kQWords + 64);

  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  if constexpr (BITS == 3) {
    if (threadIdx.x < 64) {
      const _Float16 lo = (_Float16)(kIsoLevelScale * kIsoLevels[threadIdx.x & 7]);
      const _Float16 hi = (_Float16)(kIsoLevelScale * kIsoLevels[threadIdx.x >> 3]);
      lut[threadIdx.x] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
  } else {
    for (int i = (int)threadIdx.x; i < NL; i += NW * 64) {
      const _Float16 lo = (_Float16)(kIso4LevelScale * kIso4Levels[i & 15]);
      const _Float16 hi = (_Float16)(kIso4LevelScale * kIso4Levels[i >> 4]);
      lut[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
  }

  // ---- rows of this KV head: row r is (query token r / G, query head r % G of the head's list)
  int G, h0;
  if (a.g_uniform > 0) {
    G = a.g_uniform;
    h0 = kvh * G;
  } else {
    h0 = a.head_off[kvh];
    G = a.head_off[kvh + 1] - h0;
  }
  const int R = a.n_q * G;
  const int RA = a.row_alloc;
  const int cap = a.max_pages * KVQ_PAGE_SIZE;
  const bool lo_col = DUP && n >= 8;
  const int r = DUP ? (n & 7) : n;
  const bool valid = r < R;
  const int tq = valid ? r / G : 0, iq = valid ? r % G : 0;
  const int hq = a.g_uniform > 0 ? h0 + iq : a.head_list[h0 + iq];
  const int seq_len = clampi(a.seq_lens[b], 0, cap);
  const int Lrow = valid ? (a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + tq], 0, cap) : seq_len) : 0;

  // ---- q first, then this wave's first PD pages (vector-memory waits are in issue order)
  const int* bt_row = a.bt + (size_t)b * a.max_pages;
  const int p_begin = split * a.pages_per_split;
  const int p0 = p_begin + wv;
  const int p_cap = min(p_begin + a.pages_per_split, a.max_pages) - 1;
  uint4 qraw[NB][4];                                // q[row][128b + 32g + 8c .. +7]
  {
    const uint16_t* qp = a.q + ((size_t)(b * a.n_q + tq) * a.n_q_heads + hq) * D + 32 * g;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int c = 0; c < 4; ++c) qraw[bb][c] = *reinterpret_cast<const uint4*>(qp + 128 * bb + 8 * c);
  }
  // ISO3: first of the two words holding V bits 24n .. 24n+23; ISO4: the word of bits 32n .. 32n+31
  const int v_e = BITS == 3 ? min((24 * n) >> 5, 10) : n;
  const int v_off = 4 * v_e, v_shift = BITS == 3 ? 24 * n - 32 * v_e : 0;
  IsoPage<BITS, NB> buf[PD + 1];
#pragma unroll
  for (int i = 0; i < PD && i < PPW; ++i)
    load_iso_page<BITS, NB>(buf[i], a, clampi(bt_row[min(p0 + i * NW, p_cap)], 0, a.num_pages - 1), kvh, g, n, v_off);

  int Lmax = 0;
  for (int t = 0; t < a.n_q; ++t)
    Lmax = max(Lmax, a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + t], 0, cap) : seq_len);
  const int npages = (Lmax + KVQ_PAGE_SIZE - 1) / KVQ_PAGE_SIZE;
  const int p_end = min(p_begin + a.pages_per_split, npages);
  // partials: m/l [B][Hkv][RA][n_splits][2], then O [B][Hkv][RA][n_splits][D]
  const size_t row0 = (size_t)(b * a.hkv + kvh) * RA;
  float* part_ml = a.part;
  float* part_o = a.part + (size_t)a.batch * a.hkv * RA * a.n_splits * 2;
  if (R == 0) return;
  if (p_begin >= p_end) {                           // nothing visible in this split
    if (a.n_splits == 1) {                          // the only split writes the output: zeros
      for (int i = (int)threadIdx.x; i < R * (D / 4); i += NW * 64)
        *reinterpret_cast<float4*>(a.out + (size_t)decode_out_row(a, b, kvh, i / (D / 4), G, h0) * D +
                                   4 * (i % (D / 4))) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else if ((int)threadIdx.x < R) {
      float* ml = part_ml + ((row0 + threadIdx.x) * a.n_splits + split) * 2;
      ml[0] = kNegInf; ml[1] = 0.0f;
    }
    return;
  }

  // ---- B operands of QK: r (x) q per 4-value group, times 2^ex (max |.| of the row in
  // [2^14, 2^15)), as fp16 hi + lo parts
  const float quat[4] = {a.quat[0], a.quat[1], a.quat[2], a.quat[3]};
  if (wv == 0) {
    float qr[NB][32];
    float mx = 0.0f;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w[4] = {qraw[bb][c].x, qraw[bb][c].y, qraw[bb][c].z, qraw[bb][c].w};
#pragma unroll
        for (int h = 0; h < 2; ++h) {               // groups of dims 8c + 4h .. +3
          const float u[4] = {valid ? bf16f(w[2 * h] & 0xffffu) : 0.0f, valid ? bf16f(w[2 * h] >> 16) : 0.0f,
                              valid ? bf16f(w[2 * h + 1] & 0xffffu) : 0.0f, valid ? bf16f(w[2 * h + 1] >> 16) : 0.0f};
          float o[4];
          quat_mul(quat, u, o);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qr[bb][8 * c + 4 * h + e] = o[e];
            mx = fmaxf(mx, fabsf(o[e]));
          }
        }
      }
    mx = max_over_row_lanes(mx);
    int ex = 0;
    if (mx > 0.0f) { frexpf(mx, &ex); ex = 15 - ex; }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = ldexpf(qr[bb][8 * c + j], ex);
          const _Float16 hi = (_Float16)x, lo = (_Float16)(x - (float)hi);
          if constexpr (DUP) {
            qlds[((bb * 4 + c) * NP) * 64 + lane][j] = lo_col ? lo : hi;
          } else {
            qlds[((bb * 4 + c) * NP) * 64 + lane][j] = hi;
            qlds[((bb * 4 + c) * NP + 1) * 64 + lane][j] = lo;
          }
        }
    qmul_lds[lane] = ldexpf(a.scale_log2 * (1.0f / kLevelScale<BITS>), -ex);
  }

  float m_run = kNegInf, l_run = 0.0f;
  f32x4 O[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) O[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Each wave takes pages p_begin + wv, + NW, ... (at most PPW) and keeps PD pages in flight ahead
  // of the one it processes, in a ring of PD + 1 register buffers; the loop is fully unrolled so
  // every wait on the vector memory counter covers exactly the page about to be processed.
  // Prefetches past the wave's last page re-read that page.
  __syncthreads();                                  // the pair table, the query fragments
  const float qmul = qmul_lds[lane];
  const f16x8* const qb = qlds + lane;
  if (p0 < p_end) {
    const int n_mine = (p_end - 1 - p0) / NW + 1;
    const int p_last = p0 + (n_mine - 1) * NW;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int pc = p0 + i * NW;
      if (i + PD < PPW)
        load_iso_page<BITS, NB>(buf[(i + PD) % (PD + 1)], a,
                                clampi(bt_row[min(pc + PD * NW, p_last)], 0, a.num_pages - 1), kvh, g, n, v_off);
      iso_page_step<BITS, D, DUP>(buf[i % (PD + 1)], pc, g, lo_col, Lrow, qb, qmul, v_shift, lut, m_run, l_run, O);
      if (i + 1 >= n_mine) break;
    }
  }
  l_run = sum_over_row_lanes(l_run);

  // ---- merge the NW waves, half of the tiles at a time: each stores (m, l) and its half of O in LDS,
  // then wave w merges the tile groups w, w + NW, ... of the half (4 tiles = 4 consecutive head_dim of
  // every lane: whole rotation groups)
  constexpr int NTH = NT / 2, NTGH = NTG / 2;        // tiles, tile groups per half
  static_assert(NTH % 4 == 0, "whole tile groups per half");
  float* lds_o = mrg;                               // [wave][tile of the half][lane] x f32x4
  float* lds_ml = mrg + NW * NTH * 64 * 4;          // [wave][m | l][lane]
  lds_ml[(wv * 2 + 0) * 64 + lane] = m_run;
  lds_ml[(wv * 2 + 1) * 64 + lane] = l_run;
  const bool writer = valid && !lo_col;
  // with a single split the workgroup writes the normalised output itself (no combine follows)
  const bool direct = a.n_splits == 1;
  const float cq[4] = {quat[0], -quat[1], -quat[2], -quat[3]};
  float cv[NW];
  float M = kNegInf, l = 0.0f, sc = 0.0f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    if (hf) __syncthreads();                        // the first half is merged
#pragma unroll
    for (int t = 0; t < NTH; ++t)
      *reinterpret_cast<f32x4*>(lds_o + ((wv * NTH + t) * 64 + lane) * 4) = O[hf * NTH + t];
    __syncthreads();
    if (hf == 0) {
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        cv[v] = lds_ml[(v * 2 + 0) * 64 + lane];
        M = fmaxf(M, cv[v]);
      }
      const float Mu = M == kNegInf ? 0.0f : M;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        cv[v] = __builtin_amdgcn_exp2f(cv[v] - Mu);
        l += cv[v] * lds_ml[(v * 2 + 1) * 64 + lane];
      }
      sc = direct ? (l > 0.0f ? 512.0f / l : 0.0f) : 512.0f;   // 512: the weights' 2^-9
      if (!direct && wv == 0 && g == 0 && writer) {
        float* ml = part_ml + ((row0 + r) * a.n_splits + split) * 2;
        ml[0] = M; ml[1] = l;
      }
    }
#pragma unroll
    for (int tg = hf * NTGH; tg < (hf + 1) * NTGH; ++tg) {
      if (tg % NW != wv) continue;
      f32x4 o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const int th = 4 * (tg - hf * NTGH) + q;    // tile of the half
#pragma unroll
        for (int v = 0; v < NW; ++v) acc += cv[v] * *reinterpret_cast<const f32x4*>(lds_o + ((v * NTH + th) * 64 + lane) * 4);
        if constexpr (DUP) {          // column r + 8 holds the lo-part sums of row r
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[k] += dpp_ror8(acc[k]);
        }
        o[q] = acc * sc;
      }
      // tile 4tg + q, element i: head_dim 128 * (tg / 2) + 32g + 8i + 4 * (tg % 2) + q
      if (writer) {
        float* row = (direct ? a.out + (size_t)((b * a.n_q + tq) * a.n_q_heads + hq) * D
                             : part_o + ((row0 + r) * a.n_splits + split) * D) +
                     128 * (tg >> 1) + 32 * g + 4 * (tg & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float u[4] = {o[0][i], o[1][i], o[2][i], o[3][i]};
          float y[4];
          quat_mul(cq, u, y);
          *reinterpret_cast<float4*>(row + 8 * i) = make_float4(y[0], y[1], y[2], y[3]);
        }
      }
    }
  }
}

template <int BITS, int D, bool DUP, int SH>
hipError_t launch_iso_t(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  constexpr IsoShape sh = kIsoShapes[SH];
  constexpr int pd = D == 128 ? sh.pd : (sh.pd + 1) / 2;
  k_decode_iso<BITS, D, DUP, sh.nw, sh.ppw, pd, sh.occ>
      <<<dim3((unsigned)plan.n_splits, a.hkv, a.batch), dim3(sh.nw * 64), 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return plan.n_splits > 1 ? launch_decode_combine(D, plan, a, s) : hipSuccess;   // one split wrote the output
}

template <int BITS, int D, bool DUP, int SH = 0>
hipError_t launch_iso_shape(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  if constexpr (SH + 1 < kNumIsoShapes)
    if (plan.shape != SH) return launch_iso_shape<BITS, D, DUP, SH + 1>(plan, a, s);
  return launch_iso_t<BITS, D, DUP, SH>(plan, a, s);
}

template <int BITS>
hipError_t launch_iso_bits(int D, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  const bool dup = plan.rows <= 8;
  switch (D) {
    case 128: return dup ? launch_iso_shape<BITS, 128, true>(plan, a, s) : launch_iso_shape<BITS, 128, false>(plan, a, s);
    case 256: return dup ? launch_iso_shape<BITS, 256, true>(plan, a, s) : launch_iso_shape<BITS, 256, false>(plan, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

DecodePlan plan_decode_iso(int head_dim, int hkv, int batch, int max_pages, int max_rows) {
  DecodePlan p{};
  p.rows = max_rows;
  p.row_groups = max(1, (max_rows + 7) / 8);        // partial rows: 8 (one MFMA half) or 16
  p.row_tiles = 0;
  // More 64-page splits than CUs: 4-wave workgroups (two share a CU).  Otherwise one 8-wave workgroup
  // per CU (two waves per SIMD), each wave with half the pages: 64-page splits while they fill more
  // than half of the CUs, else 32-page splits.  Measured ISO3 launches for one sequence over two KV
  // heads at head_dim 256 (4x16 / 4x8 / 8x8 / 8x4 waves x pages): 131,072 tokens 33.6 / 31.3 / 30.1 /
  // 38.9 us; 65,536 tokens 32.3 / 22.2 / 28.3 / 21.5 us; 32,768 tokens 31.8 / 21.3 / 27.6 / 20.5 us.
  auto splits_of = [&](int sh) {
    const int pps = kIsoShapes[sh].pps;
    return (max_pages + pps - 1) / pps;
  };
  p.shape = iso_shape_override();
  if (p.shape < 0) {
    const long n64 = (long)splits_of(0) * hkv * batch, cus = device_cu_count();
    p.shape = n64 > cus ? 0 : (2 * n64 > cus ? 1 : 2);
  }
  p.waves = kIsoShapes[p.shape].nw;
  p.pages_per_split = kIsoShapes[p.shape].pps;
  p.n_splits = splits_of(p.shape);
  p.part_bytes = (size_t)batch * hkv * p.n_splits * (8 * p.row_groups) * (head_dim + 2) * sizeof(float);
  return p;
}

hipError_t launch_decode_iso(int bits, int D, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  return bits == 4 ? launch_iso_bits<4>(D, plan, a, s) : launch_iso_bits<3>(D, plan, a, s);
}

}  // namespace kvq
