// MTP verify over k8v4 cells (int8-g64 K, Hadamard-rotated q4_0 V) with more than 8 query rows per
// KV head: split-K partials in the layout every decode kernel writes, finished by the log-sum-exp
// combine.
//
// strata PR #120, "What"/"How": K stays int8 and unrotated (q is never rotated), V is stored rotated
// by H = H_256/16 in q4_0 and accumulated in the rotated basis; only the output is rotated back.
// "Tests": verify rows carry their own causal lengths (per-query step arrays).
//
// Work decomposition: one workgroup of 8 waves per (sequence, KV head, split of 4 * PPP pages).  The
// waves form 4 pairs; pair p takes pages p, p + 4, ... of the split, and the two waves of a pair
// split head_dim: wave half h holds values 128h .. 128h + 127 of every row.
//   * QK: each wave contracts its half (K scale groups 2h, 2h + 1) on v_mfma_f32_16x16x32_f16 with
//     exact fp16 codes and the pre-scaled query, weights the two groups by their scales and writes
//     its partial scores to LDS (an LDS flag per wave publishes each step).  With two row tiles wave h
//     adds the two halves' partials of row tile h, runs its online softmax and hands the weights and
//     the rescale factor to its partner the same way; with one row tile both waves run it (half 0's
//     partial first, so they agree bit for bit).
//   * PV: each wave builds the exact V operand (code - 8) * d only for its four 32-value groups and
//     accumulates its half of the rows in the rotated basis (two fp16 MFMAs per tile and row tile, as
//     below).
// Per wave this is half the operand work of a wave holding whole rows, and about 200 registers, so
// two waves share a SIMD and keep two pages in flight each.
// Pair 0 builds the query fragments in LDS for all pairs.  The 4 pairs merge (m, l, O) through LDS,
// pair rt taking row tile rt; the Hadamard back-rotation of the merged partial takes its span-128
// stage between the two halves through LDS and spans 1..64 inside each wave.
#include <type_traits>

#include "kvq_internal.h"
#include "device_util.h"
#include "int8_cell.h"
#include "decode_parts.h"
#include "q4h_cell.h"

namespace kvq {
namespace {

constexpr int kD = 256;
constexpr int kPairs = 4;                 // wave pairs per workgroup
constexpr int kWaves = 2 * kPairs;
constexpr int kPD = 2;                    // pages in flight ahead of the one processed
constexpr float kLazyLog2 = 8.0f;         // weights stay below 2^8 between rescalings
constexpr uint32_t kSpinLimit = 1u << 24;  // polls of a partner's flag before giving up

// One wave's half of one (page, KV head) tile.
struct HalfPage {
  uint4 k[2];        // K: 16-byte chunk 4 * (2h + gl) + j4 of slot lane % 16 (gl = 0, 1)
  uint4 v;           // V: word gl = 4 tokens 4 * j4 .. at one pair row of V group 4h + gl
  uint32_t ks[4];    // fp16 K scales, word k = token 4 * j4 + k: (group 2h, group 2h + 1)
  uint32_t vs[8];    // fp16 V scales, token 4 * j4 + k: groups 4h .. 4h + 3 in words 2k, 2k + 1
  __device__ __forceinline__ float kscale(int k, int gl) const {
    return h2f((uint16_t)(gl ? (ks[k] >> 16) : (ks[k] & 0xffffu)));
  }
  __device__ __forceinline__ float vscale(int k, int gl) const {
    const uint32_t w = vs[2 * k + (gl >> 1)];
    return h2f((uint16_t)((gl & 1) ? (w >> 16) : (w & 0xffffu)));
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// Device-scope loads (past the CU's L1): a half page this wave wrote cells into comes back with them.
__device__ __forceinline__ uint32_t rsrc_load(const void* base, uint32_t off, int bytes, uint32_t* out) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
  if (bytes == 16) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0x10);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0x10);
    out[0] = v[0]; out[1] = v[1];
  }
  return 0;
}

template <bool DEV>
__device__ __forceinline__ void load_half(HalfPage& hp, const DecodeArgs& a, int page, int kvh, int h, int lane) {
  const int i16 = lane & 15, j4 = lane >> 4;
  const size_t tile = (size_t)page * a.hkv + kvh;
  const uint8_t* kb = a.k_codes + tile * (16 * kD);                   // chunk c of slot t at (16c + t) * 16
  const uint8_t* vb = a.v_codes + tile * (16 * (kD / 2));
  const uint8_t* ksb = reinterpret_cast<const uint8_t*>(a.k_scales + tile * 16 * 4);   // [slot][4 groups]
  const uint8_t* vsb = reinterpret_cast<const uint8_t*>(a.v_scales + tile * 16 * 8);   // [slot][8 groups]
  const uint32_t koff0 = 16u * (64 * (2 * h) + lane), koff1 = 16u * (64 * (2 * h + 1) + lane);
  const uint32_t voff = 16u * (64 * h + 4 * i16 + j4);
  if constexpr (!DEV) {
    hp.k[0] = stream_load(kb + koff0);
    hp.k[1] = stream_load(kb + koff1);
    hp.v = stream_load(vb + voff);
    const uint4 s0 = ld16(ksb + 32 * j4), s1 = ld16(ksb + 32 * j4 + 16);   // tokens 4 j4 .. + 3, 8 B each
    hp.ks[0] = h ? s0.y : s0.x; hp.ks[1] = h ? s0.w : s0.z;
    hp.ks[2] = h ? s1.y : s1.x; hp.ks[3] = h ? s1.w : s1.z;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint2 w = ld8(vsb + 16 * (4 * j4 + k) + 8 * h);
      hp.vs[2 * k] = w.x; hp.vs[2 * k + 1] = w.y;
    }
  } else {
    uint32_t t[4];
    rsrc_load(kb, koff0, 16, t); hp.k[0] = make_uint4(t[0], t[1], t[2], t[3]);
    rsrc_load(kb, koff1, 16, t); hp.k[1] = make_uint4(t[0], t[1], t[2], t[3]);
    rsrc_load(vb, voff, 16, t); hp.v = make_uint4(t[0], t[1], t[2], t[3]);
    uint32_t s[8];
    rsrc_load(ksb, 32 * j4, 16, s);
    rsrc_load(ksb, 32 * j4 + 16, 16, s + 4);
    hp.ks[0] = s[h]; hp.ks[1] = s[2 + h]; hp.ks[2] = s[4 + h]; hp.ks[3] = s[6 + h];
#pragma unroll
    for (int k = 0; k < 4; ++k) rsrc_load(vsb, 16 * (4 * j4 + k) + 8 * h, 8, hp.vs + 2 * k);
  }
}

// q fragments (B operand of QK) in LDS: [rt][g][half of the group][lane] x 16 bytes
template <int RT>
struct QFrag {
  const f16x8* p;
  __device__ __forceinline__ f16x8 operator()(int rt, int g, int x) const { return p[((rt * 4 + g) * 2 + x) * 64]; }
};

// Spans 1 .. 64 of the back-rotation on a wave's half rows (value (t, k) of O is head_dim
// 128h + 32 (t / 2) + 8 j4 + 2k + (t & 1)), then the 1/16 of H = H_256/16.  The span-128 stage
// pairs the two halves and is taken by the caller.
template <int RT>
__device__ __forceinline__ void hadamard_half(f32x4 (&O)[RT][8], int lane) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int b = 0; b < 4; ++b)                              // bit 0: tile parity
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float e = O[rt][2 * b][k], o = O[rt][2 * b + 1][k];
        O[rt][2 * b][k] = e + o; O[rt][2 * b + 1][k] = e - o;
      }
#pragma unroll
    for (int kb = 1; kb <= 2; kb <<= 1)                      // bits 1, 2: k
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (!(k & kb)) {
            const float x = O[rt][t][k], y = O[rt][t][k | kb];
            O[rt][t][k] = x + y; O[rt][t][k | kb] = x - y;
          }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {                     // bits 3, 4: lane groups
      const bool upper = (lane & o) != 0;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float other = o == 16 ? partner16(O[rt][t][k], lane) : partner32(O[rt][t][k], lane);
          O[rt][t][k] = upper ? (other - O[rt][t][k]) : (O[rt][t][k] + other);
        }
    }
#pragma unroll
    for (int bb = 1; bb <= 2; bb <<= 1)                      // bits 5, 6: group index
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (!(b & bb))
#pragma unroll
          for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float x = O[rt][2 * b + par][k], y = O[rt][2 * (b | bb) + par][k];
              O[rt][2 * b + par][k] = x + y; O[rt][2 * (b | bb) + par][k] = x - y;
            }
#pragma unroll
    for (int t = 0; t < 8; ++t) O[rt][t] *= 0.0625f;
  }
}

// LDS layout (bytes).  Page loop: q fragments, their per-row factors, partial scores.  Merge (after
// the loop, from offset 0): every wave's half rows of every row tile, and the pairs' (m, l).
template <int RT>
struct VerifyLds {
  static constexpr int kQ = RT * 4 * 2 * 64 * 16;                       // q fragments
  static constexpr int kQm = 2 * RT * 64 * 4;                           // q factors [half][rt][lane]
  static constexpr int kX = kPairs * 2 * 2 * RT * 64 * 16;              // partial scores [pair][parity][half][rt][lane]
  static constexpr int kW = kPairs * 2 * 2 * 64 * 16;                   // weight records [pair][parity][half][lane]
  static constexpr int kA = kPairs * 2 * 2 * 64 * 4;                    // rescale factors [pair][parity][half][lane]
  static constexpr int kLoop = kQ + kQm + kX + kW + kA;
  static constexpr int kMergeO = RT * kPairs * 2 * 8 * 64 * 16;         // [rt][pair][half][tile][lane]
  static constexpr int kMergeML = RT * kPairs * 2 * 64 * 4;             // [rt][pair][m | l][lane]
  static constexpr int kMerge = kMergeO + kMergeML;
  static constexpr int kBytes = kLoop > kMerge ? kLoop : kMerge;
};

template <int RT, int PPP>
__global__ __launch_bounds__(kWaves * 64, 2) void k_verify_k8v4(const DecodeArgs a) {
  constexpr int NT = 8;                                   // PV tiles of a half row
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wv >> 1, h = wv & 1;
  const int i16 = lane & 15, j4 = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  if (split >= a.n_splits) return;

  int G, h0;
  if (a.g_uniform > 0) {
    G = a.g_uniform;
    h0 = kvh * G;
  } else {
    h0 = a.head_off[kvh];
    G = a.head_off[kvh + 1] - h0;
  }
  const int R = a.n_q * G;
  const int cap = a.max_pages * KVQ_PAGE_SIZE;
  const int RA = a.row_alloc;
  int Lrow[RT], qrow[RT];
  bool valid[RT];
  const int seq_len = clampi(a.seq_lens[b], 0, cap);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 16 * rt + i16;
    valid[rt] = r < R;
    const int t = valid[rt] ? r / G : 0;
    const int i = valid[rt] ? r % G : 0;
    const int hq = a.g_uniform > 0 ? h0 + i : a.head_list[h0 + i];
    qrow[rt] = (b * a.n_q + t) * a.n_q_heads + hq;
    Lrow[rt] = valid[rt] ? (a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + t], 0, cap) : seq_len) : 0;
  }
  const int* bt_row = a.bt + (size_t)b * a.max_pages;
  const int p_begin = split * a.pages_per_split;
  const int p0 = p_begin + pair;
  const int p_cap = min(p_begin + a.pages_per_split, a.max_pages) - 1;
  // page id of the pair's i-th page by lane reads (lane l holds the id of page l)
  const int my_ids = clampi(bt_row[min(p0 + min(lane, PPP - 1) * kPairs, p_cap)], 0, a.num_pages - 1);
  auto page_id = [&](int i) -> int { return __builtin_amdgcn_readlane(my_ids, i); };

  // Fused quantize-on-write: new token t goes to position seq_len - n_q + t (skipped before 0).  Both
  // waves of the pair whose page list holds that cell encode it (identical bytes) and store it, wait
  // for the stores, and load their halves of a prologue page that holds it again past the L1.
  int fz_idx[kDecodeMaxFused], fz_slot[kDecodeMaxFused];
  uint2 fz_x[kDecodeMaxFused][2];
  int fz_mask = 0;
#pragma unroll
  for (int t = 0; t < kDecodeMaxFused; ++t) {
    fz_idx[t] = -1;
    fz_slot[t] = 0;
    if (a.k_new && t < a.n_q && seq_len - a.n_q + t >= 0) {
      const int pos = seq_len - a.n_q + t;
      const int pl = pos / KVQ_PAGE_SIZE - p_begin;
      if (pl >= 0 && pl < a.pages_per_split && pl % kPairs == pair) {
        fz_idx[t] = pl / kPairs;
        fz_slot[t] = pos % KVQ_PAGE_SIZE;
        fz_mask |= 1 << fz_idx[t];
        const size_t off = ((size_t)(b * a.n_q + t) * a.hkv + kvh) * kD + 4 * lane;
        fz_x[t][0] = *reinterpret_cast<const uint2*>(a.k_new + off);
        fz_x[t][1] = *reinterpret_cast<const uint2*>(a.v_new + off);
      }
    }
  }
  // this wave's half of the query rows (pair 0 builds the fragments for all pairs)
  uint4 raw[RT][2][2];
  if (pair == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint16_t* qp = a.q + (size_t)qrow[rt] * kD + 16 * j4;
#pragma unroll
      for (int gl = 0; gl < 2; ++gl) {
        raw[rt][gl][0] = *reinterpret_cast<const uint4*>(qp + 64 * (2 * h + gl));
        raw[rt][gl][1] = *reinterpret_cast<const uint4*>(qp + 64 * (2 * h + gl) + 8);
      }
    }
  }
  __shared__ __align__(16) uint8_t smem[VerifyLds<RT>::kBytes];
  HalfPage buf[kPD + 1];
#pragma unroll
  for (int i = 0; i < kPD && i < PPP; ++i) load_half<false>(buf[i], a, page_id(i), kvh, h, lane);

  int Lmax = 0;
  for (int t = 0; t < a.n_q; ++t)
    Lmax = max(Lmax, a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + t], 0, cap) : seq_len);
  const int npages = (Lmax + KVQ_PAGE_SIZE - 1) / KVQ_PAGE_SIZE;
  const int p_end = min(p_begin + a.pages_per_split, npages);
  const size_t row0 = (size_t)(b * a.hkv + kvh) * RA;
  float* part_ml = a.part;
  float* part_o = a.part + (size_t)a.batch * a.hkv * RA * a.n_splits * 2;

  bool fz_small = false;                                    // a new V cell's d below 2^-10
  if (fz_mask) {
#pragma unroll
    for (int t = 0; t < kDecodeMaxFused; ++t) {
      if (fz_idx[t] < 0) continue;
      const size_t tile = (size_t)page_id(fz_idx[t]) * a.hkv + kvh;
      float y[4] = {bf16f(fz_x[t][1].x & 0xffffu), bf16f(fz_x[t][1].x >> 16), bf16f(fz_x[t][1].y & 0xffffu),
                    bf16f(fz_x[t][1].y >> 16)};
      const Q4x4 e = q4h_encode_x4(y, lane);
      uint8_t* vc = const_cast<uint8_t*>(a.v_codes) + tile * (KVQ_PAGE_SIZE * (kD / 2));
      vc[v_tile_offset(2 * lane, fz_slot[t])] = e.b0;
      vc[v_tile_offset(2 * lane + 1, fz_slot[t])] = e.b1;
      if ((lane & 7) == 0)
        const_cast<uint16_t*>(a.v_scales)[(tile * KVQ_PAGE_SIZE + fz_slot[t]) * (kD / 32) + (lane >> 3)] = e.d_bits;
      fz_small = fz_small || (uint16_t)((e.d_bits & 0x7fffu) - 1u) < 0x13ffu;
      const float x[4] = {bf16f(fz_x[t][0].x & 0xffffu), bf16f(fz_x[t][0].x >> 16), bf16f(fz_x[t][0].y & 0xffffu),
                          bf16f(fz_x[t][0].y >> 16)};
      const Int8x4 ek = int8_encode_x4(x);
      uint8_t* kc = const_cast<uint8_t*>(a.k_codes) + tile * (KVQ_PAGE_SIZE * kD);
      *reinterpret_cast<uint32_t*>(kc + k_tile_offset(4 * lane, fz_slot[t])) = ek.packed;
      if ((lane & 15) == 0)
        const_cast<uint16_t*>(a.k_scales)[(tile * KVQ_PAGE_SIZE + fz_slot[t]) * (kD / 64) + (lane >> 4)] = ek.scale_bits;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < kPD && i < PPP; ++i)
      if ((fz_mask >> i) & 1) load_half<true>(buf[i], a, page_id(i), kvh, h, lane);
  }

  if (R == 0) return;
  if (p_begin >= p_end) {                                   // nothing visible in this split
    if (a.n_splits == 1) {                                  // the only split writes the output: zeros
      for (int i = (int)threadIdx.x; i < R * (kD / 4); i += kWaves * 64)
        *reinterpret_cast<float4*>(a.out + (size_t)decode_out_row(a, b, kvh, i / (kD / 4), G, h0) * kD +
                                   4 * (i % (kD / 4))) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else if ((int)threadIdx.x < R) {
      float* ml = part_ml + ((row0 + threadIdx.x) * a.n_splits + split) * 2;
      ml[0] = kNegInf; ml[1] = 0.0f;
    }
    return;
  }

  // q fragments (fp16, pre-scaled per row and half by a power of two so the bf16 values convert
  // exactly) and the factor that undoes the scaling (applied to the wave's partial scores), written
  // to LDS by pair 0
  const QFrag<RT> qf{reinterpret_cast<const f16x8*>(smem) + lane};
  float* qmul_lds = reinterpret_cast<float*>(smem + VerifyLds<RT>::kQ);      // [half][rt][lane]
#pragma unroll
  for (int rt = 0; rt < RT && pair == 0; ++rt) {
    float mx = 0.0f;
#pragma unroll
    for (int gl = 0; gl < 2; ++gl)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (!valid[rt]) raw[rt][gl][x] = make_uint4(0, 0, 0, 0);
        const uint32_t w[4] = {raw[rt][gl][x].x, raw[rt][gl][x].y, raw[rt][gl][x].z, raw[rt][gl][x].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mx = fmaxf(mx, fmaxf(fabsf(bf16f(w[e] & 0xffffu)), fabsf(bf16f(w[e] >> 16))));
      }
    mx = max_over_row_lanes(mx);
    int ex = 0;
    if (mx > 0.0f) { frexpf(mx, &ex); ex = 15 - ex; }        // max * 2^ex in [2^14, 2^15)
#pragma unroll
    for (int gl = 0; gl < 2; ++gl)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint32_t w[4] = {raw[rt][gl][x].x, raw[rt][gl][x].y, raw[rt][gl][x].z, raw[rt][gl][x].w};
        f16x8 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = (_Float16)ldexpf(bf16f(w[e] & 0xffffu), ex);
          f[2 * e + 1] = (_Float16)ldexpf(bf16f(w[e] >> 16), ex);
        }
        const_cast<f16x8*>(qf.p)[((rt * 4 + 2 * h + gl) * 2 + x) * 64] = f;
      }
    qmul_lds[(h * RT + rt) * 64 + lane] = ldexpf(a.scale_log2, -ex);
  }

  float m_run[RT], l_run[RT];
  f32x4 O[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) O[rt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  f32x4* xbuf = reinterpret_cast<f32x4*>(smem + VerifyLds<RT>::kQ + VerifyLds<RT>::kQm);   // [pair][parity][half][rt][lane]
  auto xslot = [&](int par, int hh, int rt) { return xbuf + (((pair * 2 + par) * 2 + hh) * RT + rt) * 64 + lane; };
  uint4* wbuf = reinterpret_cast<uint4*>(smem + VerifyLds<RT>::kQ + VerifyLds<RT>::kQm + VerifyLds<RT>::kX);
  float* abuf = reinterpret_cast<float*>(smem + VerifyLds<RT>::kQ + VerifyLds<RT>::kQm + VerifyLds<RT>::kX + VerifyLds<RT>::kW);
  auto wslot = [&](int par, int hh) { return wbuf + ((pair * 2 + par) * 2 + hh) * 64 + lane; };
  auto aslot = [&](int par, int hh) { return abuf + ((pair * 2 + par) * 2 + hh) * 64 + lane; };
  // With two row tiles the waves of a pair split the softmax: wave h runs it for row tile h (m_own,
  // l_own) and hands its weights to the partner through LDS.
  constexpr bool SPLIT = RT == 2;
  float m_own = kNegInf, l_own = 0.0f;
  const int L_own = SPLIT && h ? Lrow[RT - 1] : Lrow[0];

  // The pair's pages: n_mine of them.  The two waves of a pair meet once per page through LDS flags
  // (flags[w] = page steps wave w has published), not a workgroup barrier, so the pairs run apart
  // and the two waves sharing a SIMD (from different pairs) overlap each other's phases.
  const int n_mine = p0 < p_end ? (p_end - 1 - p0) / kPairs + 1 : 0;
  const int last = max(n_mine, 1) - 1;
  __shared__ uint32_t flags[kWaves];
  if (lane == 0) flags[wv] = 0;
  __syncthreads();                                          // q fragments, factors and flags written
  float qmul[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) qmul[rt] = qmul_lds[(h * RT + rt) * 64 + lane];

  // fp16 V parts need every V scale of the wave's pages to be 0 or at least 2^-10 (see the PV step)
  bool v16;
  {
    const int pl = min(lane >> 2, max(n_mine, 1) - 1);
    const int pid = __shfl(my_ids, pl);
    const uint8_t* vsp = reinterpret_cast<const uint8_t*>(a.v_scales + ((size_t)pid * a.hkv + kvh) * 16 * 8);
    u16x2 mn = {0xffff, 0xffff};
#pragma unroll
    for (int k = 0; k < 4; ++k) {                           // tokens 4 (lane % 4) + k, this half's 4 groups
      const uint2 q = ld8(vsp + 16 * (4 * (lane & 3) + k) + 8 * h);
      mn = __builtin_elementwise_min(mn, __builtin_bit_cast(u16x2, q.x & 0x7fff7fffu) - u16x2{1, 1});
      mn = __builtin_elementwise_min(mn, __builtin_bit_cast(u16x2, q.y & 0x7fff7fffu) - u16x2{1, 1});
    }
    // (the scan may read a fused cell's slot as it was before this wave's store; the encoder's own d
    // covers it)
    // one choice for the workgroup, so every wave runs the same page loop (with its barriers)
    v16 = __syncthreads_and(!__any(mn[0] < 0x13ffu || mn[1] < 0x13ffu || fz_small)) != 0;
  }

  auto run = [&](auto v16_tag) {
    constexpr bool V16 = decltype(v16_tag)::value;
#pragma unroll
    for (int i = 0; i < PPP; ++i) {
      if (i >= n_mine) break;
      // (a prefetch past the pair's last page re-reads that page, an L2 hit: no branch guards a load,
      // so every wait on the vector memory counter covers exactly the page about to be used)
      if (i + kPD < PPP) load_half<false>(buf[(i + kPD) % (kPD + 1)], a, page_id(min(i + kPD, last)), kvh, h, lane);
      const HalfPage& pb = buf[i % (kPD + 1)];
      const int tok0 = (p0 + i * kPairs) * KVQ_PAGE_SIZE + 4 * j4;
      const int par = i & 1;
      // ---- QK over this wave's half: partial scores, scaled
      f32x4 sp[RT];
      {
        f32x4 acc[RT][2];
#pragma unroll
        for (int gl = 0; gl < 2; ++gl) {
          const f16x8 a0 = codes_to_f16(pb.k[gl].x, pb.k[gl].y);
          const f16x8 a1 = codes_to_f16(pb.k[gl].z, pb.k[gl].w);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            acc[rt][gl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qf(rt, 2 * h + gl, 0), f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                                 0, 0, 0);
            acc[rt][gl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qf(rt, 2 * h + gl, 1), acc[rt][gl], 0, 0, 0);
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            sp[rt][k] = fmaf(acc[rt][1][k], pb.kscale(k, 1), acc[rt][0][k] * pb.kscale(k, 0)) * qmul[rt];
      }
      // Exchange with the partner wave through LDS slots of page parity par, each step published by a
      // flag (flags[w] counts the steps wave w has published; a wave publishes two steps per page when
      // it splits the softmax, one otherwise).  A slot is rewritten two pages later, after the partner
      // has published a later step, which it does only after reading the slot.  The partner is in this
      // workgroup and always gets there; each wait is bounded all the same.
      const uint32_t steps = SPLIT ? 2u : 1u;
      auto publish = [&](uint32_t n) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_store(&flags[wv], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      };
      auto await = [&](uint32_t n) {
        for (uint32_t spin = 0; spin < kSpinLimit; ++spin) {
          if (__hip_atomic_load(&flags[wv ^ 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= n) break;
          __builtin_amdgcn_s_sleep(0);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      };
      // (values are exchanged as whole slots, and each wave reads its own back as well: a wave-uniform
      // LDS address picks the row tile, where a choice in registers would cost a select per value)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) *xslot(par, h, rt) = sp[rt];
      publish(steps * i + 1);
      await(steps * i + 1);
      // ---- scores (half 0's partial plus half 1's), online softmax with lazy rescaling (the reference
      // max moves only when a score exceeds it by more than 2^kLazyLog2), the weights of each row tile
      // as a record {hi parts of tokens 4 j4 .. + 3, lo parts}: fp16 parts of 16 x the weight (V16)
      // or bf16 parts of the weight
      auto softmax = [&](const f32x4& s0, const f32x4& s1, int L, float& m_run_r, float& l_run_r,
                         float& alpha) -> uint4 {
        float s[4], pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) s[k] = (tok0 + k < L) ? s0[k] + s1[k] : kNegInf;
        const float mx = max_over_row_lanes(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        const bool move = mx > m_run_r + kLazyLog2;
        const float m_new = move ? mx : m_run_r;
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        const bool rescale = move && m_run_r != kNegInf;
        alpha = rescale ? __builtin_amdgcn_exp2f(m_run_r - m_use) : 1.0f;
        m_run_r = m_new;
#pragma unroll
        for (int k = 0; k < 4; ++k) pk[k] = __builtin_amdgcn_exp2f(s[k] - m_use);
        l_run_r = l_run_r * alpha + ((pk[0] + pk[1]) + (pk[2] + pk[3]));
        if constexpr (V16) {
          f16x4 wh, wl;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float x = 16.0f * pk[k];
            wh[k] = (_Float16)x;
            wl[k] = (_Float16)(x - (float)wh[k]);
          }
          const uint2 hh2 = __builtin_bit_cast(uint2, wh), ll2 = __builtin_bit_cast(uint2, wl);
          return make_uint4(hh2.x, hh2.y, ll2.x, ll2.y);
        } else {
          s16x4 ph, pl;
          split_bf16(pk, ph, pl);
          const uint2 hh2 = __builtin_bit_cast(uint2, ph), ll2 = __builtin_bit_cast(uint2, pl);
          return make_uint4(hh2.x, hh2.y, ll2.x, ll2.y);
        }
      };
      uint4 wrec[RT];
      float alpha[RT];
      if constexpr (SPLIT) {
        float a_own;
        *wslot(par, h) = softmax(*xslot(par, 0, h), *xslot(par, 1, h), L_own, m_own, l_own, a_own);
        *aslot(par, h) = a_own;
        publish(steps * i + 2);
        await(steps * i + 2);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          wrec[rt] = *wslot(par, rt);
          alpha[rt] = *aslot(par, rt);
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          wrec[rt] = softmax(*xslot(par, 0, rt), *xslot(par, 1, rt), Lrow[rt], m_run[rt], l_run[rt], alpha[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        if (__any(alpha[rt] != 1.0f)) {
#pragma unroll
          for (int t = 0; t < NT; ++t) O[rt][t] *= alpha[rt];
        }
      // ---- PV over this wave's four V groups: V enters the MFMA as the exact product (code - 8) * d in
      // two parts, built once per page for both row tiles, and the weights in two parts (the record).
      // One K = 32 MFMA takes the lane's 4 tokens twice: A = [V hi | V lo] against B = [w hi ; w hi],
      // then against [w lo ; w lo] (the full product of the two-part values; a K = 16 MFMA costs as
      // much as a K = 32 one here).  fp16 parts (V16): the product / 16 in fp16 (hi = the rounded
      // product, lo = its exact rounding error from one fma; the 1/16 keeps it below 2^15) against
      // fp16 parts of 16 x the weights; otherwise bf16 parts of the product (a 4-bit code times an
      // fp16 scale has at most 15 significant bits) against bf16 parts of the weights.
      if constexpr (V16) {
        f16x8 wh[RT], wl[RT];                               // each part twice: tokens 4 j4 .. + 3, again
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          wh[rt] = __builtin_bit_cast(f16x8, make_uint4(wrec[rt].x, wrec[rt].y, wrec[rt].x, wrec[rt].y));
          wl[rt] = __builtin_bit_cast(f16x8, make_uint4(wrec[rt].z, wrec[rt].w, wrec[rt].z, wrec[rt].w));
        }
        const f16x2 mul = {(_Float16)0.0625f, (_Float16)0.0625f}, add = {(_Float16)-64.5f, (_Float16)-64.5f};
#pragma unroll
        for (int gl = 0; gl < 4; ++gl) {
          // byte k of the word: token 4 j4 + k; its low / high nibble: head_dim 128h + 32gl + 2 i16 (+1)
          const uint32_t w = word_of(pb.v, gl);
          const uint32_t hsel = (gl & 1) ? 0x07060302u : 0x05040100u;
          const f16x2 d01 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(pb.vs[2 + (gl >> 1)], pb.vs[gl >> 1], hsel));
          const f16x2 d23 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(pb.vs[6 + (gl >> 1)], pb.vs[4 + (gl >> 1)], hsel));
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t nib = (w >> (4 * e)) & 0x0f0f0f0fu;
            // [code, 0x64] per token pair reads 1024 + code; one packed fma gives (code - 8) / 16 exactly
            const f16x2 c01 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, nib, 0x04010400u)) * mul + add;
            const f16x2 c23 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, nib, 0x04030402u)) * mul + add;
            const f16x2 h01 = c01 * d01, h23 = c23 * d23;
            const f16x2 l01 = __builtin_elementwise_fma(c01, d01, -h01), l23 = __builtin_elementwise_fma(c23, d23, -h23);
            const f16x8 av = __builtin_bit_cast(
                f16x8, make_uint4(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23),
                                  __builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              O[rt][2 * gl + e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, wh[rt], O[rt][2 * gl + e], 0, 0, 0);
              O[rt][2 * gl + e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, wl[rt], O[rt][2 * gl + e], 0, 0, 0);
            }
          }
        }
      } else {
        bf16x8 bqh[RT], bql[RT];                            // each part twice, as above
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          bqh[rt] = __builtin_bit_cast(bf16x8, make_uint4(wrec[rt].x, wrec[rt].y, wrec[rt].x, wrec[rt].y));
          bql[rt] = __builtin_bit_cast(bf16x8, make_uint4(wrec[rt].z, wrec[rt].w, wrec[rt].z, wrec[rt].w));
        }
#pragma unroll
        for (int gl = 0; gl < 4; ++gl) {
          const uint32_t w = word_of(pb.v, gl);
          float sc[4], off[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            sc[k] = pb.vscale(k, gl);
            off[k] = -8.0f * sc[k];
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t nib = (w >> (4 * e)) & 0x0f0f0f0fu;
            uint32_t hb[4], lb[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float x = fmaf((float)((nib >> (8 * k)) & 0xffu), sc[k], off[k]);   // exact
              hb[k] = __float_as_uint(x) & 0xffff0000u;
              lb[k] = __float_as_uint(x - __uint_as_float(hb[k]));                    // exact, low half 0
            }
            const bf16x8 av = __builtin_bit_cast(
                bf16x8, make_uint4(__builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u),
                                   __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u),
                                   __builtin_amdgcn_perm(lb[1], lb[0], 0x07060302u),
                                   __builtin_amdgcn_perm(lb[3], lb[2], 0x07060302u)));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              O[rt][2 * gl + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bqh[rt], O[rt][2 * gl + e], 0, 0, 0);
              O[rt][2 * gl + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bql[rt], O[rt][2 * gl + e], 0, 0, 0);
            }
          }
        }
      }
    }
  };
  if (v16) run(std::true_type{});
  else run(std::false_type{});

  // ---- per-wave row sums over the 4 lane groups
  if constexpr (SPLIT) {
    l_own = sum_over_row_lanes(l_own);
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l_run[rt] = sum_over_row_lanes(l_run[rt]);
  }

  // ---- merge the 4 pairs: every wave stores its half rows of every row tile (and the pair's m, l of
  // row tile rt: the wave that ran its softmax, else the half-0 wave); then the two waves of pair rt
  // merge row tile rt over the pairs
  f32x4* lds_o = reinterpret_cast<f32x4*>(smem);                                  // [rt][pair][half][tile][lane]
  float* lds_ml = reinterpret_cast<float*>(smem + VerifyLds<RT>::kMergeO);       // [rt][pair][m | l][lane]
  __syncthreads();                                          // the page loop's use of this LDS is over
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int t = 0; t < NT; ++t) lds_o[(((rt * kPairs + pair) * 2 + h) * NT + t) * 64 + lane] = O[rt][t];
    if (SPLIT ? rt == h : h == 0) {
      lds_ml[((rt * kPairs + pair) * 2 + 0) * 64 + lane] = SPLIT ? m_own : m_run[rt];
      lds_ml[((rt * kPairs + pair) * 2 + 1) * 64 + lane] = SPLIT ? l_own : l_run[rt];
    }
  }
  __syncthreads();
  const int mrt = pair < RT ? pair : 0;                     // the row tile this wave merges (pairs 0 .. RT - 1)
  f32x4 M[1][NT];
  float m_fin = kNegInf, l_fin = 0.0f;
  if (pair < RT) {
    float mv[kPairs], cv[kPairs];
#pragma unroll
    for (int v = 0; v < kPairs; ++v) {
      mv[v] = lds_ml[((mrt * kPairs + v) * 2 + 0) * 64 + lane];
      m_fin = fmaxf(m_fin, mv[v]);
    }
    const float Mu = m_fin == kNegInf ? 0.0f : m_fin;
#pragma unroll
    for (int v = 0; v < kPairs; ++v) {
      cv[v] = __builtin_amdgcn_exp2f(mv[v] - Mu);
      l_fin += cv[v] * lds_ml[((mrt * kPairs + v) * 2 + 1) * 64 + lane];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 acc = lds_o[(((mrt * kPairs + 0) * 2 + h) * NT + t) * 64 + lane] * cv[0];
#pragma unroll
      for (int v = 1; v < kPairs; ++v) acc += cv[v] * lds_o[(((mrt * kPairs + v) * 2 + h) * NT + t) * 64 + lane];
      M[0][t] = acc;
    }
  }
  // ---- back-rotation of the merged partial: span 128 between the two halves through LDS
  __syncthreads();
  if (pair < RT) {
#pragma unroll
    for (int t = 0; t < NT; ++t) lds_o[((mrt * 2 + h) * NT + t) * 64 + lane] = M[0][t];
  }
  __syncthreads();
  if (pair >= RT) return;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const f32x4 other = lds_o[((mrt * 2 + (1 - h)) * NT + t) * 64 + lane];
    M[0][t] = h == 0 ? M[0][t] + other : other - M[0][t];
  }
  hadamard_half<1>(M, lane);

  // ---- the partial of rows r < R (this wave's half of row tile mrt); with a single split the
  // normalised output
  const bool direct = a.n_splits == 1;
  const int r = 16 * mrt + i16;
  if (r >= R) return;
  const int qr = RT > 1 && mrt == 1 ? qrow[RT - 1] : qrow[0];
  float* row = direct ? a.out + (size_t)qr * kD : part_o + ((row0 + r) * a.n_splits + split) * kD;
  const float sc = direct ? (l_fin > 0.0f ? 1.0f / l_fin : 0.0f) : 1.0f;
  auto put4 = [&](float* p, float x0, float x1, float x2, float x3) {
    *reinterpret_cast<float4*>(p) = make_float4(x0 * sc, x1 * sc, x2 * sc, x3 * sc);
  };
  if (!direct && j4 == 0 && h == 0) {
    float* ml = part_ml + ((row0 + r) * a.n_splits + split) * 2;
    ml[0] = m_fin; ml[1] = l_fin;
  }
#pragma unroll
  for (int gl = 0; gl < 4; ++gl) {   // tiles 2gl (even d) / 2gl+1 (odd d): d = 128h + 32gl + 8 j4 + 2k (+1)
    const f32x4 e = M[0][2 * gl], o = M[0][2 * gl + 1];
    put4(row + 128 * h + 32 * gl + 8 * j4, e[0], o[0], e[1], o[1]);
    put4(row + 128 * h + 32 * gl + 8 * j4 + 4, e[2], o[2], e[3], o[3]);
  }
}

}  // namespace

// Pages per pair of a split: 16 with 64-page splits, 8 with 32-page splits.
hipError_t launch_decode_verify(int row_tiles, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)plan.n_splits, a.hkv, a.batch), block(kWaves * 64);
  // pages per wave pair: the kernel's loop takes up to PPP (8 or 16) and exits after the pair's last
  const int ppp = plan.pages_per_split / kPairs;
  if (ppp * kPairs != plan.pages_per_split || ppp < 1 || ppp > 16) return hipErrorInvalidValue;
  if (row_tiles == 2) {
    if (ppp > 8) k_verify_k8v4<2, 16><<<grid, block, 0, s>>>(a);
    else k_verify_k8v4<2, 8><<<grid, block, 0, s>>>(a);
  } else if (row_tiles == 1) {
    if (ppp > 8) k_verify_k8v4<1, 16><<<grid, block, 0, s>>>(a);
    else k_verify_k8v4<1, 8><<<grid, block, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return plan.n_splits > 1 ? launch_decode_combine(kD, plan, a, s) : hipSuccess;
}

}  // namespace kvq
