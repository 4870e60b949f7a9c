// Split-K decode attention over caches with an unquantised FP32 store.
//
// strata PR #2698, intro and "What it does": the engine's K/V caches are FP32 by default; the modes
// k8v32 / k32v8 quantise one store only (int8 codes + one FP16 scale per 64 values) and keep the
// other in FP32; decode and verify windows read the stores as they are, dequantising the int8 one on
// the fly.  Here K and V are each INT8_G64 or F32, at least one of them F32.
//
// Work decomposition (as the other decode kernels): one workgroup = one (sequence, KV head, split of
// NW * PPW pages); wave w takes pages w, w + NW, ... of the split.  Up to 32 query rows per KV head,
// in RT row tiles of 16 (one MFMA column per row).
//   * QK: S^T[token][row].  F32 K on v_mfma_f32_16x16x32_bf16: lane (j = lane / 16, t = lane % 16)
//     holds, for the 32 head_dim values of step s, the 16-byte chunks 8s + j and 8s + 4 + j of slot t
//     (each wave load is one contiguous kilobyte of the tile), split into a bf16 hi part (truncated)
//     and a bf16 lo part (the remainder, rounded); the query is bf16 and enters exactly.  INT8 K on
//     v_mfma_f32_16x16x32_f16 as the int8 kernel: exact fp16 codes against the query times a power of
//     two per row in fp16 (exact: bf16 has 8 significant bits), one accumulator per 64-group weighted
//     by its (token, group) scale.
//   * Online softmax in base 2 against a lazily moved reference max (weights stay below 2^8).
//   * PV: O^T[d][row] on v_mfma_f32_16x16x16bf16_1k with the weights of the lane's 4 tokens as the B
//     operand.  F32 V: the A operand is 4 tokens' values of one head_dim index (one 16-byte load from
//     the head_dim-major tile) split into bf16 hi + lo, and three MFMAs take hi x hi, lo x hi and
//     hi x lo (lo x lo is below 2^-16 of the term).  INT8 V: codes + 128 exact in bf16 against
//     weight x scale in bf16 hi + lo, the bias taken off at the end through the per-group weight sums.
//   * The waves merge through LDS one row tile at a time; the partial goes to the log-sum-exp combine
//     shared with the other decode kernels, or, with one split, the workgroup writes the normalised
//     output itself.
#include <stdlib.h>

#include "kvq_internal.h"
#include "device_util.h"
#include "decode_parts.h"
#include "int8_cell.h"

namespace kvq {
namespace {

constexpr float kLazyF = 8.0f;                  // weights stay below 2^8 between rescalings

// Launch shapes: waves per workgroup, pages per wave per split, pages each wave keeps in flight.
struct FShape { int nw, ppw, pd; };
constexpr FShape kFShapes[] = {{4, 16, 1}, {4, 8, 1}};
constexpr int kNumFShapes = (int)(sizeof(kFShapes) / sizeof(kFShapes[0]));

// KVQ_F32_DECODE_SHAPE overrides the choice (for tuning); -1 when unset
int f32_shape_override() {
  static int idx = -2;
  if (idx == -2) {
    idx = -1;
    if (const char* e = getenv("KVQ_F32_DECODE_SHAPE")) {
      const int v = atoi(e);
      if (v >= 0 && v < kNumFShapes) idx = v;
    }
  }
  return idx;
}

// One page of one KV head as a lane holds it.
template <int D, bool KF, bool VF>
struct FPage {
  static constexpr int NG = D / 64;              // 64-value scale groups
  static constexpr int NK = KF ? D / 16 : NG;    // 16-byte K units of the lane
  static constexpr int NV = VF ? D / 16 : NG;    // 16-byte V units of the lane
  uint4 k[NK];        // F32: unit u = chunk 4u + j of slot t; INT8: chunk 4g + j of slot t
  uint4 v[NV];        // F32: tokens 4j .. 4j+3 of head_dim 16u + t; INT8: as the int8 kernel
  uint32_t ks[KF ? 1 : 2 * NG];   // INT8 K: fp16 scales of tokens 4j .. 4j+3, half k * NG + g
  uint32_t vs[VF ? 1 : 2 * NG];
  static __device__ __forceinline__ float half_at(const uint32_t* w, int i) {
    const uint32_t x = w[i >> 1];
    return h2f((uint16_t)((i & 1) ? (x >> 16) : (x & 0xffffu)));
  }
  __device__ __forceinline__ float kscale(int k, int g) const { return half_at(ks, k * NG + g); }
  __device__ __forceinline__ float vscale(int k, int g) const { return half_at(vs, k * NG + g); }
};

template <int N>
__device__ __forceinline__ void load_scale_words(uint32_t (&dst)[N], const uint16_t* src) {
  static_assert(N % 4 == 0, "scale words come in 16-byte units");
#pragma unroll
  for (int c = 0; c < N / 4; ++c) {
    const uint4 t = stream_load(src + 8 * c);
    dst[4 * c] = t.x; dst[4 * c + 1] = t.y; dst[4 * c + 2] = t.z; dst[4 * c + 3] = t.w;
  }
}

template <int D, bool KF, bool VF>
__device__ __forceinline__ void load_fpage(FPage<D, KF, VF>& pb, const DecodeArgs& a, int page, int kvh, int lane) {
  using P = FPage<D, KF, VF>;
  const int i16 = lane & 15, j4 = lane >> 4;
  const size_t tile = (size_t)page * a.hkv + kvh;
  const uint4* kb = reinterpret_cast<const uint4*>(a.k_codes + tile * (16 * (KF ? 4 * D : D))) + lane;
#pragma unroll
  for (int u = 0; u < P::NK; ++u) pb.k[u] = stream_load(kb + 64 * u);
  if constexpr (!KF) load_scale_words(pb.ks, a.k_scales + (tile * 16 + 4 * j4) * P::NG);
  const uint4* vb = reinterpret_cast<const uint4*>(a.v_codes + tile * (16 * (VF ? 4 * D : D))) + 4 * i16 + j4;
#pragma unroll
  for (int u = 0; u < P::NV; ++u) pb.v[u] = stream_load(vb + 64 * u);
  if constexpr (!VF) load_scale_words(pb.vs, a.v_scales + (tile * 16 + 4 * j4) * P::NG);
}

// Device-scope 16-byte load at a byte offset from a wave-uniform base: it misses the CU's L1 and reads
// L2, so a page this wave loaded, then wrote a cell into (and waited for), comes back with it.
__device__ __forceinline__ uint4 load_dev(const void* base, uint32_t off) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0x10 /* sc1: device scope */);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int D, bool KF, bool VF>
__device__ __forceinline__ void load_fpage_dev(FPage<D, KF, VF>& pb, const DecodeArgs& a, int page, int kvh,
                                               int lane) {
  using P = FPage<D, KF, VF>;
  const int i16 = lane & 15, j4 = lane >> 4;
  const size_t tile = (size_t)page * a.hkv + kvh;
  const uint8_t* kb = a.k_codes + tile * (16 * (KF ? 4 * D : D));
#pragma unroll
  for (int u = 0; u < P::NK; ++u) pb.k[u] = load_dev(kb, 16 * (64 * u + lane));
  const uint8_t* vb = a.v_codes + tile * (16 * (VF ? 4 * D : D));
#pragma unroll
  for (int u = 0; u < P::NV; ++u) pb.v[u] = load_dev(vb, 16 * (64 * u + 4 * i16 + j4));
  // scales of tokens 4 j4 .. 4 j4 + 3 (NG halves each) from the tile's first scale
  if constexpr (!KF) {
    const uint16_t* ks = a.k_scales + tile * 16 * P::NG;
#pragma unroll
    for (int c = 0; c < P::NG / 2; ++c) {
      const uint4 x = load_dev(ks, 8 * j4 * P::NG + 16 * c);
      pb.ks[4 * c] = x.x; pb.ks[4 * c + 1] = x.y; pb.ks[4 * c + 2] = x.z; pb.ks[4 * c + 3] = x.w;
    }
  }
  if constexpr (!VF) {
    const uint16_t* vs = a.v_scales + tile * 16 * P::NG;
#pragma unroll
    for (int c = 0; c < P::NG / 2; ++c) {
      const uint4 x = load_dev(vs, 8 * j4 * P::NG + 16 * c);
      pb.vs[4 * c] = x.x; pb.vs[4 * c + 1] = x.y; pb.vs[4 * c + 2] = x.z; pb.vs[4 * c + 3] = x.w;
    }
  }
}

// 8 binary32 values (two 16-byte chunks) -> bf16 hi (truncated) and bf16 lo (the exact remainder,
// rounded): hi + lo keeps 16 significant bits.
__device__ __forceinline__ void split8(const uint4& p, const uint4& q, bf16x8& hi, bf16x8& lo) {
  const uint32_t x[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
  u32x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t u = x[2 * e], w = x[2 * e + 1];
    h[e] = __builtin_amdgcn_perm(w, u, 0x07060302u);
    const float ru = __uint_as_float(u) - __uint_as_float(u & 0xffff0000u);
    const float rw = __uint_as_float(w) - __uint_as_float(w & 0xffff0000u);
    l[e] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)ru) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)rw) << 16);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// One page of one wave for all row tiles: QK on MFMA, online softmax, PV on MFMA.  qb: the lane's
// query fragments in LDS, [row tile][D / 32][lane].
template <int D, int RT, bool KF, bool VF>
__device__ __forceinline__ void fpage_step(const FPage<D, KF, VF>& pb, int p, int j4, const int (&Lrow)[RT],
                                           const uint4* qb, const float (&qmul)[RT], float (&m_run)[RT],
                                           float (&l_run)[RT], float (&ls)[RT][D / 64], f32x4 (&O)[RT][D / 16]) {
  constexpr int NG = D / 64, NT = D / 16, NS = D / 32;
  // ---- QK: S^T[token 4*j4 + k][row]
  float sc[RT][4];
  if constexpr (KF) {
    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 ah, al;
      split8(pb.k[2 * s], pb.k[2 * s + 1], ah, al);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const bf16x8 bq = __builtin_bit_cast(bf16x8, qb[(rt * NS + s) * 64]);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bq, acc[rt], 0, 0, 0);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bq, acc[rt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < 4; ++k) sc[rt][k] = acc[rt][k];
  } else {
    f32x4 acc[RT][NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const f16x8 a0 = codes_to_f16(pb.k[g].x, pb.k[g].y);
      const f16x8 a1 = codes_to_f16(pb.k[g].z, pb.k[g].w);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const f16x8 b0 = __builtin_bit_cast(f16x8, qb[(rt * NS + 2 * g) * 64]);
        const f16x8 b1 = __builtin_bit_cast(f16x8, qb[(rt * NS + 2 * g + 1) * 64]);
        acc[rt][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        acc[rt][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, acc[rt][g], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float v = acc[rt][0][k] * pb.kscale(k, 0);
#pragma unroll
        for (int g = 1; g < NG; ++g) v = fmaf(acc[rt][g][k], pb.kscale(k, g), v);
        sc[rt][k] = v;
      }
  }

  // ---- online softmax per row tile (the reference max moves only by more than 2^kLazyF)
  const int tok0 = p * KVQ_PAGE_SIZE + 4 * j4;
  float pk[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float s[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) s[k] = (tok0 + k < Lrow[rt]) ? sc[rt][k] * qmul[rt] : kNegInf;
    const float mx = max_over_row_lanes(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    const bool move = mx > m_run[rt] + kLazyF;
    const float m_new = move ? mx : m_run[rt];
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const bool rescale = move && m_run[rt] != kNegInf;
    const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run[rt] - m_use) : 1.0f;
    m_run[rt] = m_new;
#pragma unroll
    for (int k = 0; k < 4; ++k) pk[rt][k] = __builtin_amdgcn_exp2f(s[k] - m_use);
    l_run[rt] = l_run[rt] * alpha + ((pk[rt][0] + pk[rt][1]) + (pk[rt][2] + pk[rt][3]));
    if (__any(rescale)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) O[rt][t] *= alpha;
      if constexpr (!VF) {
#pragma unroll
        for (int g = 0; g < NG; ++g) ls[rt][g] *= alpha;
      }
    }
  }

  // ---- PV: masked tokens have weight 0, and the values of cells past a sequence's length are finite
  // by contract, so they add exact zeros
  if constexpr (VF) {
    s16x4 bh[RT], bl[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) split_bf16(pk[rt], bh[rt], bl[rt]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float x[4] = {__uint_as_float(pb.v[t].x), __uint_as_float(pb.v[t].y), __uint_as_float(pb.v[t].z),
                          __uint_as_float(pb.v[t].w)};
      s16x4 ah, al;
      split_bf16(x, ah, al);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        O[rt][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh[rt], O[rt][t], 0, 0, 0);
        O[rt][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh[rt], O[rt][t], 0, 0, 0);
        O[rt][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl[rt], O[rt][t], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      s16x4 bh[RT], bl[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float pw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pw[k] = pk[rt][k] * pb.vscale(k, g);
        ls[rt][g] += (pw[0] + pw[1]) + (pw[2] + pw[3]);
        split_bf16(pw, bh[rt], bl[rt]);
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {              // tiles 4g .. 4g+3 (head_dim 64g .. 64g+63)
        const s16x4 av = codes_to_bf16_biased(word_of(pb.v[g], tt));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          O[rt][4 * g + tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bh[rt], O[rt][4 * g + tt], 0, 0, 0);
          O[rt][4 * g + tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bl[rt], O[rt][4 * g + tt], 0, 0, 0);
        }
      }
    }
  }
}

template <int D, int RT, bool KF, bool VF, int NW, int PPW, int PD>
__global__ __launch_bounds__(NW * 64, 1) void k_decode_f32(const DecodeArgs a) {
  constexpr int NG = D / 64, NT = D / 16, NS = D / 32;
  // one LDS allocation, the per-page operands first (their addresses then fit the 16-bit offset of
  // the LDS loads)
  constexpr int kQBytes = RT * NS * 64 * 16, kMulBytes = RT * 16 * 4;
  __shared__ __align__(16) uint8_t lds[kQBytes + kMulBytes + ((NW - 1) * NT * 64 * 4 + NW * RT * 2 * 64) * 4];
  uint4* const qlds = reinterpret_cast<uint4*>(lds);             // QK B operands: [row tile][step][lane]
  float* const qmul_lds = reinterpret_cast<float*>(lds + kQBytes);
  float* const mrg = reinterpret_cast<float*>(lds + kQBytes + kMulBytes);
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, j4 = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;

  // ---- rows of this KV head: row r is (query token r / G, query head r % G of the head's list);
  // row tile rt holds rows 16 rt .. 16 rt + 15, row 16 rt + n16 in the lane's column
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
  const int seq_len = clampi(a.seq_lens[b], 0, cap);
  int Lrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 16 * rt + n16;
    const int tq = r < R ? r / G : 0;
    Lrow[rt] = r < R ? (a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + tq], 0, cap) : seq_len) : 0;
  }

  // ---- this wave's first PD pages
  const int* bt_row = a.bt + (size_t)b * a.max_pages;
  const int p_begin = split * a.pages_per_split;
  const int p0 = p_begin + wv;
  const int p_cap = min(p_begin + a.pages_per_split, a.max_pages) - 1;
  FPage<D, KF, VF> buf[PD + 1];
#pragma unroll
  for (int i = 0; i < PD && i < PPW; ++i)
    load_fpage(buf[i], a, clampi(bt_row[min(p0 + i * NW, p_cap)], 0, a.num_pages - 1), kvh, lane);

  // Fused quantize-on-write (kvq_decode_attn_append): new token t goes to position seq_len - n_q + t.
  // The wave whose page list holds that cell encodes it (int8 store) or writes its values (FP32
  // store) before its page loop and waits for the stores; a page the prologue already loaded is
  // loaded again with device-scope loads, past the CU's L1.
  if (a.k_new) {
    int fz_mask = 0;
    for (int t = 0; t < a.n_q && t < kDecodeMaxFused; ++t) {
      const int pos = seq_len - a.n_q + t;                  // <= seq_len - 1 <= cap - 1
      if (pos < 0) continue;                                // no cell before position 0: skipped
      const int pl = pos / KVQ_PAGE_SIZE - p_begin;
      if (pl < 0 || pl >= a.pages_per_split || pl % NW != wv) continue;
      const int i = pl / NW, slot = pos % KVQ_PAGE_SIZE;
      const size_t tile = (size_t)clampi(bt_row[min(p0 + i * NW, p_cap)], 0, a.num_pages - 1) * a.hkv + kvh;
      const size_t off = ((size_t)(b * a.n_q + t) * a.hkv + kvh) * D + 4 * min(lane, D / 4 - 1);
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        const uint2 raw = *reinterpret_cast<const uint2*>((kv ? a.v_new : a.k_new) + off);
        const float x[4] = {bf16f(raw.x & 0xffffu), bf16f(raw.x >> 16), bf16f(raw.y & 0xffffu), bf16f(raw.y >> 16)};
        if (kv ? VF : KF) {                                 // FP32 store: the bf16 values widened
          uint8_t* codes = const_cast<uint8_t*>(kv ? a.v_codes : a.k_codes) + tile * (KVQ_PAGE_SIZE * 4 * D);
          if (lane < D / 4) {
            if (kv == 0) {
              *reinterpret_cast<float4*>(codes + k_tile_offset(16 * lane, slot)) = make_float4(x[0], x[1], x[2], x[3]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) *reinterpret_cast<float*>(codes + vf32_tile_offset(4 * (4 * lane + e), slot)) = x[e];
            }
          }
        } else {                                            // int8 store: the append kernel's encoder
          const Int8x4 en = int8_encode_x4(x);
          uint8_t* codes = const_cast<uint8_t*>(kv ? a.v_codes : a.k_codes) + tile * (KVQ_PAGE_SIZE * D);
          if (lane < D / 4) {
            if (kv == 0) {
              *reinterpret_cast<uint32_t*>(codes + k_tile_offset(4 * lane, slot)) = en.packed;
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) codes[v_tile_offset(4 * lane + q, slot)] = (uint8_t)(en.packed >> (8 * q));
            }
            if ((lane & 15) == 0)
              const_cast<uint16_t*>(kv ? a.v_scales : a.k_scales)[(tile * KVQ_PAGE_SIZE + slot) * NG + (lane >> 4)] =
                  en.scale_bits;
          }
        }
      }
      if (i < PD) fz_mask |= 1 << i;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the stores complete before later loads
#pragma unroll
    for (int i = 0; i < PD && i < PPW; ++i)
      if ((fz_mask >> i) & 1)
        load_fpage_dev(buf[i], a, clampi(bt_row[min(p0 + i * NW, p_cap)], 0, a.num_pages - 1), kvh, lane);
  }

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

  // ---- QK B operands, built by wave 0 into LDS (every wave holds the same rows).  F32 K: the bf16
  // query, step s holding head_dim 32s + 4j .. +3 and 32s + 16 + 4j .. +3.  INT8 K: the query times
  // 2^ex (max |.| of the row in [2^14, 2^15)) in fp16, entry 2g + h holding head_dim 64g + 16j + 8h
  // .. +7, and the scale 2^-ex folded into qmul.
  if (wv == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = 16 * rt + n16;
      const bool valid = r < R;
      const int tq = valid ? r / G : 0, iq = valid ? r % G : 0;
      const int hq = a.g_uniform > 0 ? h0 + iq : a.head_list[h0 + iq];
      const uint16_t* qp = a.q + ((size_t)(b * a.n_q + tq) * a.n_q_heads + hq) * D;
      if constexpr (KF) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint2 lo = valid ? *reinterpret_cast<const uint2*>(qp + 32 * s + 4 * j4) : make_uint2(0u, 0u);
          const uint2 hi = valid ? *reinterpret_cast<const uint2*>(qp + 32 * s + 16 + 4 * j4) : make_uint2(0u, 0u);
          qlds[(rt * NS + s) * 64 + lane] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        if (j4 == 0) qmul_lds[rt * 16 + n16] = a.scale_log2;
      } else {
        uint4 raw[NS];
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < NS; ++e) {
          raw[e] = valid ? *reinterpret_cast<const uint4*>(qp + 64 * (e >> 1) + 16 * j4 + 8 * (e & 1))
                         : make_uint4(0u, 0u, 0u, 0u);
          const uint32_t w[4] = {raw[e].x, raw[e].y, raw[e].z, raw[e].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fmaxf(fabsf(bf16f(w[c] & 0xffffu)), fabsf(bf16f(w[c] >> 16))));
        }
        mx = max_over_row_lanes(mx);
        int ex = 0;
        if (mx > 0.0f) { frexpf(mx, &ex); ex = 15 - ex; }
#pragma unroll
        for (int e = 0; e < NS; ++e) {
          const uint32_t w[4] = {raw[e].x, raw[e].y, raw[e].z, raw[e].w};
          f16x8 f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            f[2 * c] = (_Float16)ldexpf(bf16f(w[c] & 0xffffu), ex);
            f[2 * c + 1] = (_Float16)ldexpf(bf16f(w[c] >> 16), ex);
          }
          qlds[(rt * NS + e) * 64 + lane] = __builtin_bit_cast(uint4, f);
        }
        if (j4 == 0) qmul_lds[rt * 16 + n16] = ldexpf(a.scale_log2, -ex);
      }
    }
  }
  __syncthreads();
  float qmul[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) qmul[rt] = qmul_lds[rt * 16 + n16];
  const uint4* qb = qlds + lane;

  float m_run[RT], l_run[RT], ls[RT][NG];
  f32x4 O[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g) ls[rt][g] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) O[rt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Each wave takes pages p_begin + wv, + NW, ... (at most PPW) and keeps PD pages in flight ahead of
  // the one it processes; the loop is fully unrolled so every wait on the vector memory counter covers
  // exactly the page about to be processed.  Prefetches past the wave's last page re-read it.
  if (p0 < p_end) {
    const int n_mine = (p_end - 1 - p0) / NW + 1;
    const int p_last = p0 + (n_mine - 1) * NW;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int pc = p0 + i * NW;
      if (i + PD < PPW)
        load_fpage(buf[(i + PD) % (PD + 1)], a, clampi(bt_row[min(pc + PD * NW, p_last)], 0, a.num_pages - 1), kvh,
                   lane);
      fpage_step<D, RT, KF, VF>(buf[i % (PD + 1)], pc, j4, Lrow, qb, qmul, m_run, l_run, ls, O);
      if (i + 1 >= n_mine) break;
    }
  }

  // ---- per-wave totals; INT8 V: remove the operand bias (code + 128) through the group weight sums
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] = sum_over_row_lanes(l_run[rt]);
    if constexpr (!VF) {
#pragma unroll
      for (int g = 0; g < NG; ++g) ls[rt][g] = sum_over_row_lanes(ls[rt][g]);
#pragma unroll
      for (int t = 0; t < NT; ++t) O[rt][t] -= 128.0f * ls[rt][t / 4];
    }
  }

  // ---- merge the NW waves, one row tile at a time: waves 1.. store O in LDS, wave 0 merges
  float* lds_o = mrg;                                 // [wave - 1][tile][lane] x f32x4
  float* lds_ml = mrg + (NW - 1) * NT * 64 * 4;       // [wave][row tile][m | l][lane]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    lds_ml[((wv * RT + rt) * 2 + 0) * 64 + lane] = m_run[rt];
    lds_ml[((wv * RT + rt) * 2 + 1) * 64 + lane] = l_run[rt];
  }
  const bool direct = a.n_splits == 1;   // with a single split the workgroup writes the output itself
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (rt > 0) __syncthreads();                      // wave 0 has read the previous tile
    if (wv != 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<f32x4*>(lds_o + (((wv - 1) * NT + t) * 64 + lane) * 4) = O[rt][t];
    }
    __syncthreads();
    if (wv == 0) {
      float cv[NW];
      float M = kNegInf;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        cv[v] = lds_ml[((v * RT + rt) * 2 + 0) * 64 + lane];
        M = fmaxf(M, cv[v]);
      }
      const float Mu = M == kNegInf ? 0.0f : M;
      float l = 0.0f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        cv[v] = __builtin_amdgcn_exp2f(cv[v] - Mu);
        l += cv[v] * lds_ml[((v * RT + rt) * 2 + 1) * 64 + lane];
      }
      const int r = 16 * rt + n16;
      if (r < R) {
        if (!direct && j4 == 0) {
          float* ml = part_ml + ((row0 + r) * a.n_splits + split) * 2;
          ml[0] = M; ml[1] = l;
        }
        const float sc = direct ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f;
        float* row = direct ? a.out + (size_t)decode_out_row(a, b, kvh, r, G, h0) * D
                            : part_o + ((row0 + r) * a.n_splits + split) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {              // value k of tile t: head_dim 16t + 4j + k
          f32x4 acc = O[rt][t] * cv[0];
#pragma unroll
          for (int v = 1; v < NW; ++v)
            acc += cv[v] * *reinterpret_cast<const f32x4*>(lds_o + (((v - 1) * NT + t) * 64 + lane) * 4);
          acc *= sc;
          *reinterpret_cast<float4*>(row + 16 * t + 4 * j4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
  }
}

template <int D, int RT, bool KF, bool VF, int SH>
hipError_t launch_f32_t(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  constexpr FShape sh = kFShapes[SH];
  const dim3 grid((unsigned)plan.n_splits, a.hkv, a.batch), block(sh.nw * 64);
  k_decode_f32<D, RT, KF, VF, sh.nw, sh.ppw, sh.pd><<<grid, block, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return plan.n_splits > 1 ? launch_decode_combine(D, plan, a, s) : hipSuccess;   // one split wrote the output
}

template <int D, bool KF, bool VF>
hipError_t launch_f32_d(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  if (plan.row_tiles > 1)
    return plan.shape == 1 ? launch_f32_t<D, 2, KF, VF, 1>(plan, a, s) : launch_f32_t<D, 2, KF, VF, 0>(plan, a, s);
  return plan.shape == 1 ? launch_f32_t<D, 1, KF, VF, 1>(plan, a, s) : launch_f32_t<D, 1, KF, VF, 0>(plan, a, s);
}

template <bool KF, bool VF>
hipError_t launch_f32_kv(int D, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  if (D == 128) return launch_f32_d<128, KF, VF>(plan, a, s);
  if (D == 256) return launch_f32_d<256, KF, VF>(plan, a, s);
  return hipErrorInvalidValue;
}

}  // namespace

DecodePlan plan_decode_f32(int head_dim, int hkv, int batch, int max_pages, int max_rows) {
  (void)head_dim;
  DecodePlan p{};
  p.rows = max_rows;
  p.row_groups = max(1, (max_rows + 7) / 8);       // partial rows: 8 per group
  p.row_tiles = max(1, (max_rows + 15) / 16);      // MFMA row tiles of 16
  auto splits_of = [&](int sh) {
    const int pps = kFShapes[sh].nw * kFShapes[sh].ppw;
    return (max_pages + pps - 1) / pps;
  };
  // 64-page splits unless they would fill at most about half of the CUs; then 32-page splits
  p.shape = f32_shape_override();
  if (p.shape < 0) p.shape = ((long)splits_of(0) * hkv * batch * 20 <= (long)device_cu_count() * 11) ? 1 : 0;
  p.waves = kFShapes[p.shape].nw;
  p.pages_per_split = kFShapes[p.shape].nw * kFShapes[p.shape].ppw;
  p.n_splits = splits_of(p.shape);
  p.part_bytes = (size_t)batch * hkv * p.n_splits * (8 * p.row_groups) * (head_dim + 2) * sizeof(float);
  return p;
}

hipError_t launch_decode_f32(bool k_f32, bool v_f32, int head_dim, const DecodePlan& plan, const DecodeArgs& a,
                             hipStream_t s) {
  if (k_f32 && v_f32) return launch_f32_kv<true, true>(head_dim, plan, a, s);
  if (k_f32) return launch_f32_kv<true, false>(head_dim, plan, a, s);
  if (v_f32) return launch_f32_kv<false, true>(head_dim, plan, a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
