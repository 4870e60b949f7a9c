// Split-K decode / MTP-verify attention over the packed paged cache.
//
// strata PR #2698, "What it does": decode and verify windows dequantise K and V on the fly inside
// the attention kernels, which split the context into parts whose partial results are combined.
// strata PR #120, "How": k8v4 keeps K int8 and unrotated (q is never rotated) and accumulates V
// in the Hadamard-rotated basis, rotating only the output back; "Tests": verify rows carry their
// own causal lengths (per-query step arrays).
//
// Work decomposition (one workgroup = one (sequence, KV head, split) triple):
//   * The query rows of a KV head are its (query token, query head) pairs: n_q * G <= 32 rows, in
//     groups of 8 (one workgroup each; MFMA columns 8..15 repeat the group's rows, see DUP below).
//     k8v4 with more than 8 rows per KV head runs in the wave-pair verify kernel (decode_verify.hip).
//   * Each wave streams every NW-th page of the split: K codes token-major (16 B per lane per
//     64-group: the lane's token is lane % 16), V codes d-major (4 tokens of one head_dim
//     position per 32-bit load), both with 256-byte-coalesced wave accesses.
//   * QK: S^T[token][row] with v_mfma_f32_16x16x32_f16.  int8 codes become fp16 exactly through
//     a byte permute into 0x64xx (= 1024 + byte) and one packed fp16 subtract; q is pre-scaled
//     by a power of two per row so that its bf16 values convert to fp16 exactly.  Each 64-group
//     accumulates separately and is weighted by its (token, group) scale in fp32.
//   * Online softmax in base 2 per row; the row max is shared by the 4 lanes holding a row's 16
//     tokens of a page; the running sum stays per lane until the end.
//   * PV: O^T[d][row] with a 16x16x16 MFMA.  The B operand is the S^T accumulator layout itself
//     (lane: 4 tokens x 1 row) after exp2 and multiplication by the (token, group) V scale, split
//     into a hi and a lo part.  int8 V: fp16 parts (22 significant bits) against the 4 tokens'
//     codes at one head_dim position as exact fp16 values (the permute above); every weight
//     carries the wave's factor 2^kexp, from the largest V scale of its pages, which keeps weight
//     times scale below 2^15 (no fp16 overflow, small weights clear of the subnormals); the
//     partial records the reference max minus kexp.  q4_0 V (k8v4, up to 8 rows): bf16 parts
//     (16 bits) against (code + 128) in bf16 -- 4-bit code, value code - 8 -- with the offset
//     removed at the end from the per-group sums of the weights.  Every MFMA tile of 16 head_dim
//     rows lies inside one scale group, so one weight vector per group serves all its tiles.
//   * The NW waves of a workgroup merge (m, l, O) through LDS in one round (each wave merges and
//     writes a share of the head_dim tiles; k8v4 rotates the merged partial back by H); the
//     workgroup writes one unnormalised partial.  A second kernel merges the splits with a
//     log-sum-exp combine, normalises and writes fp32 rows.
#include "kvq_internal.h"
#include "device_util.h"
#include "int8_cell.h"
#include "decode_parts.h"
#include "q4h_cell.h"

namespace kvq {
namespace {

// Launch shapes: waves per workgroup, pages per wave per split (a split is NW * PPW pages), pages
// each wave keeps in flight ahead of the one it processes, and waves per SIMD the registers allow.
// The last shape plans the k8v4 verify kernel's 64-page splits (decode_verify.hip: 4 wave pairs of
// 16 pages each); with 32-page splits it takes shape 1 (4 pairs of 8 pages).
struct Shape { int nw, ppw, pd, occ; };
constexpr Shape kShapes[] = {{4, 16, 2, 2}, {4, 8, 1, 2}, {8, 8, 1, 2}, {4, 16, 1, 2}};
constexpr int kRowTileShape = 3;
constexpr int kNumShapes = (int)(sizeof(kShapes) / sizeof(kShapes[0]));

// KVQ_DECODE_SHAPE overrides the choice (for tuning); -1 when unset
int shape_override() {
  static int idx = -2;
  if (idx == -2) {
    idx = -1;
    if (const char* e = getenv("KVQ_DECODE_SHAPE")) {
      const int v = atoi(e);
      if (v >= 0 && v < kNumShapes) idx = v;
    }
  }
  return idx;
}


// Cache loads: non-temporal when each page is read by one workgroup (streamed once), plain when the
// row groups of a split read it in turn (the later ones then find it in L2).
template <bool NT>
__device__ __forceinline__ uint4 page_load(const void* p) {
  if constexpr (NT) return stream_load(p);
  else return *reinterpret_cast<const uint4*>(p);
}

template <int N>
__device__ __forceinline__ void load_words(uint32_t (&dst)[N], const uint32_t* src) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const uint4 t = stream_load(src + 4 * c);
      dst[4 * c] = t.x; dst[4 * c + 1] = t.y; dst[4 * c + 2] = t.z; dst[4 * c + 3] = t.w;
    }
  } else {
    static_assert(N == 2, "scale words come in pairs or multiples of 4");
    const uint2 t = *reinterpret_cast<const uint2*>(src);
    dst[0] = t.x; dst[1] = t.y;
  }
}

// One page of one KV head as a lane holds it.  Every code load is one 16-byte load per lane that
// covers a contiguous kilobyte of the tile across the wave (see the tile byte orders in kvq.h).
template <int D, int VF>
struct PageBuf {
  static constexpr int NG = D / 64;                      // K scale groups (one 16-byte K load each)
  static constexpr int NVG = VF == 1 ? D / 64 : D / 32;  // V scale groups
  static constexpr int NVQ = VF == 1 ? D / 64 : D / 128; // 16-byte V loads
  uint4 k[NG];                // K: token lane%16, head_dim 64g + 16*(lane/16) .. +15
  uint4 v[NVQ];               // V: word k of v[G] = 4 tokens 4*(lane/16).. at one head_dim row of tile 4G+k
  uint32_t ks[2 * NG];        // fp16 pairs: K scale of token 4*(lane/16) + k, group g is half k*NG + g
  uint32_t vs[2 * NVG];       // V scales likewise
  __device__ __forceinline__ float kscale(int k, int g) const { return half_at(ks, k * NG + g); }
  __device__ __forceinline__ float vscale(int k, int g) const { return half_at(vs, k * NVG + g); }
  static __device__ __forceinline__ float half_at(const uint32_t* w, int i) {
    const uint32_t x = w[i >> 1];
    return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (x >> 16) : (x & 0xffffu))));
  }
};

template <int D, int VF, bool NT>
__device__ __forceinline__ void load_page(PageBuf<D, VF>& pb, const DecodeArgs& a, int page, int kvh, int lane) {
  constexpr int NG = PageBuf<D, VF>::NG, NVG = PageBuf<D, VF>::NVG;
  const int i16 = lane & 15, j4 = lane >> 4;
  const size_t tile = (size_t)page * a.hkv + kvh;
  // K tile: 16-byte chunk c of slot t at (c * 16 + t) * 16; this lane's chunk for group g is 4g + j4
  const uint4* kb = reinterpret_cast<const uint4*>(a.k_codes + tile * (16 * D)) + lane;
#pragma unroll
  for (int g = 0; g < NG; ++g) pb.k[g] = page_load<NT>(kb + 64 * g);
  load_words<2 * NG>(pb.ks, reinterpret_cast<const uint32_t*>(a.k_scales + (tile * 16 + 4 * j4) * NG));
  // V tile: 16-byte unit (64*G + 4*i16 + j4) holds tiles 4G..4G+3 (one word each) of row i16
  const uint4* vb = reinterpret_cast<const uint4*>(a.v_codes + tile * (16 * (VF == 1 ? D : D / 2))) + 4 * i16 + j4;
#pragma unroll
  for (int G = 0; G < PageBuf<D, VF>::NVQ; ++G) pb.v[G] = page_load<NT>(vb + 64 * G);
  load_words<2 * NVG>(pb.vs, reinterpret_cast<const uint32_t*>(a.v_scales + (tile * 16 + 4 * j4) * NVG));
}

// q fragments (B operand of QK) in LDS, 64 lanes apart
template <int NG>
struct QLds {
  const f16x8* p;
  __device__ __forceinline__ f16x8 operator()(int rt, int g, int h) const { return p[((rt * NG + g) * 2 + h) * 64]; }
};

// Device-scope loads of a page (int8 V): they miss the CU's L1 and read L2, so a page this wave
// loaded, then wrote cells into (and waited for), comes back with them.
__device__ __forceinline__ uint4 load_dev16(const void* base, uint32_t off) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0x10 /* sc1: device scope */);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int D>
__device__ __forceinline__ void load_page_dev(PageBuf<D, 1>& pb, const DecodeArgs& a, int page, int kvh, int lane) {
  constexpr int NG = D / 64;
  const int i16 = lane & 15, j4 = lane >> 4;
  const size_t tile = (size_t)page * a.hkv + kvh;
  const uint8_t* kb = a.k_codes + tile * (16 * D);
  const uint8_t* vb = a.v_codes + tile * (16 * D);
#pragma unroll
  for (int g = 0; g < NG; ++g) pb.k[g] = load_dev16(kb, 16 * (64 * g + lane));
#pragma unroll
  for (int g = 0; g < NG; ++g) pb.v[g] = load_dev16(vb, 16 * (64 * g + 4 * i16 + j4));
  const uint8_t* ks = reinterpret_cast<const uint8_t*>(a.k_scales + (tile * 16 + 4 * j4) * NG);
  const uint8_t* vs = reinterpret_cast<const uint8_t*>(a.v_scales + (tile * 16 + 4 * j4) * NG);
#pragma unroll
  for (int c = 0; c < 2 * NG; c += 4) {
    if constexpr (NG >= 2) {
      const uint4 k4 = load_dev16(ks, 4 * c), v4 = load_dev16(vs, 4 * c);
      pb.ks[c] = k4.x; pb.ks[c + 1] = k4.y; pb.ks[c + 2] = k4.z; pb.ks[c + 3] = k4.w;
      pb.vs[c] = v4.x; pb.vs[c + 1] = v4.y; pb.vs[c + 2] = v4.z; pb.vs[c + 3] = v4.w;
    }
  }
  if constexpr (NG == 1) {
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ks), (short)0, 0x7fffffff, 0x00020000);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vs), (short)0, 0x7fffffff, 0x00020000);
    pb.ks[0] = __builtin_amdgcn_raw_buffer_load_b32(rk, 0, 0, 0x10);
    pb.ks[1] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4, 0, 0x10);
    pb.vs[0] = __builtin_amdgcn_raw_buffer_load_b32(rv, 0, 0, 0x10);
    pb.vs[1] = __builtin_amdgcn_raw_buffer_load_b32(rv, 4, 0, 0x10);
  }
}

// The same for an int8 K + Hadamard-rotated q4_0 V page (head_dim 256).
template <int D>
__device__ __forceinline__ void load_page_dev(PageBuf<D, 2>& pb, const DecodeArgs& a, int page, int kvh, int lane) {
  constexpr int NG = D / 64, NVG = D / 32;
  const int i16 = lane & 15, j4 = lane >> 4;
  const size_t tile = (size_t)page * a.hkv + kvh;
  const uint8_t* kb = a.k_codes + tile * (16 * D);
  const uint8_t* vb = a.v_codes + tile * (16 * (D / 2));
#pragma unroll
  for (int g = 0; g < NG; ++g) pb.k[g] = load_dev16(kb, 16 * (64 * g + lane));
#pragma unroll
  for (int G = 0; G < PageBuf<D, 2>::NVQ; ++G) pb.v[G] = load_dev16(vb, 16 * (64 * G + 4 * i16 + j4));
  // scales of tokens 4 j4 .. 4 j4 + 3: (tile * 16 + 4 j4) * N halves from the (uniform) tile start
  const uint8_t* ks = reinterpret_cast<const uint8_t*>(a.k_scales + tile * 16 * NG);
  const uint8_t* vs = reinterpret_cast<const uint8_t*>(a.v_scales + tile * 16 * NVG);
  static_assert((2 * NG) % 4 == 0 && (2 * NVG) % 4 == 0, "scale words in 16-byte units");
#pragma unroll
  for (int c = 0; c < 2 * NG; c += 4) {
    const uint4 x = load_dev16(ks, 8 * j4 * NG + 4 * c);
    pb.ks[c] = x.x; pb.ks[c + 1] = x.y; pb.ks[c + 2] = x.z; pb.ks[c + 3] = x.w;
  }
#pragma unroll
  for (int c = 0; c < 2 * NVG; c += 4) {
    const uint4 x = load_dev16(vs, 8 * j4 * NVG + 4 * c);
    pb.vs[c] = x.x; pb.vs[c + 1] = x.y; pb.vs[c + 2] = x.z; pb.vs[c + 3] = x.w;
  }
}

constexpr float kLazyLog2 = 8.0f;     // weights stay below 2^8 between rescalings

// One page of one wave: QK on MFMA, online softmax, PV on MFMA.
// DUP (at most 8 rows): MFMA columns 8..15 repeat rows 0..7; columns 0..7 take the hi part of the
// softmax weights and columns 8..15 the lo part, so one PV MFMA per tile does both (int8 V: fp16
// parts against the exact fp16 codes; q4_0 V: bf16 parts against biased bf16 codes).  (k8v4 with
// more than 8 rows per KV head runs in the wave-pair verify kernel.)
template <int D, int RT, int VF, bool DUP, class QF>
__device__ __forceinline__ void page_step(const PageBuf<D, VF>& pb, int p, int j4, bool lo_col, const int (&Lrow)[RT],
                                          const QF& qf, const float (&qmul)[RT], float kexp,
                                          float (&m_run)[RT], float (&l_run)[RT],
                                          float (&ls)[RT][VF == 1 ? D / 64 : D / 32], f32x4 (&O)[RT][D / 16]) {
  constexpr int NG = D / 64;
  constexpr int NVG = VF == 1 ? D / 64 : D / 32;
  constexpr int NT = D / 16;
  static_assert(DUP, "rows beyond 8 per KV head take one workgroup per group of 8 rows");

  // ---- QK: S^T[token 4*j4 + k][row] per 64-group
  f32x4 acc[RT][NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const f16x8 a0 = codes_to_f16(pb.k[g].x, pb.k[g].y);
    const f16x8 a1 = codes_to_f16(pb.k[g].z, pb.k[g].w);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const f16x8 b0 = qf(rt, g, 0), b1 = qf(rt, g, 1);
      acc[rt][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      acc[rt][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, acc[rt][g], 0, 0, 0);
    }
  }
  const int tok0 = p * KVQ_PAGE_SIZE + 4 * j4;

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float s[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v = acc[rt][0][k] * pb.kscale(k, 0);
#pragma unroll
      for (int g = 1; g < NG; ++g) v = fmaf(acc[rt][g][k], pb.kscale(k, g), v);
      s[k] = (tok0 + k < Lrow[rt]) ? v * qmul[rt] : kNegInf;
    }
    // Lazy rescaling: the exponentials are taken against a reference max m_run that moves only
    // when a score exceeds it by more than kLazyLog2 (so every weight stays below 2^kLazyLog2),
    // not on every increase of the running max; O and l are rescaled only then, and not at all
    // while they are still zero.  The partial's (m, l, O) all refer to m_run, which is all the
    // log-sum-exp combine needs.
    const float mx = max_over_row_lanes(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    const bool move = mx > m_run[rt] + kLazyLog2;
    const float m_new = move ? mx : m_run[rt];
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const bool rescale = move && m_run[rt] != kNegInf;
    const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run[rt] - m_use) : 1.0f;
    m_run[rt] = m_new;
    // int8 V: the weights carry the wave's factor 2^kexp (l and O with them; the partial's m is
    // m_run - kexp)
    const float m_w = VF == 1 ? m_use - kexp : m_use;
    float pk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pk[k] = __builtin_amdgcn_exp2f(s[k] - m_w);
    l_run[rt] = l_run[rt] * alpha + ((pk[0] + pk[1]) + (pk[2] + pk[3]));
    if (__any(rescale)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) O[rt][t] *= alpha;
      if constexpr (VF != 1) {
#pragma unroll
        for (int g = 0; g < NVG; ++g) ls[rt][g] *= alpha;
      }
    }

    // ---- PV per V scale group
#pragma unroll
    for (int g = 0; g < NVG; ++g) {
      float pw[4];
#pragma unroll
      // masked tokens have pk == 0; the scales of cells past a sequence's length are finite by
      // contract (zero-initialised slabs), so their weights are exact zeros without a select
      for (int k = 0; k < 4; ++k) pw[k] = pk[k] * pb.vscale(k, g);
      if constexpr (VF == 1) {
        // fp16 parts of the weights (below 2^15 by the choice of kexp) against the exact fp16 codes:
        // columns 0..7 the rounded weight, 8..15 its rounding error
        f16x4 bw;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const _Float16 hi = (_Float16)pw[k];
          bw[k] = lo_col ? (_Float16)(pw[k] - (float)hi) : hi;
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int t = 4 * g + tt;
          O[rt][t] = __builtin_amdgcn_mfma_f32_16x16x16f16(codes_to_f16x4(word_of(pb.v[g], tt)), bw, O[rt][t], 0, 0, 0);
        }
        continue;
      }
      // q4_0 V: biased bf16 codes (pair row 16g + i16: d = 32g + 2*i16 (+1)) against bf16 parts
      s16x4 bhi;
      float used[4];
      split_bf16_select(pw, lo_col ? 0xffffffffu : 0u, bhi, used);
      ls[rt][g] += (used[0] + used[1]) + (used[2] + used[3]);
      const uint32_t w = word_of(pb.v[g >> 2], g & 3);
      O[rt][2 * g] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(nibbles_to_bf16_biased(w & 0x0f0f0f0fu), bhi,
                                                               O[rt][2 * g], 0, 0, 0);
      O[rt][2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(nibbles_to_bf16_biased((w >> 4) & 0x0f0f0f0fu),
                                                                   bhi, O[rt][2 * g + 1], 0, 0, 0);
    }
  }
}

template <int D, int RT, int VF, int NW, int PPW, int PD, int OCC, bool DUP, bool NTL>
__global__ __launch_bounds__(NW * 64, OCC) void k_decode_split(const DecodeArgs a) {
  constexpr int NG = D / 64;
  constexpr int NVG = VF == 1 ? D / 64 : D / 32;
  constexpr int NT = D / 16;                                // PV tiles of 16 head_dim rows
  constexpr float kOff = 136.0f;                            // bias carried by the q4_0 V A-operand
  const int RA = a.row_alloc;                               // allocated rows per (sequence, KV head)

  // wave-uniform wave index: page addresses are scalar arithmetic
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, j4 = lane >> 4;
  // blockIdx.x -> (split, row group) so that the row groups of a split share blockIdx.x % 8, i.e.
  // run on the same XCD (workgroups are dealt to the 8 XCDs round robin) and share its L2.
  // Without duplicated columns one workgroup holds all rows (RT row tiles of 16).
  const int n_rg = DUP ? a.row_groups : 1;
  const int xg = blockIdx.x, rem = xg % (8 * n_rg);
  const int rg = rem >> 3, split = (xg / (8 * n_rg)) * 8 + (rem & 7);
  const int kvh = blockIdx.y, b = blockIdx.z;
  if (split >= a.n_splits) return;                          // the grid is rounded up to 8 splits

  // ---- rows of this KV head.  With the default grouping (query head h reads KV head h / G) the
  // q addresses are arithmetic on kernel arguments; an explicit head map goes through the lists.
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
  const bool lo_col = DUP && i16 >= 8;
  int Lrow[RT];
  bool valid[RT];
  int qrow[RT];
  const int seq_len = clampi(a.seq_lens[b], 0, cap);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = DUP ? 8 * (rg + rt) + (i16 & 7) : 16 * rt + i16;
    valid[rt] = r < R;
    const int t = valid[rt] ? r / G : 0;
    const int i = valid[rt] ? r % G : 0;
    const int hq = a.g_uniform > 0 ? h0 + i : a.head_list[h0 + i];
    qrow[rt] = (b * a.n_q + t) * a.n_q_heads + hq;
    Lrow[rt] = valid[rt] ? (a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + t], 0, cap) : seq_len) : 0;
  }
  // ---- then q (one batch), then this wave's first PD pages.  Vector-memory waits are in issue
  // order, so everything the prologue needs is issued before the page stream; the pages depend
  // only on page-table entries of this split (clamped to the table), not on lengths or rows, and a
  // page past the sequence's end is loaded but never processed.
  const int* bt_row = a.bt + (size_t)b * a.max_pages;
  const int p_begin = split * a.pages_per_split;
  const int p0 = p_begin + wv;
  const int p_cap = min(p_begin + a.pages_per_split, a.max_pages) - 1;
  // Page id of this wave's i-th page (clamped to the split and the table).  The kernel may store
  // the step's new cells, so the compiler cannot prove the table unchanged by those stores: scalar
  // loads of it would become vector loads, each waited for with vmcnt(0).  Instead lane l reads the
  // id of the wave's page l in one vector load at entry, and the page loop takes the ids with lane
  // reads.
  const int my_ids = clampi(bt_row[min(p0 + min(lane, PPW - 1) * NW, p_cap)], 0, a.num_pages - 1);
  auto page_id = [&](int i) -> int {          // i: index in this wave's page list, uniform
    return __builtin_amdgcn_readlane(my_ids, i);
  };
  // Fused quantize-on-write (int8 K; int8 or, at head_dim 256, Hadamard-rotated q4_0 V): new token t
  // of this sequence goes to position
  // seq_len - n_q + t.  The wave whose page list holds that cell loads the token now, encodes and
  // stores it before the page loop and waits for the stores, so the loop's load of that page
  // returns the cell; a page the prologue already loaded is loaded again (device scope, past the
  // CU's L1).  Every row-group workgroup of the split stores the cell itself: the bytes are
  // identical, and each reads back after its own store.
  int fz_idx[kDecodeMaxFused], fz_slot[kDecodeMaxFused];   // page index in this wave's list (-1: not ours)
  uint2 fz_x[kDecodeMaxFused][2];
  int fz_mask = 0;                                          // bit i: page i of this wave has new cells
#pragma unroll
  for (int t = 0; t < kDecodeMaxFused; ++t) {
    fz_idx[t] = -1;
    fz_slot[t] = 0;
    // a sequence shorter than the window (an idle slot of length 0, say) has no cell for the
    // tokens that would sit before position 0: they are skipped, never written elsewhere
    if (a.k_new && t < a.n_q && seq_len - a.n_q + t >= 0) {
      const int pos = seq_len - a.n_q + t;                  // <= seq_len - 1 <= cap - 1
      const int pl = pos / KVQ_PAGE_SIZE - p_begin;
      if (pl >= 0 && pl < a.pages_per_split && pl % NW == wv) {
        fz_idx[t] = pl / NW;
        fz_slot[t] = pos % KVQ_PAGE_SIZE;
        fz_mask |= 1 << fz_idx[t];
        const size_t off = ((size_t)(b * a.n_q + t) * a.hkv + kvh) * D + 4 * min(lane, D / 4 - 1);
        fz_x[t][0] = *reinterpret_cast<const uint2*>(a.k_new + off);
        fz_x[t][1] = *reinterpret_cast<const uint2*>(a.v_new + off);
      }
    }
  }
  uint4 raw[RT][NG][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const uint16_t* qp = a.q + (size_t)qrow[rt] * D + 16 * j4;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      raw[rt][g][0] = *reinterpret_cast<const uint4*>(qp + 64 * g);
      raw[rt][g][1] = *reinterpret_cast<const uint4*>(qp + 64 * g + 8);
    }
  }
  // LDS: q fragments (one copy for the workgroup: every wave holds the same rows), then the wave
  // merge buffers
  constexpr int kQBytes = RT * NG * 2 * 64 * 16;
  constexpr int kMergeBytes = NW * (NT * 64 * 16 + 2 * 64 * 4);   // one row tile at a time
  __shared__ __align__(16) uint8_t smem[kQBytes + kMergeBytes];
  // int8 V: the V scales of this wave's pages (lane l reads a quarter of the scales of page l / 4 of
  // the wave's list), issued before the page stream so that waiting for them waits for nothing else
  constexpr int kScanWords = 2 * NG;
  uint32_t vscan[kScanWords] = {};
  if constexpr (VF == 1) {
    const int pid = __shfl(my_ids, min(lane >> 2, PPW - 1));
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(a.v_scales + ((size_t)pid * a.hkv + kvh) * KVQ_PAGE_SIZE * NG) +
        (lane & 3) * kScanWords;
    if constexpr (kScanWords == 2) {
      const uint2 t = *reinterpret_cast<const uint2*>(src);
      vscan[0] = t.x; vscan[1] = t.y;
    } else {
#pragma unroll
      for (int c = 0; c < kScanWords / 4; ++c) {
        const uint4 t = *reinterpret_cast<const uint4*>(src + 4 * c);
        vscan[4 * c] = t.x; vscan[4 * c + 1] = t.y; vscan[4 * c + 2] = t.z; vscan[4 * c + 3] = t.w;
      }
    }
  }
  PageBuf<D, VF> buf[PD + 1];
#pragma unroll
  for (int i = 0; i < PD && i < PPW; ++i)
    load_page<D, VF, NTL>(buf[i], a, page_id(i), kvh, lane);

  int Lmax = 0;
  for (int t = 0; t < a.n_q; ++t)
    Lmax = max(Lmax, a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + t], 0, cap) : seq_len);
  const int npages = (Lmax + KVQ_PAGE_SIZE - 1) / KVQ_PAGE_SIZE;
  const int p_end = min(p_begin + a.pages_per_split, npages);
  // partials: m/l [B][Hkv][RA][n_splits][2], then O [B][Hkv][RA][n_splits][D]
  const size_t row0 = (size_t)(b * a.hkv + kvh) * RA;
  float* part_ml = a.part;
  float* part_o = a.part + (size_t)a.batch * a.hkv * RA * a.n_splits * 2;
  // ---- encode this wave's new cells into the cache; pages of the prologue that hold one are
  // loaded again once the stores have completed
  uint32_t fz_vmax = 0;                                     // the new cells' V scales (int8 V)
  if (fz_mask) {
#pragma unroll
    for (int t = 0; t < kDecodeMaxFused; ++t) {
      if (fz_idx[t] < 0) continue;
      const size_t tile = (size_t)page_id(fz_idx[t]) * a.hkv + kvh;
      if constexpr (VF == 2) {                              // q4_0 V: the whole wave encodes one cell
        static_assert(VF != 2 || D == 256, "Hadamard-rotated q4_0 needs head_dim 256");
        float y[4] = {bf16f(fz_x[t][1].x & 0xffffu), bf16f(fz_x[t][1].x >> 16), bf16f(fz_x[t][1].y & 0xffffu),
                      bf16f(fz_x[t][1].y >> 16)};
        const Q4x4 e = q4h_encode_x4(y, lane);
        uint8_t* codes = const_cast<uint8_t*>(a.v_codes) + tile * (KVQ_PAGE_SIZE * (D / 2));
        codes[v_tile_offset(2 * lane, fz_slot[t])] = e.b0;
        codes[v_tile_offset(2 * lane + 1, fz_slot[t])] = e.b1;
        if ((lane & 7) == 0)
          const_cast<uint16_t*>(a.v_scales)[(tile * KVQ_PAGE_SIZE + fz_slot[t]) * (D / 32) + (lane >> 3)] = e.d_bits;
      }
#pragma unroll
      for (int kv = 0; kv < (VF == 1 ? 2 : 1); ++kv) {
        const float x[4] = {bf16f(fz_x[t][kv].x & 0xffffu), bf16f(fz_x[t][kv].x >> 16),
                            bf16f(fz_x[t][kv].y & 0xffffu), bf16f(fz_x[t][kv].y >> 16)};
        const Int8x4 e = int8_encode_x4(x);
        if (lane < D / 4) {
          uint8_t* codes = const_cast<uint8_t*>(kv ? a.v_codes : a.k_codes) + tile * (KVQ_PAGE_SIZE * D);
          uint16_t* scales = const_cast<uint16_t*>(kv ? a.v_scales : a.k_scales);
          if (kv == 0) {
            *reinterpret_cast<uint32_t*>(codes + k_tile_offset(4 * lane, fz_slot[t])) = e.packed;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) codes[v_tile_offset(4 * lane + q, fz_slot[t])] = (uint8_t)(e.packed >> (8 * q));
          }
          if ((lane & 15) == 0) scales[(tile * KVQ_PAGE_SIZE + fz_slot[t]) * NG + (lane >> 4)] = e.scale_bits;
          if (kv == 1) fz_vmax = max(fz_vmax, (uint32_t)(e.scale_bits & 0x7fffu));
        }
      }
    }
    // the stores complete before any later load of this wave (the page loop's loads of these pages)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < PD && i < PPW; ++i)
      if ((fz_mask >> i) & 1) load_page_dev<D>(buf[i], a, page_id(i), kvh, lane);
  }

  // int8 V: the weights' factor 2^kexp, from the largest V scale d of the wave's visible pages (the
  // scan may read a new cell's slot as it was before this wave's store: the encoder's own scales are
  // included).  With weights below 2^8 (lazy rescaling) and d < 2^(E - 14) (E: d's fp16 exponent
  // field), 2^(21 - E) keeps every weight times d below 2^15, where its fp16 hi and lo parts are
  // exact to 22 bits, and small weights stay clear of the fp16 subnormals.
  float kexp = 0.0f;
  if constexpr (VF == 1) {
    const int n_w = p0 < p_end ? (p_end - 1 - p0) / NW + 1 : 0;
    uint32_t mx = fz_vmax;
    if ((lane >> 2) < n_w) {
#pragma unroll
      for (int c = 0; c < kScanWords; ++c) mx = max(mx, max(vscan[c] & 0x7fffu, (vscan[c] >> 16) & 0x7fffu));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    kexp = (float)(21 - clampi((int)(mx >> 10), 1, 31));
  }

  if (R == 0) return;
  if (p_begin >= p_end) {                                   // nothing visible in this split
    const int r_lo = DUP ? 8 * rg : 0, r_hi = min(R, r_lo + (DUP ? 8 * RT : RA));
    if (a.n_splits == 1) {                                  // the only split writes the output: zeros
      for (int i = (int)threadIdx.x; i < (r_hi - r_lo) * (D / 4); i += NW * 64)
        *reinterpret_cast<float4*>(a.out + (size_t)decode_out_row(a, b, kvh, r_lo + i / (D / 4), G, h0) * D +
                                   4 * (i % (D / 4))) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else if ((int)threadIdx.x < r_hi - r_lo) {
      float* ml = part_ml + ((row0 + r_lo + threadIdx.x) * a.n_splits + split) * 2;
      ml[0] = kNegInf; ml[1] = 0.0f;
    }
    return;
  }

  // q fragments of this lane (B operand of QK) live in LDS: [rt][g][half][lane] x 16 bytes,
  // written by wave 0
  const QLds<NG> qlds{reinterpret_cast<const f16x8*>(smem) + lane};
  float qmul[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float mx = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (!valid[rt]) raw[rt][g][h] = make_uint4(0, 0, 0, 0);
        const uint32_t w[4] = {raw[rt][g][h].x, raw[rt][g][h].y, raw[rt][g][h].z, raw[rt][g][h].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mx = fmaxf(mx, fmaxf(fabsf(bf16f(w[e] & 0xffffu)), fabsf(bf16f(w[e] >> 16))));
      }
    mx = max_over_row_lanes(mx);
    int ex = 0;
    if (mx > 0.0f) { frexpf(mx, &ex); ex = 15 - ex; }        // max * 2^ex in [2^14, 2^15)
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w[4] = {raw[rt][g][h].x, raw[rt][g][h].y, raw[rt][g][h].z, raw[rt][g][h].w};
        f16x8 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = (_Float16)ldexpf(bf16f(w[e] & 0xffffu), ex);
          f[2 * e + 1] = (_Float16)ldexpf(bf16f(w[e] >> 16), ex);
        }
        if (wv == 0) const_cast<f16x8*>(qlds.p)[((rt * NG + g) * 2 + h) * 64] = f;
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

  // Each wave takes pages p_begin + wv, + NW, ... (at most PPW of them) and keeps PD pages in
  // flight ahead of the one it processes, in a ring of PD + 1 register buffers (the first PD were
  // issued at kernel entry).  The page loop is
  // fully unrolled, so the ring index is a constant and the code is straight-line with forward
  // exits only: every wait on the vector memory counter then covers exactly the page about to be
  // processed.  Prefetches past the wave's last page re-read that page (an L2 hit), so no branch
  // guards a load.
  __syncthreads();                                          // q fragments written by wave 0
  if (p0 < p_end) {
    const int n_mine = (p_end - 1 - p0) / NW + 1;          // pages of this wave, >= 1
    // page i of the wave sits in ring slot i % (PD + 1)
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int pc = p0 + i * NW;
      if (i + PD < PPW) load_page<D, VF, NTL>(buf[(i + PD) % (PD + 1)], a, page_id(min(i + PD, n_mine - 1)), kvh, lane);
      page_step<D, RT, VF, DUP>(buf[i % (PD + 1)], pc, j4, lo_col, Lrow, qlds, qmul, kexp, m_run, l_run, ls, O);
      if (i + 1 >= n_mine) break;
    }
  }

  // ---- per-wave totals: row sums over the 4 lane groups; int8 V: the reference of l and O is
  // m_run - kexp; q4_0 V: remove the V operand bias
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] = sum_over_row_lanes(l_run[rt]);
    if constexpr (VF == 1) {
      if (m_run[rt] != kNegInf) m_run[rt] -= kexp;
    } else {
#pragma unroll
      for (int g = 0; g < NVG; ++g) ls[rt][g] = sum_over_row_lanes(ls[rt][g]);
#pragma unroll
      for (int t = 0; t < NT; ++t) O[rt][t] -= kOff * ls[rt][t / 2];
    }
  }

  // ---- merge the NW waves, one row tile at a time.  Every wave stores (m, l, O) in LDS, then
  // wave w merges tiles w, w + NW, ... of all waves (int8 V); k8v4 needs whole rows for its
  // Hadamard, so there wave 0 merges everything.
  float* lds_o = reinterpret_cast<float*>(smem + kQBytes);           // [wave][t][lane] x f32x4
  float* lds_ml = lds_o + NW * NT * 64 * 4;                           // [wave][m | l][lane]
  const bool direct = a.n_splits == 1;
  if constexpr (VF == 1 && NW > 1 && (D / 16) % NW == 0) {
    // int8 V (one row tile, duplicated columns): straight-line code -- wave w's tiles are
    // t = w + NW * tt, held in a statically indexed array, so the LDS reads of all of them are in
    // flight together and no branch separates them
    static_assert(RT == 1 && DUP, "one row tile of duplicated columns");
    constexpr int TPW = NT / NW;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(lds_o + ((wv * NT + t) * 64 + lane) * 4) = O[0][t];
    lds_ml[(wv * 2 + 0) * 64 + lane] = m_run[0];
    lds_ml[(wv * 2 + 1) * 64 + lane] = l_run[0];
    __syncthreads();
    float mv[NW], lv[NW], cv[NW];
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      mv[v] = lds_ml[(v * 2 + 0) * 64 + lane];
      lv[v] = lds_ml[(v * 2 + 1) * 64 + lane];
      M = fmaxf(M, mv[v]);
    }
    const float Mu = M == kNegInf ? 0.0f : M;
    float l = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      cv[v] = __builtin_amdgcn_exp2f(mv[v] - Mu);
      l += cv[v] * lv[v];
    }
    f32x4 mo[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int t = wv + NW * tt;
      f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int v = 0; v < NW; ++v) acc += cv[v] * *reinterpret_cast<const f32x4*>(lds_o + ((v * NT + t) * 64 + lane) * 4);
      // column r + 8 holds the lo-part sums of row r: add them in (each DPP source a scalar copy,
      // written to a fresh vector: see dpp_ror8)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x = acc[k];
        mo[tt][k] = x + dpp_ror8(x);
      }
    }
    // the workgroup's partial for rows r < R; with a single split the normalised output itself
    const int r = 8 * rg + i16;
    if (r >= R || i16 >= 8) return;
    float* row = direct ? a.out + (size_t)qrow[0] * D : part_o + ((row0 + r) * a.n_splits + split) * D;
    const float sc = direct ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f;
    if (!direct && j4 == 0 && wv == 0) {
      float* ml = part_ml + ((row0 + r) * a.n_splits + split) * 2;
      ml[0] = M; ml[1] = l;
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)                   // lane holds d = 16t + 4*j4 + k
      *reinterpret_cast<float4*>(row + 16 * (wv + NW * tt) + 4 * j4) =
          make_float4(mo[tt][0] * sc, mo[tt][1] * sc, mo[tt][2] * sc, mo[tt][3] * sc);
    return;
  }
  if constexpr (NW > 1) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (rt > 0) __syncthreads();                          // the previous row tile is merged
      if (VF == 1 || wv != 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(lds_o + ((wv * NT + t) * 64 + lane) * 4) = O[rt][t];
      }
      lds_ml[(wv * 2 + 0) * 64 + lane] = m_run[rt];
      lds_ml[(wv * 2 + 1) * 64 + lane] = l_run[rt];
      __syncthreads();
      if (VF == 2 && wv != 0) continue;
      float mv[NW], cv[NW];
      float M = kNegInf;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        mv[v] = lds_ml[(v * 2 + 0) * 64 + lane];
        M = fmaxf(M, mv[v]);
      }
      const float Mu = M == kNegInf ? 0.0f : M;
      float l = 0.0f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        cv[v] = __builtin_amdgcn_exp2f(mv[v] - Mu);
        l += cv[v] * lds_ml[(v * 2 + 1) * 64 + lane];
      }
      m_run[rt] = M;
      l_run[rt] = l;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (VF == 1 && t % NW != wv) continue;
        f32x4 acc = VF == 1 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : O[rt][t] * cv[0];
#pragma unroll
        for (int v = (VF == 1 ? 0 : 1); v < NW; ++v)
          acc += cv[v] * *reinterpret_cast<const f32x4*>(lds_o + ((v * NT + t) * 64 + lane) * 4);
        O[rt][t] = acc;
      }
    }
    if (VF == 2 && wv != 0) return;
  }
  if constexpr (DUP) {            // column r + 8 holds the lo-part sums of row r: add them in
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (VF == 1 && NW > 1 && t % NW != wv) continue;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x = O[rt][t][k];
          O[rt][t][k] = x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
        }
      }
  }
  // k8v4: rotate the (unnormalised) partial back now; the combine is linear, so H commutes with it
  if constexpr (VF == 2) hadamard_rows<RT>(O, lane);

  // ---- write the workgroup's partial for rows r < R; with a single split, the normalised output
  // itself (no combine launch follows)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = DUP ? 8 * (rg + rt) + i16 : 16 * rt + i16;
    if (r >= R || (DUP && i16 >= 8)) continue;
    float* row = direct ? a.out + (size_t)qrow[rt] * D : part_o + ((row0 + r) * a.n_splits + split) * D;
    const float sc = direct ? (l_run[rt] > 0.0f ? 1.0f / l_run[rt] : 0.0f) : 1.0f;
    auto put4 = [&](float* p, float x0, float x1, float x2, float x3) {
      *reinterpret_cast<float4*>(p) = make_float4(x0 * sc, x1 * sc, x2 * sc, x3 * sc);
    };
    if (!direct && j4 == 0 && wv == 0) {
      float* ml = part_ml + ((row0 + r) * a.n_splits + split) * 2;
      ml[0] = m_run[rt]; ml[1] = l_run[rt];
    }
    if constexpr (VF == 1) {
#pragma unroll
      for (int t = 0; t < NT; ++t)   // lane holds d = 16t + 4*j4 + k
        if (NW == 1 || t % NW == wv) put4(row + 16 * t + 4 * j4, O[rt][t][0], O[rt][t][1], O[rt][t][2], O[rt][t][3]);
    } else {
#pragma unroll
      for (int g = 0; g < NVG; ++g) {  // tiles 2g (even d) / 2g+1 (odd d): d = 32g + 8*j4 + 2k (+1)
        const f32x4 e = O[rt][2 * g], o = O[rt][2 * g + 1];
        put4(row + 32 * g + 8 * j4, e[0], o[0], e[1], o[1]);
        put4(row + 32 * g + 8 * j4 + 4, e[2], o[2], e[3], o[3]);
      }
    }
  }
}

// Log-sum-exp combine of the split partials of one (64 head_dim values, row, KV head, sequence)
// slice by one workgroup of 256 threads: M = max of the split maxima, then 16 groups of 16 lanes
// stream the splits' 64-value slices weighted by 2^(m_s - M) and an LDS reduction normalises.
constexpr int kMaxSplits = 8192;

template <int D, int KPER>
__device__ __forceinline__ void combine_slice(const DecodeArgs& a, int row_alloc, int b, int kvh, int r, int c) {
  __shared__ float red[256];
  __shared__ float4 acc_s[256];
  const int tid = threadIdx.x;
  const bool act = tid < 256;                               // a split workgroup may have more threads
  const int h0 = a.g_uniform > 0 ? kvh * a.g_uniform : a.head_off[kvh];
  const int G = a.g_uniform > 0 ? a.g_uniform : a.head_off[kvh + 1] - h0;
  const int t = r / G, hq = a.g_uniform > 0 ? h0 + r % G : a.head_list[h0 + r % G];
  const int S = a.n_splits;
  const size_t row = (size_t)(b * a.hkv + kvh) * row_alloc + r;
  const float* ml = a.part + row * S * 2;
  const float* po = a.part + (size_t)a.batch * a.hkv * row_alloc * S * 2 + row * S * D;   // row's [S][D]
  // (m, l) of split s; 4 values of split s at head_dim d
  auto ml_of = [&](int s) -> float2 { return *reinterpret_cast<const float2*>(ml + 2 * s); };
  auto o_of = [&](int s, int d) -> float4 { return *reinterpret_cast<const float4*>(po + (size_t)s * D + d); };

  // Each thread reads the (m, l) and 4 output values of its splits s = sl, sl + 16, ... up front, KPER
  // of them per pass (all loads of a pass in flight together), then the row max and the sum of weights
  // come from LDS reductions over the 16 split lanes that share a head_dim group.
  constexpr int kPer = KPER;                                // splits per thread held in registers
  const int sl = tid >> 4, d = 64 * c + 4 * (tid & 15);
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float mx = kNegInf, den = 0.0f;                           // acc and den are relative to 2^mx
  for (int s0 = 0; s0 < S; s0 += 16 * kPer) {
    float2 mlv[kPer];
    float4 ov[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s = min(s0 + sl + 16 * k, S - 1);
      mlv[k] = act ? ml_of(s) : make_float2(kNegInf, 0.0f);
      ov[k] = act ? o_of(s, d) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (s0 + sl + 16 * k >= S) mlv[k].y = 0.0f;           // past the last split: weight 0
    }
    // running rescale: acc is kept relative to mx
    float m_new = mx;
#pragma unroll
    for (int k = 0; k < kPer; ++k) m_new = mlv[k].y > 0.0f ? fmaxf(m_new, mlv[k].x) : m_new;
    const float mu = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = mx == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mx - mu);
    acc.x *= alpha; acc.y *= alpha; acc.z *= alpha; acc.w *= alpha;
    den *= alpha;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const bool on = mlv[k].y > 0.0f;
      const float w = on ? __builtin_amdgcn_exp2f(mlv[k].x - mu) : 0.0f;
      acc.x += on ? w * ov[k].x : 0.0f; acc.y += on ? w * ov[k].y : 0.0f;
      acc.z += on ? w * ov[k].z : 0.0f; acc.w += on ? w * ov[k].w : 0.0f;
      den += on ? w * mlv[k].y : 0.0f;
    }
    mx = m_new;
  }
  // merge the 16 split lanes: common max, rescale, sum
  if (act) red[tid] = mx;
  __syncthreads();
  float M = kNegInf;
  if (act) {
#pragma unroll
    for (int g = 0; g < 16; ++g) M = fmaxf(M, red[16 * g + (tid & 15)]);
  }
  const float Mu = M == kNegInf ? 0.0f : M;
  const float scale = mx == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mx - Mu);
  __syncthreads();
  if (act) {
    acc.x *= scale; acc.y *= scale; acc.z *= scale; acc.w *= scale;
    acc_s[tid] = acc;
    red[tid] = den * scale;
  }
  __syncthreads();
  float total = 0.0f;                                       // one den per split lane group
#pragma unroll
  for (int g = 0; g < 16; ++g) total += red[16 * g];
  if (tid < 16) {
    float4 sum = acc_s[tid];
#pragma unroll
    for (int g = 1; g < 16; ++g) {
      const float4 v = acc_s[16 * g + tid];
      sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
    }
    const float inv = total > 0.0f ? 1.0f / total : 0.0f;
    float* out = a.out + (((size_t)b * a.n_q + t) * a.n_q_heads + hq) * D + 64 * c + 4 * tid;
    *reinterpret_cast<float4*>(out) = make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
  }
  __syncthreads();                                          // red / acc_s are reused by the next slice
}

template <int D, int KPER>
__global__ __launch_bounds__(256) void k_decode_combine(const DecodeArgs a, int row_alloc) {
  constexpr int NC = D / 64;
  const int c = blockIdx.x % NC, r = blockIdx.x / NC, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.g_uniform > 0 ? a.g_uniform : a.head_off[kvh + 1] - a.head_off[kvh];
  if (r >= a.n_q * G) return;
  combine_slice<D, KPER>(a, row_alloc, b, kvh, r, c);
}


template <int D>
hipError_t launch_combine_t(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  // splits per thread and pass: 8 for many splits (one pass covers 128), 2 for at most 32 (no loads of
  // clamped split indices; 32 sequences over 8 KV heads at 4,096-32,768 tokens: 237.0 -> 234.8 us,
  // while 128 splits take 33.5 us with 8 against 33.9 with 4 and 34.6 with 2)
  dim3 cgrid((D / 64) * plan.rows, a.hkv, a.batch);
  if (plan.n_splits <= 32) k_decode_combine<D, 2><<<cgrid, dim3(256), 0, s>>>(a, a.row_alloc);
  else k_decode_combine<D, 8><<<cgrid, dim3(256), 0, s>>>(a, a.row_alloc);
  return hipGetLastError();
}

template <int D, int RT, int VF, int SH>
hipError_t launch_t(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  constexpr Shape sh = kShapes[SH];
  // with several row-group workgroups per split (duplicated columns, 8 rows each) the splits are
  // padded to a multiple of 8 (see the blockIdx mapping); a workgroup holding all rows in row
  // tiles of 16 needs one wave per SIMD's registers
  const bool groups = plan.row_tiles == 0 && plan.row_groups > 1;
  const int gx = groups ? (plan.n_splits + 7) / 8 * 8 * plan.row_groups : plan.n_splits;
  const dim3 grid((unsigned)gx, a.hkv, a.batch), block(sh.nw * 64);
  if (plan.row_tiles > 0) return hipErrorInvalidValue;   // the wave-pair verify kernel takes these
  if (!groups) {
    k_decode_split<D, 1, VF, sh.nw, sh.ppw, sh.pd, sh.occ, true, true><<<grid, block, 0, s>>>(a);
  } else {
    k_decode_split<D, 1, VF, sh.nw, sh.ppw, sh.pd, sh.occ, true, false><<<grid, block, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return plan.n_splits > 1 ? launch_combine_t<D>(plan, a, s) : hipSuccess;   // one split wrote the output
}

template <int D, int RT, int VF>
hipError_t launch_shape(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  switch (plan.shape) {
    case 1: return launch_t<D, RT, VF, 1>(plan, a, s);
    case 2:                                   // 8 waves: not with several row tiles (LDS)
      if constexpr (RT == 1) return launch_t<D, RT, VF, 2>(plan, a, s);
      else return launch_t<D, RT, VF, 0>(plan, a, s);
    default: return launch_t<D, RT, VF, 0>(plan, a, s);
  }
}

}  // namespace

int decode_max_splits() { return kMaxSplits; }

DecodePlan plan_decode(int v_fmt, int head_dim, int hkv, int batch, int max_pages, int max_rows) {
  DecodePlan p{};
  // up to 8 query rows per KV head share one MFMA (weights' hi parts in columns 0-7, lo parts in
  // 8-15); more rows take one workgroup per group of 8 rows, except with a k8v4 V store, where the
  // wave-pair verify kernel holds all rows in row tiles of 16 (its V operand built once per page)
  p.rows = max_rows;
  p.row_groups = max(1, (max_rows + 7) / 8);
  p.row_tiles = (v_fmt == KVQ_FMT_Q4_0_H256 && max_rows > 8) ? (max_rows + 15) / 16 : 0;
  // 64-page splits (16 pages per wave, two in flight) unless they fill at most about half of the
  // CUs; then 32-page splits (twice the workgroups, one page in flight).  Measured: 64-page splits
  // win at 90% of the CUs (232 workgroups, 31.5 vs 33.5 us), 32-page splits at 50% (128, 22.7 vs
  // 28.7 us).  The k8v4 verify kernel plans its 64-page splits as shape kRowTileShape.
  auto splits_of = [&](int sh) { return (max_pages + kShapes[sh].nw * kShapes[sh].ppw - 1) / (kShapes[sh].nw * kShapes[sh].ppw); };
  p.shape = shape_override();
  if (p.shape < 0) {
    p.shape = 0;
    if ((long)splits_of(0) * hkv * batch * (p.row_tiles ? 1 : p.row_groups) * 20 <= (long)device_cu_count() * 11)
      p.shape = 1;
    else if (p.row_tiles)
      p.shape = kRowTileShape;
  }
  if (p.shape == kRowTileShape && !p.row_tiles) p.shape = 0;
  const Shape sh = kShapes[p.shape];
  p.waves = sh.nw;
  p.pages_per_split = sh.nw * sh.ppw;
  p.n_splits = splits_of(p.shape);
  if (!p.row_tiles && shape_override() < 0 && p.shape == 1) {
    // 64-page splits fill at most about half of the CUs: the fewest pages per split (a multiple of the
    // 4 waves, at most 32) that keeps one round, so more CUs work and each takes fewer pages (40,000
    // tokens: 125 splits of 20 pages, 17.5 us, against 79 of 32, 18.6 us).  At 78-90% of the CUs the
    // same rule does not pay: the kernel is bound by HBM there (100,000 tokens 28.3 vs 27.8 us).
    const long per = (long)device_cu_count() / ((long)hkv * batch * p.row_groups);
    if (per >= 1) {
      const long need = (max_pages + per - 1) / per;
      p.pages_per_split = (int)min(32L, max(4L, (need + 3) / 4 * 4));
      p.n_splits = (max_pages + p.pages_per_split - 1) / p.pages_per_split;
    }
  }
  if (p.row_tiles && shape_override() < 0) {
    // the verify kernel (one 8-wave workgroup per CU): the fewest pages per split, a multiple of its 4
    // wave pairs and at most 64, that keeps the workgroups within one round of the CUs, so every CU
    // works and each takes fewer pages (118,750 tokens: 116 splits of 64 pages on 232 CUs ->
    // 124 of 60 on 248)
    const long per = max(1L, (long)device_cu_count() / ((long)hkv * batch));
    const long need = (max_pages + per - 1) / per;
    p.pages_per_split = (int)min(64L, max(4L, (need + 3) / 4 * 4));
    p.n_splits = (max_pages + p.pages_per_split - 1) / p.pages_per_split;
  }
  p.part_bytes = (size_t)batch * hkv * p.n_splits * (8 * p.row_groups) * (head_dim + 2) * sizeof(float);
  return p;
}

hipError_t launch_decode_combine(int D, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  switch (D) {
    case 64: return launch_combine_t<64>(plan, a, s);
    case 128: return launch_combine_t<128>(plan, a, s);
    case 256: return launch_combine_t<256>(plan, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(int v_fmt, int D, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  if (v_fmt == KVQ_FMT_Q4_0_H256)
    return plan.row_tiles > 0 ? launch_decode_verify(plan.row_tiles, plan, a, s) : launch_shape<256, 1, 2>(plan, a, s);
  switch (D) {
    case 64: return launch_shape<64, 1, 1>(plan, a, s);
    case 128: return launch_shape<128, 1, 1>(plan, a, s);
    case 256: return launch_shape<256, 1, 1>(plan, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
