// Split-K decode attention over Hadamard-rotated q4_0 K and V stores.
//
// strata PR #2698, "Not in this PR": a q4_0 cache rotates K (after RoPE) and V by the FWHT-256,
// rotates the queries, and rotates the output back; strata PR #120, "What": such a cell takes 576
// bytes over two KV heads.  With H = H_256/16 orthonormal and symmetric, a stored key is z = Hk, and
// <q, k> = <Hq, z>: the query is rotated once per workgroup, the codes are used as stored, and the
// values accumulate in the rotated basis (the partial is rotated back, as for k8v4).
//
// Work decomposition: one workgroup = one (sequence, KV head, split of NW * PPW pages); wave w takes
// pages w, w + NW, ... of the split.  At most 16 query rows per KV head, one MFMA column each; with
// at most 8 rows the columns 8-15 repeat them and take the lo parts of split operands (one MFMA
// where 9-16 rows need two).
//   * QK: S^T[token][row] on v_mfma_f32_16x16x32_f16, one MFMA per 32-value scale group.  Lane
//     (w = lane / 16, t = lane % 16) holds slot t's 8 codes 32G + 8w .. +7 of group G (4 bytes of
//     one 16-byte unit of the K tile order); they become the exact fp16 values code - 8 with one
//     byte permute, a mask and a packed fp16 fma per pair.  The B operand is Hq scaled per row by
//     a power of two in fp16 hi + lo parts; each group's accumulator is weighted by its (token,
//     group) d in fp32.
//   * Online softmax in base 2 with a lazily moved reference max (as the other decode kernels).
//   * PV: O^T[d][row] on v_mfma_f32_16x16x16f16: the A operand is 4 tokens' 4-bit codes at one
//     head_dim row as the exact fp16 values code - 8 (a byte permute into 0x64xx and one packed
//     subtract), the B operand the weights times the token's V d in fp16 hi and lo parts (22
//     significant bits).  Every weight carries the wave's factor 2^kexp, from the largest V d of its
//     pages (scanned before the page stream), which keeps weight times d below 2^15 (no fp16
//     overflow, small weights clear of the subnormals); the partial records the reference max
//     minus kexp.
//   * The waves merge through LDS (wave 0 takes whole rows), the partial is rotated back by H and
//     goes to the log-sum-exp combine shared with the other decode kernels.
#include "kvq_internal.h"
#include "device_util.h"
#include "decode_parts.h"

namespace kvq {
namespace {

constexpr int kD = 256;                         // Q4_0_H256: head_dim 256, 8 groups of 32
constexpr int kGroups = 8;
constexpr int kTiles = 16;                      // PV tiles of 16 head_dim rows
constexpr float kLazyQ4 = 8.0f;                 // weights stay below 2^8 between rescalings

// Launch shapes: waves per workgroup, pages per wave per split, pages each wave keeps in flight,
// and the occupancy hint of the launch bounds.  An 8-wave workgroup takes about 150 KB of LDS for its
// merge, so one fits a CU (two waves per SIMD).
struct Q4Shape { int nw, ppw, pd, occ; };
constexpr Q4Shape kQ4Shapes[] = {{4, 16, 1, 1}, {8, 8, 1, 1}, {8, 4, 1, 1}};
constexpr int kNumQ4Shapes = (int)(sizeof(kQ4Shapes) / sizeof(kQ4Shapes[0]));

// KVQ_Q4_DECODE_SHAPE overrides the choice (for tuning); -1 when unset
int q4_shape_override() {
  static int idx = -2;
  if (idx == -2) {
    idx = -1;
    if (const char* e = getenv("KVQ_Q4_DECODE_SHAPE")) {
      const int v = atoi(e);
      if (v >= 0 && v < kNumQ4Shapes) idx = v;
    }
  }
  return idx;
}

// One page of one KV head as a lane holds it.
struct Q4Page {
  uint4 k[2];     // K: unit (h, w, t): bytes 4w .. 4w+3 of groups 4h .. 4h+3 of slot t (word G & 3)
  uint4 ks[4];    // K d (fp16) of tokens 4w .. 4w+3: half j * 8 + G
  uint4 v[2];     // V: unit (64 G' + 4 t + w): word k = code byte 16 (4G' + k) + t of tokens 4w .. 4w+3
  uint4 vs[4];    // V d likewise
  static __device__ __forceinline__ float half_at(const uint4 (&q)[4], int i) {
    const uint32_t x = word_of(q[i >> 3], (i >> 1) & 3);
    return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (x >> 16) : (x & 0xffffu))));
  }
  __device__ __forceinline__ float kd(int j, int G) const { return half_at(ks, j * kGroups + G); }
  __device__ __forceinline__ float vd(int j, int g) const { return half_at(vs, j * kGroups + g); }
};

__device__ __forceinline__ void load_q4_page(Q4Page& pb, const DecodeArgs& a, int page, int kvh, int lane) {
  const int t = lane & 15, w = lane >> 4;
  const size_t tile = (size_t)page * a.hkv + kvh;
  const uint4* kb = reinterpret_cast<const uint4*>(a.k_codes + tile * (16 * 128));
  const uint4* vb = reinterpret_cast<const uint4*>(a.v_codes + tile * (16 * 128));
#pragma unroll
  for (int h = 0; h < 2; ++h) pb.k[h] = stream_load(kb + 64 * h + lane);          // unit (h * 4 + w) * 16 + t
#pragma unroll
  for (int h = 0; h < 2; ++h) pb.v[h] = stream_load(vb + 64 * h + 4 * t + w);
  const uint4* ksb = reinterpret_cast<const uint4*>(a.k_scales + (tile * 16 + 4 * w) * kGroups);
  const uint4* vsb = reinterpret_cast<const uint4*>(a.v_scales + (tile * 16 + 4 * w) * kGroups);
#pragma unroll
  for (int i = 0; i < 4; ++i) pb.ks[i] = ksb[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) pb.vs[i] = vsb[i];
}

// 8 codes of one K group (4 bytes, byte e: codes of dims 2e (low nibble) and 2e + 1) -> the exact
// fp16 values code - 8, in dim order.
__device__ __forceinline__ f16x8 k_group_f16(uint32_t x) {
  // [byte e, 0x64, byte e, 0x64], masked to [lo nibble | 0x6400, hi nibble << 4 | 0x6400]: the low
  // half reads 1024 + lo, the high half 1024 + 16 hi; one packed fma maps them to lo - 8, hi - 8
  const f16x2 mul = {(_Float16)1.0f, (_Float16)0.0625f};
  const f16x2 add = {(_Float16)-1032.0f, (_Float16)-72.0f};
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t sel = 0x04000400u | ((uint32_t)e << 16) | (uint32_t)e;
    const uint32_t y = __builtin_amdgcn_perm(0x64646464u, x, sel) & 0x64f0640fu;
    const f16x2 v = __builtin_bit_cast(f16x2, y) * mul + add;
    r[2 * e] = v[0];
    r[2 * e + 1] = v[1];
  }
  return r;
}

// One page of one wave: QK on MFMA, online softmax, PV on MFMA.  qb: the lane's query fragments
// in LDS, [group][part][lane] (one part with DUP: hi or lo by column).
template <bool DUP>
__device__ __forceinline__ void q4_page_step(const Q4Page& pb, int p, int w, bool lo_col, int Lrow,
                                             const f16x8* qb, float qmul, float kexp, float& m_run, float& l_run,
                                             f32x4 (&O)[kTiles]) {
  constexpr int NP = DUP ? 1 : 2;
  // ---- QK: per group, S^T[token 4w + k][column]; weighted by the group's d
  float sp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int G = 0; G < kGroups; ++G) {
    const f16x8 av = k_group_f16(word_of(pb.k[G >> 2], G & 3));
    f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qb[64 * NP * G], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
    if constexpr (!DUP) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qb[64 * (NP * G + 1)], acc, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) sp[k] = fmaf(acc[k], pb.kd(k, G), sp[k]);
  }
  const int vis = Lrow - (p * KVQ_PAGE_SIZE + 4 * w);      // this lane's tokens k < vis are visible
  float s[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x = sp[k];
    s[k] = k < vis ? (DUP ? x + dpp_ror8(x) : x) * qmul : kNegInf;   // DUP: hi + lo columns
  }
  const float mx = max_over_row_lanes(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
  const bool move = mx > m_run + kLazyQ4;
  const float m_new = move ? mx : m_run;
  const float m_use = m_new == kNegInf ? 0.0f : m_new;
  const bool rescale = move && m_run != kNegInf;
  const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
  m_run = m_new;
  // the weights carry the wave's factor 2^kexp (l and O with them; the partial's m is m_run - kexp)
  const float m_w = m_use - kexp;
  float pk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) pk[k] = __builtin_amdgcn_exp2f(s[k] - m_w);
  l_run = l_run * alpha + ((pk[0] + pk[1]) + (pk[2] + pk[3]));
  if (__any(rescale)) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) O[t] *= alpha;
  }
  // ---- PV per V group g: tiles 2g (even head_dim) and 2g + 1 (odd); masked tokens have pk == 0 (the
  // d of cells past a sequence's length are finite by contract: zero-initialised slabs)
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    // weight times the token's V d in fp16 parts: hi (the rounded product) and lo (the product minus
    // hi, rounded once)
    f16x4 bpart, blo;
    if constexpr (DUP) {
      // one part per column: both parts of a token pair from four mixed-precision fmas, then one
      // packed select per pair
      const uint32_t d0 = word_of(pb.vs[0], (g >> 1) & 3), d1 = word_of(pb.vs[1], (g >> 1) & 3),
                     d2 = word_of(pb.vs[2], (g >> 1) & 3), d3 = word_of(pb.vs[3], (g >> 1) & 3);
      const uint2 p01 = (g & 1) ? mix_parts2<1, 1, 1, 1>(pk[0], d0, pk[1], d1) : mix_parts2<1, 0, 1, 0>(pk[0], d0, pk[1], d1);
      const uint2 p23 = (g & 1) ? mix_parts2<1, 1, 1, 1>(pk[2], d2, pk[3], d3) : mix_parts2<1, 0, 1, 0>(pk[2], d2, pk[3], d3);
      bpart = __builtin_bit_cast(f16x4, lo_col ? make_uint2(p01.y, p23.y) : make_uint2(p01.x, p23.x));
      blo = bpart;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float pw = pk[k] * pb.vd(k, g);
        const _Float16 hi = (_Float16)pw, lo = (_Float16)(pw - (float)hi);
        bpart[k] = hi;
        blo[k] = lo;
      }
    }
    const uint32_t wv = word_of(pb.v[g >> 2], g & 3);      // byte k: token 4w + k; nibbles: dims 32g + 2t (+1)
    const f16x4 alo = nibbles_to_f16x4(wv & 0x0f0f0f0fu), ahi = nibbles_to_f16x4((wv >> 4) & 0x0f0f0f0fu);
    O[2 * g] = __builtin_amdgcn_mfma_f32_16x16x16f16(alo, bpart, O[2 * g], 0, 0, 0);
    O[2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(ahi, bpart, O[2 * g + 1], 0, 0, 0);
    if constexpr (!DUP) {
      O[2 * g] = __builtin_amdgcn_mfma_f32_16x16x16f16(alo, blo, O[2 * g], 0, 0, 0);
      O[2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(ahi, blo, O[2 * g + 1], 0, 0, 0);
    }
  }
}

template <bool DUP, int NW, int PPW, int PD, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void k_decode_q4(const DecodeArgs a) {
  constexpr int NP = DUP ? 1 : 2;                       // query fragment parts per group
  // one LDS allocation, the per-page operands first: the query fragments' addresses then fit the
  // 16-bit offset of the LDS loads (after the merge buffers they would need one more add per read)
  constexpr int kQBytes = kGroups * NP * 64 * 16, kMulBytes = 64 * 4;
  __shared__ __align__(16) uint8_t lds[kQBytes + kMulBytes + NW * (kTiles * 64 * 4 + 2 * 64) * 4];
  f16x8* const qlds = reinterpret_cast<f16x8*>(lds);           // B operands of QK: [group][part][lane]
  float* const qmul_lds = reinterpret_cast<float*>(lds + kQBytes);
  float* const mrg = reinterpret_cast<float*>(lds + kQBytes + kMulBytes);
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t16 = lane & 15, w = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;

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
  const bool lo_col = DUP && t16 >= 8;
  const int r = DUP ? (t16 & 7) : t16;
  const bool valid = r < R;
  const int tq = valid ? r / G : 0, iq = valid ? r % G : 0;
  const int hq = a.g_uniform > 0 ? h0 + iq : a.head_list[h0 + iq];
  const int seq_len = clampi(a.seq_lens[b], 0, cap);
  const int Lrow = valid ? (a.q_lens ? clampi(a.q_lens[(size_t)b * a.n_q + tq], 0, cap) : seq_len) : 0;

  // ---- the wave's page ids (lane l: the wave's page l, clamped to the split and the table; the page
  // loop takes them with lane reads), q, the V d of the wave's pages, then its first PD pages
  // (vector-memory waits are in issue order)
  const int* bt_row = a.bt + (size_t)b * a.max_pages;
  const int p_begin = split * a.pages_per_split;
  const int p0 = p_begin + wv;
  const int p_cap = min(p_begin + a.pages_per_split, a.max_pages) - 1;
  const int my_ids = clampi(bt_row[min(p0 + min(lane, PPW - 1) * NW, p_cap)], 0, a.num_pages - 1);
  auto page_id = [&](int i) -> int { return __builtin_amdgcn_readlane(my_ids, i); };   // i uniform
  uint4 qraw[kGroups];                              // q[row][32G + 8w .. +7]
  {
    const uint16_t* qp = a.q + ((size_t)(b * a.n_q + tq) * a.n_q_heads + hq) * kD + 8 * w;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) qraw[g] = *reinterpret_cast<const uint4*>(qp + 32 * g);
  }
  uint4 vscan[4];                                   // lane l: V d of tokens 4(l & 3) .. + 3 of page l / 4
  {
    const int pid = __shfl(my_ids, min(lane >> 2, PPW - 1));
    const uint4* src =
        reinterpret_cast<const uint4*>(a.v_scales + ((size_t)pid * a.hkv + kvh) * KVQ_PAGE_SIZE * kGroups) + 4 * (lane & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) vscan[i] = src[i];
  }
  Q4Page buf[PD + 1];
#pragma unroll
  for (int i = 0; i < PD && i < PPW; ++i) load_q4_page(buf[i], a, page_id(i), kvh, lane);

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
      for (int i = (int)threadIdx.x; i < R * (kD / 4); i += NW * 64)
        *reinterpret_cast<float4*>(a.out + (size_t)decode_out_row(a, b, kvh, i / (kD / 4), G, h0) * kD +
                                   4 * (i % (kD / 4))) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else if ((int)threadIdx.x < R) {
      float* ml = part_ml + ((row0 + threadIdx.x) * a.n_splits + split) * 2;
      ml[0] = kNegInf; ml[1] = 0.0f;
    }
    return;
  }

  // ---- B operands of QK: Hq (FWHT-256 of the row, x 1/16), times 2^ex (max |.| of the row in
  // [2^14, 2^15)), as fp16 hi + lo parts (DUP: hi in columns 0-7, lo in 8-15).  The lane holds head_dim
  // 32G + 8w + j: bits 0-2 (j) and 5-7 (G) of the index are in-lane, bits 3-4 (w) across lanes.
  // Wave 0 builds them into LDS for the workgroup (every wave holds the same rows).
  if (wv == 0) {
    float x[kGroups][8];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const uint32_t wd[4] = {qraw[g].x, qraw[g].y, qraw[g].z, qraw[g].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[g][2 * e] = valid ? bf16f(wd[e] & 0xffffu) : 0.0f;
        x[g][2 * e + 1] = valid ? bf16f(wd[e] >> 16) : 0.0f;
      }
    }
#pragma unroll
    for (int sp = 1; sp < 8; sp <<= 1)              // spans 1, 2, 4 (in-lane, j)
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!(j & sp)) {
            const float u = x[g][j], v = x[g][j | sp];
            x[g][j] = u + v; x[g][j | sp] = u - v;
          }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {            // spans 8, 16 (lanes xor 16, 32)
      const bool upper = (lane & o) != 0;
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float other = o == 16 ? partner16(x[g][j], lane) : partner32(x[g][j], lane);
          x[g][j] = upper ? (other - x[g][j]) : (x[g][j] + other);
        }
    }
#pragma unroll
    for (int sp = 1; sp < 8; sp <<= 1)              // spans 32, 64, 128 (in-lane, G)
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
        if (!(g & sp))
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float u = x[g][j], v = x[g | sp][j];
            x[g][j] = u + v; x[g | sp][j] = u - v;
          }
    float mx = 0.0f;
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[g][j] *= 0.0625f;
        mx = fmaxf(mx, fabsf(x[g][j]));
      }
    mx = max_over_row_lanes(mx);
    int ex = 0;
    if (mx > 0.0f) { frexpf(mx, &ex); ex = 15 - ex; }
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float y = ldexpf(x[g][j], ex);
        const _Float16 hi = (_Float16)y, lo = (_Float16)(y - (float)hi);
        if constexpr (DUP) {
          qlds[64 * g + lane][j] = lo_col ? lo : hi;
        } else {
          qlds[64 * (2 * g) + lane][j] = hi;
          qlds[64 * (2 * g + 1) + lane][j] = lo;
        }
      }
    qmul_lds[lane] = ldexpf(a.scale_log2, -ex);
  }
  // The weights' factor 2^kexp, from the largest V d of the wave's visible pages: with weights below
  // 2^8 (lazy rescaling) and d < 2^(E - 14) (E: d's fp16 exponent field), 2^(21 - E) keeps every
  // weight times d below 2^15, where its fp16 hi and lo parts are exact to 22 bits, and small weights
  // stay clear of the fp16 subnormals.
  float kexp;
  {
    const int n_w = p0 < p_end ? (p_end - 1 - p0) / NW + 1 : 0;
    uint32_t mx = 0;
    if ((lane >> 2) < n_w) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wd[4] = {vscan[i].x, vscan[i].y, vscan[i].z, vscan[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = max(mx, max(wd[e] & 0x7fffu, (wd[e] >> 16) & 0x7fffu));
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    kexp = (float)(21 - clampi((int)(mx >> 10), 1, 31));
  }
  __syncthreads();
  const float qmul = qmul_lds[lane];
  const f16x8* qb = qlds + lane;

  float m_run = kNegInf, l_run = 0.0f;
  f32x4 O[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) O[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Each wave takes pages p_begin + wv, + NW, ... (at most PPW) and keeps PD pages in flight ahead
  // of the one it processes; the loop is fully unrolled so every wait on the vector memory counter
  // covers exactly the page about to be processed.  Prefetches past the wave's last page re-read it.
  if (p0 < p_end) {
    const int n_mine = (p_end - 1 - p0) / NW + 1;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int pc = p0 + i * NW;
      if (i + PD < PPW) load_q4_page(buf[(i + PD) % (PD + 1)], a, page_id(min(i + PD, n_mine - 1)), kvh, lane);
      q4_page_step<DUP>(buf[i % (PD + 1)], pc, w, lo_col, Lrow, qb, qmul, kexp, m_run, l_run, O);
      if (i + 1 >= n_mine) break;
    }
  }
  // ---- per-wave totals: row sums over the 4 lane groups; the reference of l and O is m_run - kexp
  l_run = sum_over_row_lanes(l_run);
  if (m_run != kNegInf) m_run -= kexp;

  // ---- merge the NW waves: every wave stores (m, l, O) in LDS; wave 0 merges whole rows (the
  // back-rotation needs them)
  float* lds_o = mrg;                               // [wave][tile][lane] x f32x4
  float* lds_ml = mrg + NW * kTiles * 64 * 4;       // [wave][m | l][lane]
  if (wv != 0) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) *reinterpret_cast<f32x4*>(lds_o + ((wv * kTiles + t) * 64 + lane) * 4) = O[t];
  }
  lds_ml[(wv * 2 + 0) * 64 + lane] = m_run;
  lds_ml[(wv * 2 + 1) * 64 + lane] = l_run;
  __syncthreads();
  if (wv != 0) return;
  float cv[NW];
  float M = kNegInf;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    cv[v] = lds_ml[(v * 2 + 0) * 64 + lane];
    M = fmaxf(M, cv[v]);
  }
  const float Mu = M == kNegInf ? 0.0f : M;
  float l = 0.0f;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    cv[v] = __builtin_amdgcn_exp2f(cv[v] - Mu);
    l += cv[v] * lds_ml[(v * 2 + 1) * 64 + lane];
  }
  f32x4 Om[1][kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    f32x4 acc = O[t] * cv[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) acc += cv[v] * *reinterpret_cast<const f32x4*>(lds_o + ((v * kTiles + t) * 64 + lane) * 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {   // DUP: column r + 8 holds the lo-part sums of row r
      const float x = acc[k];
      Om[0][t][k] = DUP ? x + dpp_ror8(x) : x;
    }
  }
  hadamard_rows<1>(Om, lane);
  if (!valid || lo_col) return;
  // with a single split the workgroup writes the normalised output itself (no combine follows)
  const bool direct = a.n_splits == 1;
  if (!direct && w == 0) {
    float* ml = part_ml + ((row0 + r) * a.n_splits + split) * 2;
    ml[0] = M; ml[1] = l;
  }
  const float sc = direct ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f;
  // value (t, k) of Om: head_dim 32 * (t / 2) + 8w + 2k + (t & 1)
  float* row = direct ? a.out + (size_t)((b * a.n_q + tq) * a.n_q_heads + hq) * kD
                      : part_o + ((row0 + r) * a.n_splits + split) * kD;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const f32x4 e = Om[0][2 * g] * sc, o = Om[0][2 * g + 1] * sc;
    *reinterpret_cast<float4*>(row + 32 * g + 8 * w) = make_float4(e[0], o[0], e[1], o[1]);
    *reinterpret_cast<float4*>(row + 32 * g + 8 * w + 4) = make_float4(e[2], o[2], e[3], o[3]);
  }
}

template <int SH>
hipError_t launch_q4_t(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  constexpr Q4Shape sh = kQ4Shapes[SH];
  const dim3 grid((unsigned)plan.n_splits, a.hkv, a.batch), block(sh.nw * 64);
  if (plan.rows <= 8)
    k_decode_q4<true, sh.nw, sh.ppw, sh.pd, sh.occ><<<grid, block, 0, s>>>(a);
  else
    k_decode_q4<false, sh.nw, sh.ppw, sh.pd, sh.occ><<<grid, block, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return plan.n_splits > 1 ? launch_decode_combine(kD, plan, a, s) : hipSuccess;   // one split wrote the output
}

template <int SH = 0>
hipError_t launch_q4_shape(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  if constexpr (SH + 1 < kNumQ4Shapes)
    if (plan.shape != SH) return launch_q4_shape<SH + 1>(plan, a, s);
  return launch_q4_t<SH>(plan, a, s);
}

}  // namespace

DecodePlan plan_decode_q4(int hkv, int batch, int max_pages, int max_rows) {
  DecodePlan p{};
  p.rows = max_rows;
  p.row_groups = max(1, (max_rows + 7) / 8);       // partial rows: 8 or 16
  p.row_tiles = 0;
  auto splits_of = [&](int sh) {
    const int pps = kQ4Shapes[sh].nw * kQ4Shapes[sh].ppw;
    return (max_pages + pps - 1) / pps;
  };
  // More 64-page splits than CUs: 4-wave workgroups (two share a CU).  Otherwise one 8-wave workgroup
  // per CU, each wave with half the pages: 64-page splits while they fill more than half of the CUs,
  // else 32-page splits.  Measured launches for one sequence over two KV heads (4x16 / 4x8 / 8x8 /
  // 8x4 waves x pages): 131,072 tokens 37.8 / 39.8 / 35.5 / 48.8 us; 65,536 tokens 37.0 / 26.9 / 34.3
  // / 26.4 us; 32,768 tokens 36.6 / 26.3 / 33.8 / 25.8 us.
  p.shape = q4_shape_override();
  if (p.shape < 0) {
    const long n64 = (long)splits_of(0) * hkv * batch, cus = device_cu_count();
    p.shape = n64 > cus ? 0 : (2 * n64 > cus ? 1 : 2);
  }
  p.waves = kQ4Shapes[p.shape].nw;
  p.pages_per_split = kQ4Shapes[p.shape].nw * kQ4Shapes[p.shape].ppw;
  p.n_splits = splits_of(p.shape);
  p.part_bytes = (size_t)batch * hkv * p.n_splits * (8 * p.row_groups) * (kD + 2) * sizeof(float);
  return p;
}

hipError_t launch_decode_q4(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s) {
  return launch_q4_shape(plan, a, s);
}

}  // namespace kvq
