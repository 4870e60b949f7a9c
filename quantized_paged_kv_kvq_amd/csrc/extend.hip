// Extend (prefill chunk) attention over an ISO3- or int8-packed prefix plus the chunk's own bf16 tokens.
//
// FreeToken PR #398, "What": a prefill chunk attends the cached prefix, which is held packed,
// and its own new tokens, which are packed only after the chunk's attention (deferred packing);
// prompt-chunk attention dequantises the packed prefix once into a scratch that a tiled kernel
// then reads.  Token i of a chunk at position P + i sees the P prefix cells and new tokens 0..i.
//
// Two kernels:
//   * k_extend_stage writes, for every 64-key tile of every (sequence, KV head), the image of the
//     tile as the attention kernel's LDS holds it: K as [key][head_dim] and V as [head_dim][key]
//     (transposed for the PV contraction), both with rows padded so that the MFMA operand reads
//     are free of bank conflicts, plus the per-key norms.  Prefix tiles come from the
//     ISO3 cells (the dequantisation runs once per cell, not once per query tile); chunk tiles from
//     the bf16 tokens.
//   * k_extend_attn: one workgroup = 8 waves = one (sequence, KV head, 8 * T query tokens) tile; a
//     wave owns 32 query rows (T tokens x G_pad query heads), the 32 columns of 32x32x16 MFMA
//     tiles: lane l holds row l % 32 and, per 32-key block, 16 of its scores.  Tile images stream
//     into LDS with direct global-to-LDS loads (no registers) through a ring of three buffers.
//     The waves form two groups of 4 that run one barrier phase apart, so that one group's
//     softmax overlaps the other group's MFMAs (one workgroup per CU).
//
// Prefix phase (rotated basis).  An ISO3 key is k = n * conj(r) (x) c with c the centroid values of
// its codes, so <q, k> = n * <r (x) q, c>: the query is rotated once, the codes are used as they
// are, and the norm scales the score.  Likewise sum_j p_j v_j = conj(r) (x) sum_j (p_j n_j) c_j:
// values accumulate in the rotated basis and the accumulator is rotated back once at the end of
// the phase.  The centroid values enter the fp16 MFMA as S * c rounded to fp16, with the common
// factor S chosen so that all eight products lie within 2^-15.9 of their fp16 roundings (plain
// fp16 rounding of c would cost 2^-12); 1/S is folded into the query and into the weights.  The
// rotated query and the weights p * n / S are split into fp16 hi + lo parts (22 significant bits),
// so each QK and each PV tile takes two MFMAs.
//
// Chunk phase (original basis, bf16 MFMA).  q and the new K/V are bf16 and enter the bf16 MFMA
// exactly; the weights are split into bf16 hi + lo parts (16 significant bits).  Causal mask per
// row; tiles past a wave's last token are skipped.
//
// Online softmax in base 2 per row across both phases; the row max is shared by the 4 lanes that
// hold a row's keys, the running sums stay per lane until the end.
//
// INT8_G64 prefix (strata PR #2698, "What it does": a prompt chunk reads the int8 cache range
// dequantised, there by a dequantise-to-f16 kernel feeding a GEMM).  Here the stage writes the exact
// codes as fp16 (|code| <= 127) and the fp32 scales of both 64-value groups of every key; the
// attention forms each key's score from its two group partials weighted by the group scales (the
// query enters unscaled and exact in one fp16 part), and splits
// the weights times the key's V group scale into fp16 hi + lo parts per group.  Rounding the
// dequantised values to fp16 instead (code x scale has up to 18 significant bits) measured up to
// 1.8e-3 off on the CPU for short prefixes.  No rotation; head_dim 128 as ISO3.
#include "kvq_internal.h"
#include "iso_levels.h"
#include "device_util.h"

namespace kvq {
namespace {

constexpr int kD = 128;
constexpr int kWaves = kExtendWaves;                       // attention workgroup: two groups of 4 waves
constexpr int kKeys = 64;                                  // keys per tile
constexpr int kQkDepth = 2;                                // QK operand reads in flight ahead of the MFMAs (steps)
constexpr int kKRow = kD * 2 + 16;                         // K image row: one key, 256 B + 16 B pad
constexpr int kVRow = kKeys * 2 + 16;                      // V image row: one head_dim, 128 B + 16 B pad
constexpr int kImgK = kKeys * kKRow;                       // K image bytes: [key][d] fp16/bf16
constexpr int kImgV = kD * kVRow;                          // V image bytes: [d][key position]
constexpr int kNormOff = kImgK + kImgV;                    // fp32 K norms [64], then V norms / S [64]
static_assert(kNormOff + 2 * kKeys * 4 <= kExtendTileBytes, "tile image layout");
// int8 prefix tiles: fp32 [K s0 / s1, K s1, V s0, V s1][64] (s_g: group scales) instead
static_assert(kNormOff + 4 * kKeys * 4 <= kExtendTileBytes, "int8 tile image layout");
static_assert(kExtendTileBytes % 1024 == 0, "a tile image is whole kilobytes");

// Byte offsets inside a tile image: 16-byte chunk c (head_dim 8c .. 8c+7) of key k, and 16-byte
// chunk c (key positions 8c .. 8c+7) of head_dim row d.  The 16-byte row padding makes the 16 rows
// that a 16-lane group of an MFMA operand read touches start in 16 different bank quads.
__device__ __forceinline__ int k_img_off(int key, int c) { return key * kKRow + (c << 4); }
__device__ __forceinline__ int v_img_off(int d, int c) { return kImgK + d * kVRow + (c << 4); }

// Position order of a tile's keys in a V row: inside each 16-key group, positions 8h .. 8h+7 hold
// keys 4h .. 4h+3 and 8+4h .. 8+4h+3, the 8 keys that lane half h of a 32x32 MFMA accumulator holds
// for one 16-key step, so one 16-byte read gives a PV A-operand lane the keys of its B operand.
__device__ __forceinline__ int key_at(int pos) {
  const int p16 = pos & 15, e = p16 & 7;
  return (pos & ~15) + 8 * (e >> 2) + 4 * (p16 >> 3) + (e & 3);
}

// r (x) u for a quaternion r = (w, x, y, z) and a group u = (u0, u1, u2, u3).
__device__ __forceinline__ void qmul(float w, float x, float y, float z, const float u[4], float t[4]) {
  t[0] = ((w * u[0] - x * u[1]) - y * u[2]) - z * u[3];
  t[1] = ((w * u[1] + x * u[0]) + y * u[3]) - z * u[2];
  t[2] = ((w * u[2] - x * u[3]) + y * u[0]) + z * u[1];
  t[3] = ((w * u[3] + x * u[2]) - y * u[1]) + z * u[0];
}

__device__ __forceinline__ uint8_t* prefix_image(const ExtendArgs& a, int b, int kvh, int t) {
  return a.ws + ((size_t)(b * a.hkv + kvh) * a.pt_max + t) * kExtendTileBytes;
}
__device__ __forceinline__ uint8_t* chunk_image(const ExtendArgs& a, int b, int kvh, int t) {
  return a.ws + (size_t)a.batch * a.hkv * a.pt_max * kExtendTileBytes +
         ((size_t)(b * a.hkv + kvh) * a.nt_max + t) * kExtendTileBytes;
}

// ============================== staging ==============================
struct StageLds {
  union {
    uint32_t raw[2][kKeys * 12 + 4];                        // ISO3 codes of the tile's keys (K, V), 48 B each
    uint4 raw8[2][4 * KVQ_PAGE_SIZE * kD / 16];             // int8: the 4 pages' K and V code tiles
  };
  uint16_t level[8];                                         // S * c as fp16
  __attribute__((aligned(16))) uint8_t img[kExtendTileBytes];
};

// 3-bit code of head_dim d of key `key` from the staged 48-byte rows (little-endian bit stream).
__device__ __forceinline__ uint32_t code_at(const uint32_t* raw, int key, int d) {
  const int bit = 3 * d, w = key * 12 + (bit >> 5);
  return __builtin_amdgcn_alignbit(raw[w + 1], raw[w], bit & 31) & 7u;
}

__global__ __launch_bounds__(256) void k_extend_stage(const ExtendArgs a) {
  __shared__ StageLds s;
  const int tid = threadIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int s0 = clampi(a.cu_new[b], 0, a.n_new);
  const int n_b = clampi(a.cu_new[b + 1], s0, a.n_new) - s0;
  const int P = clampi(a.prefix_lens[b], 0, a.max_pages * KVQ_PAGE_SIZE);

  if ((int)blockIdx.x < a.pt_max && a.int8) {
    // INT8_G64 prefix tile (4 whole pages): images of the exact codes in fp16 and the fp32 scales of
    // both 64-value groups of every key; the attention weights each group's partial sums by them.
    const int t = blockIdx.x;
    if (t * kKeys >= P) return;
    const int* bt_row = a.bt + (size_t)b * a.max_pages;
    for (int i = tid; i < 2 * 4 * 128; i += 256) {          // 16-byte units: store, page j, unit u
      const int st = i >> 9, j = (i >> 7) & 3, u = i & 127;
      const int pos = min(t * kKeys + 16 * j, P - 1);
      const int page = clampi(bt_row[pos >> 4], 0, a.num_pages - 1);
      const uint8_t* src = (st ? a.v_codes : a.k_codes) + ((size_t)page * a.hkv + kvh) * (KVQ_PAGE_SIZE * kD);
      s.raw8[st][j * 128 + u] = reinterpret_cast<const uint4*>(src)[u];
    }
    if (tid < kKeys) {
      const int pos = t * kKeys + tid;
      const bool live = pos < P;
      const int pc = min(pos, P - 1);
      const int page = clampi(bt_row[pc >> 4], 0, a.num_pages - 1);
      const size_t cell = ((size_t)page * a.hkv + kvh) * KVQ_PAGE_SIZE + (pc & 15);
      // K: the factors of (S0 * s0 / s1 + S1) * s1 (S0 * s0 when s1 = 0); V: the group scales
      float* sc = reinterpret_cast<float*>(s.img + kNormOff);
      const float k0 = live ? h2f(a.k_norms[cell * 2]) : 0.0f, k1 = live ? h2f(a.k_norms[cell * 2 + 1]) : 0.0f;
      sc[tid] = k1 > 0.0f ? k0 / k1 : k0;
      sc[kKeys + tid] = k1 > 0.0f ? k1 : 1.0f;
#pragma unroll
      for (int g = 0; g < 2; ++g) sc[(2 + g) * kKeys + tid] = live ? h2f(a.v_norms[cell * 2 + g]) : 0.0f;
    }
    __syncthreads();
    {   // K image: thread = (key, 32 head_dim values = chunks 2q, 2q + 1 of the key's slot)
      const int key = tid >> 2, q = tid & 3;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 ch = s.raw8[0][(key >> 4) * 128 + (2 * q + (c >> 1)) * 16 + (key & 15)];
        const uint32_t w0 = (c & 1) ? ch.z : ch.x, w1 = (c & 1) ? ch.w : ch.y;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t src = e < 2 ? w0 : w1;
          const int sh = 16 * (e & 1);
          const _Float16 lo = (_Float16)(float)(int8_t)(src >> sh), hi = (_Float16)(float)(int8_t)(src >> (sh + 8));
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *reinterpret_cast<uint4*>(s.img + k_img_off(key, 4 * q + c)) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    {   // V image: thread = (head_dim row, 32 key positions)
      const int d = tid >> 1, h = tid & 1;
      const uint8_t* vr = reinterpret_cast<const uint8_t*>(s.raw8[1]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = 32 * h + 8 * c + 2 * e;
          const int k0 = key_at(p), k1 = key_at(p + 1);
          const _Float16 lo = (_Float16)(float)(int8_t)vr[(k0 >> 4) * 2048 + v_tile_offset(d, k0 & 15)];
          const _Float16 hi = (_Float16)(float)(int8_t)vr[(k1 >> 4) * 2048 + v_tile_offset(d, k1 & 15)];
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *reinterpret_cast<uint4*>(s.img + v_img_off(d, 4 * h + c)) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    __syncthreads();
    uint4* dst = reinterpret_cast<uint4*>(prefix_image(a, b, kvh, t));
    const uint4* src = reinterpret_cast<const uint4*>(s.img);
    for (int i = tid; i < kExtendTileBytes / 16; i += 256) dst[i] = src[i];
  } else if ((int)blockIdx.x < a.pt_max) {
    const int t = blockIdx.x;
    if (t * kKeys >= P) return;
    const int* bt_row = a.bt + (size_t)b * a.max_pages;
    for (int i = tid; i < kKeys * 12; i += 256) {
      const int key = i / 12, w = i % 12;
      const int pos = min(t * kKeys + key, P - 1);
      const int page = clampi(bt_row[pos >> 4], 0, a.num_pages - 1);
      const size_t cell = ((size_t)page * a.hkv + kvh) * KVQ_PAGE_SIZE + (pos & 15);
      s.raw[0][i] = reinterpret_cast<const uint32_t*>(a.k_codes + cell * 48)[w];
      s.raw[1][i] = reinterpret_cast<const uint32_t*>(a.v_codes + cell * 48)[w];
    }
    if (tid < 8) s.level[tid] = __builtin_bit_cast(uint16_t, (_Float16)(kIsoLevelScale * kIsoLevels[tid]));
    if (tid < 4) { s.raw[0][kKeys * 12 + tid] = 0u; s.raw[1][kKeys * 12 + tid] = 0u; }
    if (tid < kKeys) {
      const int pos = t * kKeys + tid;
      const bool live = pos < P;
      const int pc = min(pos, P - 1);
      const int page = clampi(bt_row[pc >> 4], 0, a.num_pages - 1);
      const size_t cell = ((size_t)page * a.hkv + kvh) * KVQ_PAGE_SIZE + (pc & 15);
      float* norms = reinterpret_cast<float*>(s.img + kNormOff);
      norms[tid] = live ? h2f(a.k_norms[cell]) : 0.0f;
      norms[kKeys + tid] = live ? h2f(a.v_norms[cell]) * (1.0f / kIsoLevelScale) : 0.0f;
    }
    __syncthreads();
    {   // K image: thread = (key, 32 head_dim values)
      const int key = tid >> 2, q = tid & 3;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 32 * q + 8 * c + 2 * e;
          w[e] = (uint32_t)s.level[code_at(s.raw[0], key, d)] |
                 ((uint32_t)s.level[code_at(s.raw[0], key, d + 1)] << 16);
        }
        *reinterpret_cast<uint4*>(s.img + k_img_off(key, 4 * q + c)) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    {   // V image: thread = (head_dim row, 32 key positions)
      const int d = tid >> 1, h = tid & 1;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = 32 * h + 8 * c + 2 * e;
          w[e] = (uint32_t)s.level[code_at(s.raw[1], key_at(p), d)] |
                 ((uint32_t)s.level[code_at(s.raw[1], key_at(p + 1), d)] << 16);
        }
        *reinterpret_cast<uint4*>(s.img + v_img_off(d, 4 * h + c)) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    __syncthreads();
    uint4* dst = reinterpret_cast<uint4*>(prefix_image(a, b, kvh, t));
    const uint4* src = reinterpret_cast<const uint4*>(s.img);
    for (int i = tid; i < kExtendTileBytes / 16; i += 256) dst[i] = src[i];
  } else {
    const int t = blockIdx.x - a.pt_max;
    if (t * kKeys >= n_b) return;
    uint8_t* img = chunk_image(a, b, kvh, t);
    {   // K image straight from the bf16 rows
      const int key = tid >> 2, q = tid & 3;
      const int kk = min(t * kKeys + key, n_b - 1);
      const uint4* src = reinterpret_cast<const uint4*>(a.k_new + ((size_t)(s0 + kk) * a.hkv + kvh) * kD + 32 * q);
#pragma unroll
      for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(img + k_img_off(key, 4 * q + c)) = src[c];
    }
    {   // V image: transpose through registers
      const int d = tid >> 1, h = tid & 1;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = 32 * h + 8 * c + 2 * e;
          const int k0 = min(t * kKeys + key_at(p), n_b - 1), k1 = min(t * kKeys + key_at(p + 1), n_b - 1);
          w[e] = (uint32_t)a.v_new[((size_t)(s0 + k0) * a.hkv + kvh) * kD + d] |
                 ((uint32_t)a.v_new[((size_t)(s0 + k1) * a.hkv + kvh) * kD + d] << 16);
        }
        *reinterpret_cast<uint4*>(img + v_img_off(d, 4 * h + c)) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

// ============================== attention ==============================
__device__ __forceinline__ void split_f16x8(const float x[8], f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const _Float16 h = (_Float16)x[e];
    hi[e] = h;
    lo[e] = (_Float16)(x[e] - (float)h);
  }
}

__device__ __forceinline__ void split_bf16x8(const float x[8], bf16x8& hi, bf16x8& lo) {
  uint32_t hb[8], lb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hb[e] = __float_as_uint(x[e]) & 0xffff0000u;                                   // truncated
    lb[e] = __float_as_uint(x[e] - __uint_as_float(hb[e])) & 0xffff0000u;          // exact remainder, truncated
  }
  uint4 h, l;
  h.x = __builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u); h.y = __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u);
  h.z = __builtin_amdgcn_perm(hb[5], hb[4], 0x07060302u); h.w = __builtin_amdgcn_perm(hb[7], hb[6], 0x07060302u);
  l.x = __builtin_amdgcn_perm(lb[1], lb[0], 0x07060302u); l.y = __builtin_amdgcn_perm(lb[3], lb[2], 0x07060302u);
  l.z = __builtin_amdgcn_perm(lb[5], lb[4], 0x07060302u); l.w = __builtin_amdgcn_perm(lb[7], lb[6], 0x07060302u);
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// Online-softmax update of one row from u (32 values per lane: key 16*s + 8*(e/4) + 4*h + e%4 of
// the tile at u[8*s + e], -inf where masked; the other 32 keys sit in lane l ^ 32) with true scores
// u * rs (rs > 0).  u becomes the weights.
__device__ __forceinline__ void softmax_step(float (&u)[32], float rs, float& m_run, float& l_run, f32x16 (&O)[4],
                                             int lane) {
  float mx = fmaxf(fmaxf(u[0], u[1]), u[2]);
#pragma unroll
  for (int i = 3; i < 31; i += 2) mx = fmaxf(fmaxf(mx, u[i]), u[i + 1]);
  mx = fmaxf(mx, u[31]);
  mx = fmaxf(mx, partner32(mx, lane)) * rs;
  const float m_new = fmaxf(m_run, mx);
  const float m_use = m_new == kNegInf ? 0.0f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  m_run = m_new;
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    u[i] = __builtin_amdgcn_exp2f(fmaf(u[i], rs, -m_use));
    sum += u[i];
  }
  l_run = l_run * alpha + sum;
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) O[t] *= alpha;
  }
}

// Scheduling groups (instruction classes of the AMDGPU scheduler): operand reads for the next MFMA
// step are issued ahead of the current step's MFMAs so that LDS latency hides behind them.
constexpr int kSchedMfma = 0x008, kSchedValu = 0x002, kSchedDsRead = 0x100;

template <typename V8, int NQ>
struct TileOps;
template <int NQ>
struct TileOps<f16x8, NQ> {
  static __device__ __forceinline__ f32x16 mma(const f16x8& a, const f16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <int NQ>
struct TileOps<bf16x8, NQ> {
  static __device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// S^T for the tile's 64 keys (two 32-key blocks) against this wave's 32 rows over the head_dim steps
// KS0 .. KS1 - 1 (16 values each); q is given as NQ parts (hi, lo) whose products accumulate.  Part
// LP of steps KL .. 7 comes from LDS (q_lds[(ks - KL) * 64], this lane's copy) instead of registers.
template <typename V8, int NQ, int KS0 = 0, int KS1 = 8, bool ACC = false, int KL = 8, int LP = NQ - 1>
__device__ __forceinline__ void qk_tile(const uint8_t* buf, int l32, int h, const V8 (&q)[NQ][8], f32x16 (&S)[2],
                                        const V8* q_lds = nullptr) {
  using Ops = TileOps<V8, NQ>;
  if constexpr (!ACC) {
    S[0] = f32x16{};
    S[1] = f32x16{};
  }
  // LDS operand reads run kQkDepth steps ahead of the MFMAs that use them, in a ring of kQkDepth + 1
  // register sets: the K rows of both 32-key blocks and, from step KL on, the LDS-held query part
  // (int8 prefix at C5's shapes: 1,798 -> 1,765 us against one step ahead with the query part read at
  // its MFMAs; ISO3 unchanged)
  constexpr int R = kQkDepth + 1;
  V8 ka[R][2], ql[R];
  auto issue = [&](int ks, int slot) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ka[slot][kb] = *reinterpret_cast<const V8*>(buf + k_img_off(32 * kb + l32, 2 * ks + h));
    if (ks >= KL) ql[slot] = q_lds[(ks - KL) * 64];
  };
#pragma unroll
  for (int d = 0; d < kQkDepth; ++d)
    if (KS0 + d < KS1) issue(KS0 + d, d);
#pragma unroll
  for (int ks = KS0; ks < KS1; ++ks) {
    const int slot = (ks - KS0) % R;
    if (ks + kQkDepth < KS1) issue(ks + kQkDepth, (ks - KS0 + kQkDepth) % R);
    // the later steps' operand reads are issued before this step's MFMAs (a real ring: the scheduler
    // would otherwise reuse one register set and wait for each read)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int part = 0; part < NQ; ++part) {
      const V8 qv = (part == LP && ks >= KL) ? ql[slot] : q[part][ks];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) S[kb] = Ops::mma(ka[slot][kb], qv, S[kb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T += V^T P^T for the tile: per 16-key step st, the weights' hi and lo parts (as MFMA B operands)
// against the 4 head_dim blocks of V; head_dim block t takes the weights P[t * NPG / 4] (NPG = 1: one
// set for all; NPG = 2: one set per 64-value group).
template <typename V8, int NPG = 1>
__device__ __forceinline__ void pv_tile(const uint8_t* buf, int l32, int h, const u32x4 (&P)[NPG][4][2],
                                        f32x16 (&O)[4]) {
  using Ops = TileOps<V8, 1>;
  V8 va[2][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) va[0][t] = *reinterpret_cast<const V8*>(buf + v_img_off(32 * t + l32, h));
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int cb = st & 1;
    if (st + 1 < 4) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        va[cb ^ 1][t] = *reinterpret_cast<const V8*>(buf + v_img_off(32 * t + l32, 2 * (st + 1) + h));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) O[t] = Ops::mma(va[cb][t], __builtin_bit_cast(V8, P[t * NPG / 4][st][0]), O[t]);
#pragma unroll
    for (int t = 0; t < 4; ++t) O[t] = Ops::mma(va[cb][t], __builtin_bit_cast(V8, P[t * NPG / 4][st][1]), O[t]);
    if (st + 1 < 4) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 1);
  }
}

// Prefix tiles: rotated basis, fp16 MFMAs, per-key norms.
struct PrefixTiles {
  using Weights = u32x4[1][4][2];
  static constexpr int kQLoLds = 4;      // lo parts of head_dim steps 4 .. 7 sit in LDS (16 fewer registers)
  const ExtendArgs& a;
  int b, kvh, P;
  const f16x8 (&q)[2][8];
  const f16x8* q_lds;                    // this lane's copies: [step - kQLoLds][64 lanes]
  float rs;
  __device__ __forceinline__ const uint8_t* image(int t) const { return prefix_image(a, b, kvh, t); }
  __device__ __forceinline__ bool active(int) const { return true; }
  __device__ __forceinline__ void qk(const uint8_t* buf, int l32, int h, f32x16 (&S)[2]) const {
    qk_tile<f16x8, 2, 0, 8, false, kQLoLds>(buf, l32, h, q, S, q_lds);
  }
  // scores / rs of tile t into u (masked past the prefix), returns rs
  __device__ __forceinline__ float scores(const uint8_t* buf, int t, int h, const f32x16 (&S)[2], float (&u)[32]) const {
    const float* nk = reinterpret_cast<const float*>(buf + kNormOff);
    const int limit = P - t * kKeys;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const int key = 16 * (i >> 3) + 8 * ((i >> 2) & 1) + 4 * h;   // keys key .. key+3
      const float4 n4 = *reinterpret_cast<const float4*>(nk + key);
      const float nn[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) u[i + j] = S[i >> 4][(i & 15) + j] * nn[j];
    }
    if (limit < kKeys) {                                     // the prefix ends inside this tile
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (16 * (i >> 3) + 8 * ((i >> 2) & 1) + 4 * h + (i & 3) >= limit) u[i] = kNegInf;
    }
    return rs;
  }
  __device__ __forceinline__ void weights(const uint8_t* buf, int h, const float (&u)[32], Weights& Pw) const {
    const float* nv = reinterpret_cast<const float*>(buf + kNormOff) + kKeys;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      float x[8];
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) {
        const float4 n4 = *reinterpret_cast<const float4*>(nv + 16 * st + 8 * e4 + 4 * h);
        x[4 * e4 + 0] = u[8 * st + 4 * e4 + 0] * n4.x;
        x[4 * e4 + 1] = u[8 * st + 4 * e4 + 1] * n4.y;
        x[4 * e4 + 2] = u[8 * st + 4 * e4 + 2] * n4.z;
        x[4 * e4 + 3] = u[8 * st + 4 * e4 + 3] * n4.w;
      }
      f16x8 ph, pl;
      split_f16x8(x, ph, pl);
      Pw[0][st][0] = __builtin_bit_cast(u32x4, ph);
      Pw[0][st][1] = __builtin_bit_cast(u32x4, pl);
    }
  }
  __device__ __forceinline__ void pv(const uint8_t* buf, int l32, int h, const Weights& Pw, f32x16 (&O)[4]) const {
    pv_tile<f16x8>(buf, l32, h, Pw, O);
  }
};

// INT8_G64 prefix tiles: exact fp16 codes, one partial sum per 64-value group weighted by the key's
// group scale (QK), and per group the weights times the key's V group scale (PV); no rotation.
struct PrefixTilesI8 {
  using Weights = u32x4[2][4][2];
  static constexpr int kQLds = 4;        // the query's head_dim steps 4 .. 7 sit in LDS (16 fewer registers)
  const ExtendArgs& a;
  int b, kvh, P;
  const f16x8 (&q)[2][8];
  const f16x8* q_lds;                    // this lane's copies: [step - kQLds][64 lanes]
  float rs;
  __device__ __forceinline__ const uint8_t* image(int t) const { return prefix_image(a, b, kvh, t); }
  __device__ __forceinline__ bool active(int) const { return true; }
  // The query is bf16 and unscaled, so its fp16 image (times a power of two) is exact in one part.
  // Per key, S = s0 * S0 + s1 * S1 (S_g: the partial over group g) is formed as (S0 * s0 / s1 + S1) * s1
  // in one accumulator (as S0 * s0 when s1 = 0: that group's codes are all zero), with both factors
  // from the stage.
  __device__ __forceinline__ void qk(const uint8_t* buf, int l32, int h, f32x16 (&S)[2]) const {
    const f16x8 (&qh)[1][8] = reinterpret_cast<const f16x8 (&)[1][8]>(q[0]);
    const float* sk = reinterpret_cast<const float*>(buf + kNormOff);
    qk_tile<f16x8, 1, 0, 4>(buf, l32, h, qh, S);             // head_dim 0 .. 63
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const int key = 16 * (i >> 3) + 8 * ((i >> 2) & 1) + 4 * h;   // keys key .. key+3
      const float4 s0 = *reinterpret_cast<const float4*>(sk + key);
      const float4 s1 = *reinterpret_cast<const float4*>(sk + kKeys + key);
      const float a0[4] = {s0.x, s0.y, s0.z, s0.w}, a1[4] = {s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i >> 4][(i & 15) + j] *= a0[j];
    }
    qk_tile<f16x8, 1, 4, 8, true, kQLds, 0>(buf, l32, h, qh, S, q_lds);   // head_dim 64 .. 127, accumulated
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const int key = 16 * (i >> 3) + 8 * ((i >> 2) & 1) + 4 * h;
      const float4 s1 = *reinterpret_cast<const float4*>(sk + kKeys + key);
      const float a1[4] = {s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i >> 4][(i & 15) + j] *= a1[j];
    }
  }
  __device__ __forceinline__ float scores(const uint8_t*, int t, int h, const f32x16 (&S)[2], float (&u)[32]) const {
    const int limit = P - t * kKeys;
#pragma unroll
    for (int i = 0; i < 32; ++i) u[i] = S[i >> 4][i & 15];
    if (limit < kKeys) {                                     // the prefix ends inside this tile
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (16 * (i >> 3) + 8 * ((i >> 2) & 1) + 4 * h + (i & 3) >= limit) u[i] = kNegInf;
    }
    return rs * a.scale_log2;                                // the query entered unscaled
  }
  __device__ __forceinline__ void weights(const uint8_t* buf, int h, const float (&u)[32], Weights& Pw) const {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float* nv = reinterpret_cast<const float*>(buf + kNormOff) + (2 + g) * kKeys;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float x[8];
#pragma unroll
        for (int e4 = 0; e4 < 2; ++e4) {
          const float4 n4 = *reinterpret_cast<const float4*>(nv + 16 * st + 8 * e4 + 4 * h);
          x[4 * e4 + 0] = u[8 * st + 4 * e4 + 0] * n4.x;
          x[4 * e4 + 1] = u[8 * st + 4 * e4 + 1] * n4.y;
          x[4 * e4 + 2] = u[8 * st + 4 * e4 + 2] * n4.z;
          x[4 * e4 + 3] = u[8 * st + 4 * e4 + 3] * n4.w;
        }
        f16x8 ph, pl;
        split_f16x8(x, ph, pl);
        Pw[g][st][0] = __builtin_bit_cast(u32x4, ph);
        Pw[g][st][1] = __builtin_bit_cast(u32x4, pl);
      }
    }
  }
  __device__ __forceinline__ void pv(const uint8_t* buf, int l32, int h, const Weights& Pw, f32x16 (&O)[4]) const {
    pv_tile<f16x8, 2>(buf, l32, h, Pw, O);
  }
};

// Chunk tiles: original basis, bf16 MFMAs, causal mask; tiles past a wave's last token are skipped.
struct ChunkTiles {
  using Weights = u32x4[1][4][2];
  const ExtendArgs& a;
  int b, kvh, tok, wave_first, wave_last;
  const bf16x8 (&q)[1][8];
  __device__ __forceinline__ const uint8_t* image(int t) const { return chunk_image(a, b, kvh, t); }
  __device__ __forceinline__ bool active(int t) const { return t * kKeys <= wave_last; }
  __device__ __forceinline__ void qk(const uint8_t* buf, int l32, int h, f32x16 (&S)[2]) const {
    qk_tile<bf16x8, 1>(buf, l32, h, q, S);
  }
  __device__ __forceinline__ float scores(const uint8_t*, int t, int h, const f32x16 (&S)[2], float (&u)[32]) const {
#pragma unroll
    for (int i = 0; i < 32; ++i) u[i] = S[i >> 4][i & 15];
    if ((t + 1) * kKeys > wave_first) {                      // the tile reaches this wave's diagonal
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (t * kKeys + 16 * (i >> 3) + 8 * ((i >> 2) & 1) + 4 * h + (i & 3) > tok) u[i] = kNegInf;
    }
    return a.scale_log2;
  }
  __device__ __forceinline__ void weights(const uint8_t*, int, const float (&u)[32], Weights& Pw) const {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 ph, pl;
      split_bf16x8(u + 8 * st, ph, pl);
      Pw[0][st][0] = __builtin_bit_cast(u32x4, ph);
      Pw[0][st][1] = __builtin_bit_cast(u32x4, pl);
    }
  }
  __device__ __forceinline__ void pv(const uint8_t* buf, int l32, int h, const Weights& Pw, f32x16 (&O)[4]) const {
    pv_tile<bf16x8>(buf, l32, h, Pw, O);
  }
};

// A tile image into LDS: 36 one-kilobyte direct loads shared by the 8 waves.
__device__ __forceinline__ void issue_tile(const uint8_t* src, uint8_t* dst, int wv, int lane) {
  for (int i = wv; i < kExtendTileBytes / 1024; i += kWaves) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + i * 1024 + lane * 16),
                                     (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
  }
}

// Register values that must exist at this point of the instruction stream.
template <int NPG>
__device__ __forceinline__ void pin(u32x4 (&P)[NPG][4][2], f32x16 (&O)[4]) {
#pragma unroll
  for (int g = 0; g < NPG; ++g)
#pragma unroll
    for (int st = 0; st < 4; ++st) asm volatile("" : "+v"(P[g][st][0]), "+v"(P[g][st][1]));
  asm volatile("" : "+v"(O[0]), "+v"(O[1]), "+v"(O[2]), "+v"(O[3]));
}
__device__ __forceinline__ void pin(f32x16 (&S)[2], f32x16 (&O)[4]) {
  asm volatile("" : "+v"(S[0]), "+v"(S[1]));
  asm volatile("" : "+v"(O[0]), "+v"(O[1]), "+v"(O[2]), "+v"(O[3]));
}

// Barrier; with `loads` it first waits until this wave's direct-to-LDS tile loads have landed.
__device__ __forceinline__ void sync_tiles(bool loads) {
  if (loads) __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
  __syncthreads();
}

// Ping-pong over n tiles.  The two 4-wave groups alternate between an MFMA cluster (PV of tile
// it, QK of tile it+1) and a VALU cluster (softmax of tile it's scores, the weights' split); group
// B runs one barrier phase behind group A, so one group's MFMAs overlap the other's softmax.
// Tiles live in a ring of three LDS buffers; tile it+2 is loaded during barrier phase 2*it+1 (by
// group A in its MFMA cluster, group B in its VALU cluster), after the last read of tile it-1
// (group B's PV in phase 2*it); each wave waits for its loads at the end of the following phase,
// before the tile's first read in phase 2*it+3.
template <typename Tiles>
__device__ __forceinline__ void run_tiles(const Tiles& k, int n, uint8_t* ring, bool group_b, int wv, int lane, int l32,
                                          int h, float& m_run, float& l_run, f32x16 (&O)[4]) {
  if (n <= 0) return;
  auto buf = [&](int t) { return ring + (t % 3) * kExtendTileBytes; };
  issue_tile(k.image(0), buf(0), wv, lane);
  if (n > 1) issue_tile(k.image(1), buf(1), wv, lane);
  sync_tiles(true);
  if (group_b) sync_tiles(false);
  f32x16 S[2];
  if (k.active(0)) k.qk(buf(0), l32, h, S);
  sync_tiles(false);
  typename Tiles::Weights Pw;
  for (int it = 0; it < n; ++it) {
    // ---- VALU cluster: softmax of tile it
    if (group_b && it + 2 < n) issue_tile(k.image(it + 2), buf(it + 2), wv, lane);
    const bool act = k.active(it);
    if (act) {
      float u[32];
      const float rs = k.scores(buf(it), it, h, S, u);
      softmax_step(u, rs, m_run, l_run, O, lane);
      k.weights(buf(it), h, u, Pw);
    }
    // keep each cluster's work on its side of the barrier (the compiler would otherwise sink the
    // weights and the rescale into the MFMA cluster, next to their uses)
    pin(Pw, O);
    sync_tiles(!group_b);            // group A: tile it+1's loads, issued one phase ago, have landed
    // ---- MFMA cluster: PV of tile it, then QK of tile it+1 (in this order the weights are dead
    // before the scores are born, which leaves registers for operand double buffering); group A
    // issues tile it+2's loads after them, so that no wait on the vector memory counter inside the
    // cluster (a register reload) waits for the tile
    if (act) k.pv(buf(it), l32, h, Pw, O);
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < n && k.active(it + 1)) k.qk(buf(it + 1), l32, h, S);
    pin(S, O);
    __builtin_amdgcn_sched_barrier(0);
    if (!group_b && it + 2 < n) issue_tile(k.image(it + 2), buf(it + 2), wv, lane);
    sync_tiles(group_b);             // group B: tile it+2's loads, issued one phase ago, have landed
  }
  if (!group_b) sync_tiles(true);
}

template <bool I8>
__global__ __launch_bounds__(kWaves * 64, 1) void k_extend_attn(const ExtendArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[3 * kExtendTileBytes];
  // each wave's query parts of the last head_dim steps, read by the prefix QK from LDS: ISO3 the lo
  // parts of the rotated query, int8 the (single) query part
  static_assert(PrefixTiles::kQLoLds == PrefixTilesI8::kQLds, "one LDS region for both prefix formats");
  __shared__ __attribute__((aligned(16))) f16x8 q_lo[kWaves][8 - PrefixTiles::kQLoLds][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_b = wv >= kWaves / 2;
  const int l32 = lane & 31, h = lane >> 5;
  const int kvh = blockIdx.x % a.hkv, tile = blockIdx.x / a.hkv, b = blockIdx.y;

  const int s0 = clampi(a.cu_new[b], 0, a.n_new);
  const int n_b = clampi(a.cu_new[b + 1], s0, a.n_new) - s0;
  const int tw = 32 / a.g_pad;                              // tokens per wave
  const int tok0 = tile * kWaves * tw;                      // first token of the workgroup
  if (tok0 >= n_b) return;
  const int P = clampi(a.prefix_lens[b], 0, a.max_pages * KVQ_PAGE_SIZE);

  int G, h0;
  if (a.g_uniform > 0) { G = a.g_uniform; h0 = kvh * G; }
  else { h0 = a.head_off[kvh]; G = a.head_off[kvh + 1] - h0; }

  // ---- this lane's row: (token tw*wv + l32 / g_pad, head slot l32 % g_pad)
  const int tok = tok0 + wv * tw + l32 / a.g_pad;
  const int hs = l32 % a.g_pad;
  const bool valid = tok < n_b && hs < G;
  const int qrow = valid ? (s0 + tok) * a.n_q_heads + (a.g_uniform > 0 ? h0 + hs : a.head_list[h0 + hs]) : 0;
  const uint16_t* qp = a.q + (size_t)qrow * kD + 8 * h;     // head_dim 16*ks + 8*h .. +7 for ks = 0..7

  f32x16 O[4] = {};
  float m_run = kNegInf, l_run = 0.0f;

  // ================= prefix phase (rotated basis, fp16 MFMA) =================
  const int n_pt = (P + kKeys - 1) / kKeys;
  if (n_pt > 0) {
    const float rw = a.quat[0], rx = a.quat[1], ry = a.quat[2], rz = a.quat[3];
    // rotated, scaled query as fp16 hi + lo
    f16x8 qs[2][8];                                         // [hi, lo][ks]
    float rs;
    {
      float v[8][8];
      float mx = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint4 raw = *reinterpret_cast<const uint4*>(qp + 16 * ks);
        if (!valid) raw = make_uint4(0, 0, 0, 0);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
          const float u[4] = {bf16f(w[2 * grp] & 0xffffu), bf16f(w[2 * grp] >> 16), bf16f(w[2 * grp + 1] & 0xffffu),
                              bf16f(w[2 * grp + 1] >> 16)};
          float t[4];
          if constexpr (I8) {                               // int8 prefix: original basis
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = u[e];
          } else {
            qmul(rw, rx, ry, rz, u, t);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[ks][4 * grp + e] = t[e] * a.q_scale;
            mx = fmaxf(mx, fabsf(v[ks][4 * grp + e]));
          }
        }
      }
      mx = fmaxf(mx, partner32(mx, lane));
      int ex = 0;
      if (mx > 0.0f) { frexpf(mx, &ex); ex = 14 - ex; }      // max * 2^ex in [2^13, 2^14)
      rs = ldexpf(1.0f, -ex);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = ldexpf(v[ks][e], ex);
        split_f16x8(x, qs[0][ks], qs[1][ks]);
      }
    }
    if constexpr (I8) {
#pragma unroll
      for (int k = PrefixTilesI8::kQLds; k < 8; ++k) q_lo[wv][k - PrefixTilesI8::kQLds][lane] = qs[0][k];
      const PrefixTilesI8 pk{a, b, kvh, P, qs, &q_lo[wv][0][lane], rs};
      run_tiles(pk, n_pt, ring, group_b, wv, lane, l32, h, m_run, l_run, O);
    } else {
#pragma unroll
      for (int k = PrefixTiles::kQLoLds; k < 8; ++k) q_lo[wv][k - PrefixTiles::kQLoLds][lane] = qs[1][k];
      const PrefixTiles pk{a, b, kvh, P, qs, &q_lo[wv][0][lane], rs};
      run_tiles(pk, n_pt, ring, group_b, wv, lane, l32, h, m_run, l_run, O);
    }
    // back to the original basis: O[t][4g .. 4g+3] is head_dim 32t + 8g + 4h .. +3, one group
#pragma unroll
    for (int t = 0; t < 4 && !I8; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float u[4] = {O[t][4 * g], O[t][4 * g + 1], O[t][4 * g + 2], O[t][4 * g + 3]};
        float r[4];
        qmul(rw, -rx, -ry, -rz, u, r);
#pragma unroll
        for (int e = 0; e < 4; ++e) O[t][4 * g + e] = r[e];
      }
  }

  // ================= chunk phase (original basis, bf16 MFMA) =================
  {
    const int kmax = min(n_b, tok0 + kWaves * tw);          // new keys any row of the workgroup sees
    const int n_nt = (kmax + kKeys - 1) / kKeys;
    bf16x8 qb[1][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 raw = *reinterpret_cast<const uint4*>(qp + 16 * ks);
      if (!valid) raw = make_uint4(0, 0, 0, 0);
      qb[0][ks] = __builtin_bit_cast(bf16x8, raw);
    }
    const ChunkTiles ck{a, b, kvh, tok, tok0 + wv * tw, tok0 + wv * tw + tw - 1, qb};
    run_tiles(ck, n_nt, ring, group_b, wv, lane, l32, h, m_run, l_run, O);
  }

  // ---- normalise and write: lanes l and l ^ 32 hold the two halves of a row's sum
  const float l = l_run + partner32(l_run, lane);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (valid) {
    float* o = a.out + (size_t)qrow * kD + 4 * h;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(o + 32 * t + 8 * g) =
            make_float4(O[t][4 * g] * inv, O[t][4 * g + 1] * inv, O[t][4 * g + 2] * inv, O[t][4 * g + 3] * inv);
  }
}

}  // namespace

float extend_level_scale() { return kIsoLevelScale; }

hipError_t launch_extend(const ExtendArgs& a, int tiles_per_seq, hipStream_t s) {
  k_extend_stage<<<dim3((unsigned)(a.pt_max + a.nt_max), (unsigned)a.hkv, (unsigned)a.batch), dim3(256), 0, s>>>(a);
  if (a.int8)
    k_extend_attn<true><<<dim3((unsigned)(a.hkv * tiles_per_seq), (unsigned)a.batch), dim3(kWaves * 64), 0, s>>>(a);
  else
    k_extend_attn<false><<<dim3((unsigned)(a.hkv * tiles_per_seq), (unsigned)a.batch), dim3(kWaves * 64), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
