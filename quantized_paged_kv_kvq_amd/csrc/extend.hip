// Extend (prefill chunk) attention over an ISO3-packed prefix plus the chunk's own bf16 tokens.
//
// FreeToken PR #398, "What": a prefill chunk attends the cached prefix, which is held packed,
// and its own new tokens, which are packed only after the chunk's attention (deferred packing).
// Token i of a chunk at position P + i sees the P prefix cells and new tokens 0..i.
//
// Work decomposition: one workgroup = 4 waves = one (sequence, KV head, 4 * T query tokens) tile;
// a wave owns 32 query rows (T tokens x G_pad query heads of the KV head) as two 16-column MFMA
// tiles.  Keys stream through LDS 64 at a time, double-buffered, one barrier per tile.
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
// New-token phase (original basis, bf16 MFMA).  q and the new K/V are bf16 and enter the bf16 MFMA
// exactly; the weights are split into bf16 hi + lo parts (16 significant bits).  Causal mask per
// row; tiles past a wave's last token are skipped.
//
// Online softmax in base 2 per row across both phases; the row max is shared by the 4 lanes that
// hold a row's keys, the running sums stay per lane until the end.
#include "kvq_internal.h"
#include "device_util.h"

namespace kvq {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kKeys = 64;                 // keys per tile
constexpr int kKStride = kD + 8;          // halves per key row of the K tile (272 B)
constexpr int kVStride = kKeys + 8;       // halves per head_dim row of the V tile (144 B)
constexpr int kLutEntries = 4096;         // every 12-bit group of 4 codes
constexpr float kLevelScale = 1.2495174407958984f;   // S: S * c is within 2^-15.9 of fp16 for all 8 levels

constexpr double kSqrt128 = 11.3137084989847603904135327140;
__constant__ float kLevels[8] = {
    (float)(-2.1520 / kSqrt128), (float)(-1.3440 / kSqrt128), (float)(-0.7560 / kSqrt128),
    (float)(-0.2451 / kSqrt128), (float)(0.2451 / kSqrt128),  (float)(0.7560 / kSqrt128),
    (float)(1.3440 / kSqrt128),  (float)(2.1520 / kSqrt128)};

// r (x) u for a quaternion r = (w, x, y, z) and a group u = (u0, u1, u2, u3).
__device__ __forceinline__ void qmul(float w, float x, float y, float z, const float u[4], float t[4]) {
  t[0] = ((w * u[0] - x * u[1]) - y * u[2]) - z * u[3];
  t[1] = ((w * u[1] + x * u[0]) + y * u[3]) - z * u[2];
  t[2] = ((w * u[2] - x * u[3]) + y * u[0]) + z * u[1];
  t[3] = ((w * u[3] + x * u[2]) - y * u[1]) + z * u[0];
}

// Position of key k of a tile in the V tile rows: inside each 32-key half, the 4 keys of lane
// group g from the first 16 and the 4 from the second 16 sit side by side, so that one 16-byte LDS
// read gives a PV A-operand lane the same 8 keys its B operand holds.
__device__ __forceinline__ int vpos(int k) {
  const int k32 = k & 31;
  return (k & 32) + ((k32 & 15) >> 2) * 8 + (k32 >> 4) * 4 + (k & 3);
}

struct Lds {
  uint2 lut[kLutEntries];                               // 4 codes -> 4 fp16 values S * c
  uint16_t k[2][kKeys * kKStride];                      // [key][d]
  uint16_t v[2][kD * kVStride];                         // [d][vpos(key)]
  float nk[2][kKeys];                                   // K norms
  float nv[2][kKeys];                                   // V norms / S
};

// ---- tile loaders.  Waves 0-1 handle K (thread: one key, 64 head_dim values), waves 2-3 handle V
// (thread: two adjacent keys, 32 head_dim values), so every role is wave-uniform.
struct IsoRegs {
  uint32_t c[6];     // K: 64 codes of one key; V: 32 codes of each of two keys
  uint32_t norm;     // K: norm (low half); V: norms of the two keys
};

__device__ __forceinline__ int iso_page_index(int it, int tid) {
  const int key = tid < 128 ? (tid >> 1) : 2 * (tid & 31);
  return (it * kKeys + key) >> 4;
}

__device__ __forceinline__ void iso_load(const ExtendArgs& a, int it, int page, int kvh, int tid, IsoRegs& r) {
  const size_t tile = (size_t)page * a.hkv + kvh;
  if (tid < 128) {
    const int key = tid >> 1, half = tid & 1;
    const int slot = (it * kKeys + key) & 15;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.k_codes + (tile * 16 + slot) * 48 + 24 * half);
#pragma unroll
    for (int i = 0; i < 6; ++i) r.c[i] = src[i];
    r.norm = half == 0 ? a.k_norms[tile * 16 + slot] : 0u;
  } else {
    const int m = tid & 31, chunk = (tid - 128) >> 5;
    const int slot = (it * kKeys + 2 * m) & 15;
    const uint32_t* src0 = reinterpret_cast<const uint32_t*>(a.v_codes + (tile * 16 + slot) * 48 + 12 * chunk);
    const uint32_t* src1 = src0 + 12;                   // next slot: 48 bytes further
#pragma unroll
    for (int i = 0; i < 3; ++i) { r.c[i] = src0[i]; r.c[3 + i] = src1[i]; }
    r.norm = chunk == 0 ? *reinterpret_cast<const uint32_t*>(a.v_norms + tile * 16 + slot) : 0u;
  }
}

// 12-bit group g (0..7) of a 96-bit little-endian code stream held in three words.
__device__ __forceinline__ uint32_t group12(const uint32_t* w, int g) {
  const int bit = 12 * g, wi = bit >> 5, sh = bit & 31;
  const uint64_t two = (uint64_t)w[wi] | ((uint64_t)(wi + 1 < 3 ? w[wi + 1] : 0u) << 32);
  return (uint32_t)(two >> sh) & 0xfffu;
}

__device__ __forceinline__ void iso_store(Lds& s, int buf, int tid, const IsoRegs& r) {
  if (tid < 128) {
    const int key = tid >> 1, half = tid & 1;
    uint32_t h[32];                                     // 64 fp16 values, two per word
#pragma unroll
    for (int part = 0; part < 2; ++part)
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const uint2 e = s.lut[group12(r.c + 3 * part, g)];
        h[part * 16 + 2 * g] = e.x;
        h[part * 16 + 2 * g + 1] = e.y;
      }
    uint4* dst = reinterpret_cast<uint4*>(&s.k[buf][key * kKStride + 64 * half]);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = make_uint4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);
    if (half == 0) s.nk[buf][key] = h2f((uint16_t)(r.norm & 0xffffu));
  } else {
    const int m = tid & 31, chunk = (tid - 128) >> 5;
    uint32_t h0[16], h1[16];                            // 32 fp16 values of each key
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint2 e0 = s.lut[group12(r.c, g)];
      const uint2 e1 = s.lut[group12(r.c + 3, g)];
      h0[2 * g] = e0.x; h0[2 * g + 1] = e0.y;
      h1[2 * g] = e1.x; h1[2 * g + 1] = e1.y;
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(&s.v[buf][(32 * chunk) * kVStride + vpos(2 * m)]);
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;   // high or low halves of both keys
      dst[d * (kVStride / 2)] = __builtin_amdgcn_perm(h1[d >> 1], h0[d >> 1], sel);
    }
    if (chunk == 0) {
      s.nv[buf][2 * m] = h2f((uint16_t)(r.norm & 0xffffu)) / kLevelScale;
      s.nv[buf][2 * m + 1] = h2f((uint16_t)(r.norm >> 16)) / kLevelScale;
    }
  }
}

// ---- new-token tiles: bf16 K/V of the chunk, same roles and LDS layout.
struct NewRegs {
  uint4 c[8];        // K: 64 values of one key; V: 32 values of each of two keys
};

__device__ __forceinline__ void new_load(const ExtendArgs& a, int s0, int kmax, int nt, int kvh, int tid, NewRegs& r) {
  if (tid < 128) {
    const int key = min(nt * kKeys + (tid >> 1), kmax - 1), half = tid & 1;
    const uint4* src = reinterpret_cast<const uint4*>(a.k_new + ((size_t)(s0 + key) * a.hkv + kvh) * kD + 64 * half);
#pragma unroll
    for (int i = 0; i < 8; ++i) r.c[i] = src[i];
  } else {
    const int m = tid & 31, chunk = (tid - 128) >> 5;
    const int k0 = min(nt * kKeys + 2 * m, kmax - 1), k1 = min(nt * kKeys + 2 * m + 1, kmax - 1);
    const uint4* src0 = reinterpret_cast<const uint4*>(a.v_new + ((size_t)(s0 + k0) * a.hkv + kvh) * kD + 32 * chunk);
    const uint4* src1 = reinterpret_cast<const uint4*>(a.v_new + ((size_t)(s0 + k1) * a.hkv + kvh) * kD + 32 * chunk);
#pragma unroll
    for (int i = 0; i < 4; ++i) { r.c[i] = src0[i]; r.c[4 + i] = src1[i]; }
  }
}

__device__ __forceinline__ uint32_t word_of4(const uint4* q, int w) {
  const uint4 t = q[w >> 2];
  const int k = w & 3;
  return k == 0 ? t.x : k == 1 ? t.y : k == 2 ? t.z : t.w;
}

__device__ __forceinline__ void new_store(Lds& s, int buf, int tid, const NewRegs& r) {
  if (tid < 128) {
    const int key = tid >> 1, half = tid & 1;
    uint4* dst = reinterpret_cast<uint4*>(&s.k[buf][key * kKStride + 64 * half]);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = r.c[i];
  } else {
    const int m = tid & 31, chunk = (tid - 128) >> 5;
    uint32_t* dst = reinterpret_cast<uint32_t*>(&s.v[buf][(32 * chunk) * kVStride + vpos(2 * m)]);
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
      dst[d * (kVStride / 2)] = __builtin_amdgcn_perm(word_of4(r.c + 4, d >> 1), word_of4(r.c, d >> 1), sel);
    }
  }
}

// ---- hi/lo splits of 8 weights into MFMA B operands
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

// Online-softmax update of one 16-column tile from its 16 scores per lane (key kb*16 + 4*g4 + j
// at s[4*kb + j], -inf where masked); returns the weights in p.
__device__ __forceinline__ void softmax_step(float (&s)[16], float& m_run, float& l_run, f32x4 (&O)[8]) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
  mx = max_over_row_lanes(mx);
  const float m_new = fmaxf(m_run, mx);
  const float m_use = m_new == kNegInf ? 0.0f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  m_run = m_new;
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
    sum += s[i];
  }
  l_run = l_run * alpha + sum;
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int t = 0; t < 8; ++t) O[t] *= alpha;
  }
}

__global__ __launch_bounds__(256, 1) void k_extend_iso3(const ExtendArgs a) {
  __shared__ __attribute__((aligned(16))) Lds s;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int kvh = blockIdx.x % a.hkv, tile = blockIdx.x / a.hkv, b = blockIdx.y;

  const int s0 = clampi(a.cu_new[b], 0, a.n_new);
  const int n_b = clampi(a.cu_new[b + 1], s0, a.n_new) - s0;
  const int tw = 32 / a.g_pad;                              // tokens per wave
  const int tok0 = tile * kWaves * tw;                      // first token of the workgroup
  if (tok0 >= n_b) return;
  const int cap = a.max_pages * KVQ_PAGE_SIZE;
  const int P = clampi(a.prefix_lens[b], 0, cap);
  const int* bt_row = a.bt + (size_t)b * a.max_pages;

  int G, h0;
  if (a.g_uniform > 0) { G = a.g_uniform; h0 = kvh * G; }
  else { h0 = a.head_off[kvh]; G = a.head_off[kvh + 1] - h0; }

  // ---- rows: row 16*rb + c16 of this wave = (token tw*wv + r / g_pad, head slot r % g_pad)
  int tok[2], qrow[2];
  bool valid[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 16 * rb + c16;
    tok[rb] = tok0 + wv * tw + r / a.g_pad;
    const int hs = r % a.g_pad;
    valid[rb] = tok[rb] < n_b && hs < G;
    const int hq = valid[rb] ? (a.g_uniform > 0 ? h0 + hs : a.head_list[h0 + hs]) : 0;
    qrow[rb] = valid[rb] ? (s0 + tok[rb]) * a.n_q_heads + hq : 0;
  }

  f32x4 O[2][8];
#pragma unroll
  for (int t = 0; t < 8; ++t) O[0][t] = O[1][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.0f, 0.0f};

  // ================= prefix phase (rotated basis, fp16 MFMA) =================
  const int n_pt = (P + kKeys - 1) / kKeys;
  if (n_pt > 0) {
    const float rw = a.quat[0], rx = a.quat[1], ry = a.quat[2], rz = a.quat[3];
    // LUT of 4-code groups: S * c rounded to fp16
    for (int e = tid; e < kLutEntries; e += 256) {
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        h[i] = __builtin_bit_cast(uint16_t, (_Float16)(kLevelScale * kLevels[(e >> (3 * i)) & 7]));
      s.lut[e] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
    IsoRegs regs;
    int pg_next = clampi(bt_row[min(iso_page_index(0, tid), a.max_pages - 1)], 0, a.num_pages - 1);
    iso_load(a, 0, pg_next, kvh, tid, regs);
    if (n_pt > 1) pg_next = clampi(bt_row[min(iso_page_index(1, tid), a.max_pages - 1)], 0, a.num_pages - 1);

    // rotated, scaled query as fp16 hi + lo: lane holds head_dim 32*ks + 8*g4 .. +7 of its rows
    f16x8 qh[2][4], ql[2][4];
    float rowscale[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float v[4][8];
      float mx = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        uint4 raw = *reinterpret_cast<const uint4*>(a.q + (size_t)qrow[rb] * kD + 32 * ks + 8 * g4);
        if (!valid[rb]) raw = make_uint4(0, 0, 0, 0);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
          const float u[4] = {bf16f(w[2 * grp] & 0xffffu), bf16f(w[2 * grp] >> 16), bf16f(w[2 * grp + 1] & 0xffffu),
                              bf16f(w[2 * grp + 1] >> 16)};
          float t[4];
          qmul(rw, rx, ry, rz, u, t);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[ks][4 * grp + e] = t[e] * a.q_scale;
            mx = fmaxf(mx, fabsf(v[ks][4 * grp + e]));
          }
        }
      }
      mx = max_over_row_lanes(mx);
      int ex = 0;
      if (mx > 0.0f) { frexpf(mx, &ex); ex = 14 - ex; }      // max * 2^ex in [2^13, 2^14)
      rowscale[rb] = ldexpf(1.0f, -ex);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = ldexpf(v[ks][e], ex);
        split_f16x8(x, qh[rb][ks], ql[rb][ks]);
      }
    }

    __syncthreads();                                        // LUT ready
    iso_store(s, 0, tid, regs);
    __syncthreads();

    for (int it = 0; it < n_pt; ++it) {
      const int buf = it & 1;
      const bool more = it + 1 < n_pt;
      if (more) {
        iso_load(a, it + 1, pg_next, kvh, tid, regs);
        if (it + 2 < n_pt)
          pg_next = clampi(bt_row[min(iso_page_index(it + 2, tid), a.max_pages - 1)], 0, a.num_pages - 1);
      }
      const int limit = P - it * kKeys;                     // keys of this tile inside the prefix

      // QK: S^T[key][row]; A = K tile (16 keys x 32 head_dim), B = q hi, then q lo
      f32x4 S[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) S[kb][0] = S[kb][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f16x8 ka = __builtin_bit_cast(
              f16x8, *reinterpret_cast<const uint4*>(&s.k[buf][(16 * kb + c16) * kKStride + 32 * ks + 8 * g4]));
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            S[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qh[rb][ks], S[kb][rb], 0, 0, 0);
            S[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, ql[rb][ks], S[kb][rb], 0, 0, 0);
          }
        }
      float nk[16], nv[16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float4 a4 = *reinterpret_cast<const float4*>(&s.nk[buf][16 * kb + 4 * g4]);
        const float4 b4 = *reinterpret_cast<const float4*>(&s.nv[buf][16 * kb + 4 * g4]);
        nk[4 * kb] = a4.x; nk[4 * kb + 1] = a4.y; nk[4 * kb + 2] = a4.z; nk[4 * kb + 3] = a4.w;
        nv[4 * kb] = b4.x; nv[4 * kb + 1] = b4.y; nv[4 * kb + 2] = b4.z; nv[4 * kb + 3] = b4.w;
      }
      f16x8 ph[2][2], pl[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 16 * (i >> 2) + 4 * g4 + (i & 3);
          p[i] = key < limit ? S[i >> 2][rb][i & 3] * nk[i] * rowscale[rb] : kNegInf;
        }
        softmax_step(p, m_run[rb], l_run[rb], O[rb]);
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = 8 * ks2 + e;                      // key block 2*ks2 + e/4, slot e%4
            const int key = 16 * (i >> 2) + 4 * g4 + (i & 3);
            x[e] = key < limit ? p[i] * nv[i] : 0.0f;
          }
          split_f16x8(x, ph[rb][ks2], pl[rb][ks2]);
        }
      }
      // PV: O^T[d][row] in the rotated basis; A = V tile (16 head_dim x 32 keys)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const f16x8 va = __builtin_bit_cast(
              f16x8, *reinterpret_cast<const uint4*>(&s.v[buf][(16 * t + c16) * kVStride + 32 * ks2 + 8 * g4]));
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            O[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph[rb][ks2], O[rb][t], 0, 0, 0);
            O[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pl[rb][ks2], O[rb][t], 0, 0, 0);
          }
        }
      if (more) iso_store(s, buf ^ 1, tid, regs);
      __syncthreads();
    }
    // back to the original basis: lane's 4 values of O[rb][t] are head_dim 16t + 4*g4 .. +3, one group
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float u[4] = {O[rb][t][0], O[rb][t][1], O[rb][t][2], O[rb][t][3]};
        float r[4];
        qmul(rw, -rx, -ry, -rz, u, r);
        O[rb][t] = f32x4{r[0], r[1], r[2], r[3]};
      }
  }

  // ================= new-token phase (original basis, bf16 MFMA) =================
  const int kmax = min(n_b, tok0 + kWaves * tw);            // new keys any row of the workgroup sees
  const int n_nt = (kmax + kKeys - 1) / kKeys;
  const int wave_last = tok0 + wv * tw + tw - 1;
  bf16x8 qb[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 raw = *reinterpret_cast<const uint4*>(a.q + (size_t)qrow[rb] * kD + 32 * ks + 8 * g4);
      if (!valid[rb]) raw = make_uint4(0, 0, 0, 0);
      qb[rb][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  NewRegs nr;
  new_load(a, s0, kmax, 0, kvh, tid, nr);
  new_store(s, 0, tid, nr);
  __syncthreads();
  for (int nt = 0; nt < n_nt; ++nt) {
    const int buf = nt & 1;
    const bool more = nt + 1 < n_nt;
    if (more) new_load(a, s0, kmax, nt + 1, kvh, tid, nr);
    if (nt * kKeys <= wave_last) {
      f32x4 S[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) S[kb][0] = S[kb][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 ka = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4*>(&s.k[buf][(16 * kb + c16) * kKStride + 32 * ks + 8 * g4]));
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            S[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[rb][ks], S[kb][rb], 0, 0, 0);
        }
      bf16x8 ph[2][2], pl[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = nt * kKeys + 16 * (i >> 2) + 4 * g4 + (i & 3);
          p[i] = key <= tok[rb] ? S[i >> 2][rb][i & 3] * a.scale_log2 : kNegInf;
        }
        softmax_step(p, m_run[rb], l_run[rb], O[rb]);
        split_bf16x8(p, ph[rb][0], pl[rb][0]);
        split_bf16x8(p + 8, ph[rb][1], pl[rb][1]);
      }
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 va = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4*>(&s.v[buf][(16 * t + c16) * kVStride + 32 * ks2 + 8 * g4]));
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            O[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph[rb][ks2], O[rb][t], 0, 0, 0);
            O[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl[rb][ks2], O[rb][t], 0, 0, 0);
          }
        }
    }
    if (more) new_store(s, buf ^ 1, tid, nr);
    __syncthreads();
  }

  // ---- normalise and write
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float l = sum_over_row_lanes(l_run[rb]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (valid[rb]) {
      float* o = a.out + (size_t)qrow[rb] * kD + 4 * g4;
#pragma unroll
      for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(o + 16 * t) = O[rb][t] * inv;
    }
  }
}

}  // namespace
}  // namespace kvq

namespace kvq {

float extend_level_scale() { return kLevelScale; }

hipError_t launch_extend(const ExtendArgs& a, int tiles_per_seq, hipStream_t s) {
  k_extend_iso3<<<dim3((unsigned)(a.hkv * tiles_per_seq), (unsigned)a.batch), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
