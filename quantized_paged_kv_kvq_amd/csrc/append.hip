// Quantize-on-write kernels: encode bf16 K/V head vectors into paged cells.
//
// Built with -ffp-contract=off: every binary32 product and sum is rounded on its own,
// division and sqrt are the correctly rounded HIP defaults, rintf rounds half to even,
// and the binary32 -> binary16 conversion rounds to nearest even.  Under that contract
// each encoder is a pure function of its input vector.
//
//   INT8_G64   strata PR #2698, "What it does" (int8 codes + one FP16 scale = absmax/127 per
//              64 values); strata PR #120, "Tests" (INT8 rounding ties to even).
//   Q4_0_H256  strata PR #120, "What"/"How" and strata PR #2698, "Not in this PR"
//              (orthonormal FWHT-256 of V, then q4_0 blocks of 32 with d = signed max-abs / -8).
//   ISO3       FreeToken PR #398, "What" (per 128 values: L2-normalise, rotate each 4-group by a
//              unit quaternion, nearest 3-bit Lloyd-Max centroid, corrected norm).
//   ISO4       FreeToken PR #398, "What" (the 4-bit sibling: sixteen levels, nibble codes, the
//              corrected norm kept in binary32).
//   F32        strata PR #2698, intro and "What it does" (the unquantised FP32 store of the
//              single-store modes k8v32 / k32v8): the bf16 value widened to binary32, exact.
#include "kvq_internal.h"
#include "iso_levels.h"
#include "int8_cell.h"
#include "q4h_cell.h"

namespace kvq {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// (tile, slot) of appended token `tok`: tile = page * hkv + head is added by the caller.
// Device-side indices are clamped so a bad entry can never address outside the slabs.
__device__ __forceinline__ void locate(const AppendArgs& a, int tok, int& page, int& slot) {
  int seq, pos;
  if (a.cu_new) {
    int lo = 0, hi = a.batch - 1;                 // last b with cu_new[b] <= tok
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (a.cu_new[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    seq = lo;
    pos = a.seq_lens[seq] + (tok - a.cu_new[seq]);
  } else {
    seq = a.tok_seq[tok];
    pos = a.tok_pos[tok];
  }
  seq = clampi(seq, 0, a.batch - 1);
  pos = clampi(pos, 0, a.max_pages * KVQ_PAGE_SIZE - 1);
  page = clampi(a.bt[(size_t)seq * a.max_pages + pos / KVQ_PAGE_SIZE], 0, a.num_pages - 1);
  slot = pos % KVQ_PAGE_SIZE;
}

// ---------------------------------------------------------------------------------------------
// INT8_G64.  One thread encodes 4 consecutive values (int8_encode_x4); the 16 threads of a
// 64-group are 16 consecutive lanes.
template <int CPT>
__device__ __forceinline__ void append_int8(const AppendArgs& a, const uint16_t* __restrict__ x,
                                            uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, int D,
                                            bool is_v, int block) {
  const int tpc = D >> 2;                          // threads per cell
  const int cpb = blockDim.x / tpc;                // cells per block and pass
  const int local = threadIdx.x / tpc;
  const int part = threadIdx.x - local * tpc;      // values 4*part .. 4*part+3
  const long n_cells = (long)a.n_tok * a.hkv;
  // the block's CPT passes take CPT * cpb consecutive cells; every pass's load is issued before the
  // first encode, so a thread keeps CPT loads in flight
  uint2 raw[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const long cell = ((long)block * CPT + i) * cpb + local;
    const long c = cell < n_cells ? cell : 0;
    raw[i] = *reinterpret_cast<const uint2*>(x + (size_t)c * D + 4 * part);
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const long cell = ((long)block * CPT + i) * cpb + local;
    float v[4] = {bf16_to_f32(raw[i].x & 0xffffu), bf16_to_f32(raw[i].x >> 16), bf16_to_f32(raw[i].y & 0xffffu),
                  bf16_to_f32(raw[i].y >> 16)};
    const Int8x4 enc = int8_encode_x4(v);          // (lane shuffles: every lane takes part)
    if (cell >= n_cells) continue;
    const uint32_t packed = enc.packed;
    const int tok = (int)(cell / a.hkv), head = (int)(cell % a.hkv);
    int page, slot;
    locate(a, tok, page, slot);
    const size_t tile = (size_t)page * a.hkv + head;
    uint8_t* base = codes + tile * KVQ_PAGE_SIZE * D;
    if (!is_v) {
      *reinterpret_cast<uint32_t*>(base + k_tile_offset(4 * part, slot)) = packed;   // 4 bytes of one chunk
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) base[v_tile_offset(4 * part + e, slot)] = (uint8_t)(packed >> (8 * e));
    }
    if ((part & 15) == 0)
      scales[(tile * KVQ_PAGE_SIZE + slot) * (D / 64) + (part >> 4)] = enc.scale_bits;
  }
}

// ---------------------------------------------------------------------------------------------
// F32: one thread writes 4 consecutive values of a cell.  K tiles take them as one 16-byte chunk;
// V tiles keep each value's 16 slots together (4-byte stores, 64 bytes apart).
template <int CPT>
__device__ __forceinline__ void append_f32(const AppendArgs& a, const uint16_t* __restrict__ x,
                                           uint8_t* __restrict__ codes, int D, bool is_v, int block) {
  const int tpc = D >> 2;                          // threads per cell
  const int cpb = blockDim.x / tpc;                // cells per block and pass
  const int local = threadIdx.x / tpc;
  const int part = threadIdx.x - local * tpc;      // values 4*part .. 4*part+3
  const long n_cells = (long)a.n_tok * a.hkv;
  uint2 raw[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const long cell = ((long)block * CPT + i) * cpb + local;
    raw[i] = cell < n_cells ? *reinterpret_cast<const uint2*>(x + (size_t)cell * D + 4 * part) : make_uint2(0, 0);
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const long cell = ((long)block * CPT + i) * cpb + local;
    if (cell >= n_cells) continue;
    const float v[4] = {bf16_to_f32(raw[i].x & 0xffffu), bf16_to_f32(raw[i].x >> 16),
                        bf16_to_f32(raw[i].y & 0xffffu), bf16_to_f32(raw[i].y >> 16)};
    const int tok = (int)(cell / a.hkv), head = (int)(cell % a.hkv);
    int page, slot;
    locate(a, tok, page, slot);
    uint8_t* base = codes + ((size_t)page * a.hkv + head) * KVQ_PAGE_SIZE * (4 * D);
    if (!is_v) {
      *reinterpret_cast<float4*>(base + k_tile_offset(16 * part, slot)) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<float*>(base + vf32_tile_offset(4 * (4 * part + e), slot)) = v[e];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Q4_0_H256 (K or V; their tiles differ in byte order).  One wave per cell; lane l holds elements
// 4l .. 4l+3 (the encoder is q4h_encode_x4).
template <int CPT>
__device__ __forceinline__ void append_q4h(const AppendArgs& a, const uint16_t* __restrict__ x,
                                           uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, bool is_v,
                                           int block) {
  const int lane = threadIdx.x & 63;
  const int wpb = blockDim.x >> 6;                 // cells per block and pass
  const long n_cells = (long)a.n_tok * a.hkv;
  uint2 raw[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const long cell = ((long)block * CPT + i) * wpb + (threadIdx.x >> 6);
    const long c = cell < n_cells ? cell : 0;
    raw[i] = *reinterpret_cast<const uint2*>(x + (size_t)c * 256 + 4 * lane);
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const long cell = ((long)block * CPT + i) * wpb + (threadIdx.x >> 6);
    float y[4] = {bf16_to_f32(raw[i].x & 0xffffu), bf16_to_f32(raw[i].x >> 16), bf16_to_f32(raw[i].y & 0xffffu),
                  bf16_to_f32(raw[i].y >> 16)};
    const Q4x4 e = q4h_encode_x4(y, lane);         // (wave-wide shuffles: every lane takes part)
    if (cell >= n_cells) continue;
    const int tok = (int)(cell / a.hkv), head = (int)(cell % a.hkv);
    int page, slot;
    locate(a, tok, page, slot);
    const size_t tile = (size_t)page * a.hkv + head;
    uint8_t* base = codes + tile * KVQ_PAGE_SIZE * 128;
    const int o0 = is_v ? v_tile_offset(2 * lane, slot) : k4_tile_offset(2 * lane, slot);
    const int o1 = is_v ? v_tile_offset(2 * lane + 1, slot) : k4_tile_offset(2 * lane + 1, slot);
    base[o0] = e.b0;
    base[o1] = e.b1;
    if ((lane & 7) == 0) scales[(tile * KVQ_PAGE_SIZE + slot) * 8 + (lane >> 3)] = e.d_bits;
  }
}

// ---------------------------------------------------------------------------------------------
// ISO3.  One wave per 128-value block; lane l holds elements l and l + 64, so the pairwise
// halving sum (upper half onto lower half: spans 64, 32, ..., 1) is an in-lane add followed by
// xor-shuffles 32 .. 1.

__device__ __forceinline__ float halving_sum128(float lo, float hi) {
  float s = lo + hi;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s = s + __shfl_xor(s, o);
  return s;
}

// Component `comp` of the Hamilton product (w,x,y,z) * (a,b,c,d), each evaluated left to right.
__device__ __forceinline__ float hamilton(int comp, float w, float x, float y, float z, float a, float b,
                                          float c, float d) {
  const float r0 = ((w * a - x * b) - y * c) - z * d;
  const float r1 = ((w * b + x * a) + y * d) - z * c;
  const float r2 = ((w * c - x * d) + y * a) + z * b;
  const float r3 = ((w * d + x * c) - y * b) + z * a;
  return comp == 0 ? r0 : comp == 1 ? r1 : comp == 2 ? r2 : r3;
}

template <int BITS>
__device__ __forceinline__ float iso_level(int k) { return BITS == 3 ? kIsoLevels[k] : kIso4Levels[k]; }

template <int BITS>
__device__ __forceinline__ int nearest_centroid(float r) {
  int best = 0;
  float bd = fabsf(r - iso_level<BITS>(0));
#pragma unroll
  for (int k = 1; k < (1 << BITS); ++k) {
    const float dk = fabsf(r - iso_level<BITS>(k));
    if (dk < bd) { bd = dk; best = k; }
  }
  return best;
}

__device__ __forceinline__ float rotate_component(float u, int lane, float w, float x, float y, float z) {
  const int base = lane & ~3;
  const float a = __shfl(u, base + 0), b = __shfl(u, base + 1), c = __shfl(u, base + 2), d = __shfl(u, base + 3);
  return hamilton(lane & 3, w, x, y, z, a, b, c, d);
}

// ISO4 (FreeToken PR #398, "What": the 4-bit sibling) takes the same steps with sixteen levels,
// packs the codes as nibbles and keeps the corrected norm in binary32 (two 16-bit scale slots).
template <int BITS, int P>
__device__ __forceinline__ void append_iso(const AppendArgs& a, const uint16_t* __restrict__ x,
                                           uint8_t* __restrict__ codes, uint16_t* __restrict__ norms, int D,
                                           const float quat[4], int block) {
  // P passes per wave: the wave encodes P 128-value blocks whose steps are independent, so their
  // loads, shuffle reductions and searches overlap (one block's chain is latency-bound)
  __shared__ uint8_t lds_codes[4][P][128];
  const float qw = quat[0], qx = quat[1], qy = quat[2], qz = quat[3];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nb = D / 128;
  const long n_blk = (long)a.n_tok * a.hkv * nb;
  float x0[P], x1[P], n[P], norm[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const long blk_id = ((long)block * P + i) * 4 + wv;
    const long bi = blk_id < n_blk ? blk_id : 0;
    const uint16_t* src = x + (size_t)(bi / nb) * D + (int)(bi % nb) * 128;
    x0[i] = bf16_to_f32(src[lane]);
    x1[i] = bf16_to_f32(src[64 + lane]);
  }
#pragma unroll
  for (int i = 0; i < P; ++i) n[i] = sqrtf(halving_sum128(x0[i] * x0[i], x1[i] * x1[i]));
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const float u0 = n[i] > 0.0f ? x0[i] / n[i] : 0.0f;
    const float u1 = n[i] > 0.0f ? x1[i] / n[i] : 0.0f;
    const float r0 = rotate_component(u0, lane, qw, qx, qy, qz);
    const float r1 = rotate_component(u1, lane, qw, qx, qy, qz);
    const int c0 = nearest_centroid<BITS>(r0), c1 = nearest_centroid<BITS>(r1);
    x0[i] = iso_level<BITS>(c0);                       // (the levels replace the inputs)
    x1[i] = iso_level<BITS>(c1);
    lds_codes[wv][i][lane] = (uint8_t)c0;
    lds_codes[wv][i][64 + lane] = (uint8_t)c1;
  }
#pragma unroll
  for (int i = 0; i < P; ++i) norm[i] = n[i] / sqrtf(halving_sum128(x0[i] * x0[i], x1[i] * x1[i]));
  __syncthreads();
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const long blk_id = ((long)block * P + i) * 4 + wv;
    if (blk_id >= n_blk) continue;
    const long cell = blk_id / nb;
    const int blk = (int)(blk_id % nb);
    const int tok = (int)(cell / a.hkv), head = (int)(cell % a.hkv);
    int page, slot;
    locate(a, tok, page, slot);
    const size_t tile = (size_t)page * a.hkv + head;
    if constexpr (BITS == 3) {
      const int cb = nb * 48;
      if (lane < 48) {
        const int t = lane / 3;                        // 3 bytes hold codes 8t .. 8t+7
        uint32_t word = 0;
#pragma unroll
        for (int m = 0; m < 8; ++m) word |= (uint32_t)lds_codes[wv][i][8 * t + m] << (3 * m);
        codes[(tile * KVQ_PAGE_SIZE + slot) * cb + blk * 48 + lane] = (uint8_t)(word >> (8 * (lane % 3)));
      }
      if (lane == 0) norms[(tile * KVQ_PAGE_SIZE + slot) * nb + blk] = f32_to_f16_bits(norm[i]);
    } else {
      const int cb = nb * 64;                          // byte j: code 2j (low nibble), 2j + 1 (high)
      codes[(tile * KVQ_PAGE_SIZE + slot) * cb + blk * 64 + lane] =
          (uint8_t)(lds_codes[wv][i][2 * lane] | (lds_codes[wv][i][2 * lane + 1] << 4));
      if (lane == 0) reinterpret_cast<float*>(norms)[(tile * KVQ_PAGE_SIZE + slot) * nb + blk] = norm[i];
    }
  }
}

// Blocks needed by one store's encoder for n_tok tokens (256 threads per block).
// `passes`: cells per thread of the int8 and q4_0 encoders, 128-value blocks per wave of the ISO
// encoders (FP32 takes one).
long blocks_for(int fmt, int D, long cells, int passes) {
  if (fmt == KVQ_FMT_INT8_G64 || fmt == KVQ_FMT_F32) {
    const int cpb = 256 / (D / 4) * (fmt == KVQ_FMT_INT8_G64 ? passes : 1);
    return (cells + cpb - 1) / cpb;
  }
  if (fmt == KVQ_FMT_Q4_0_H256) return (cells + 4 * passes - 1) / (4 * passes);
  return (cells * (D / 128) + 4 * passes - 1) / (4 * passes);   // ISO3 / ISO4: one wave per 128-value block and pass
}

struct StoreArgs {
  int fmt;
  int is_v;
  const uint16_t* x;
  uint8_t* codes;
  uint16_t* scales;
  long blocks;
};

// One launch encodes both stores: blockIdx.y picks K (0) or V (1); blocks past a store's count exit.
// PLAIN instantiates the int8, q4_0 and FP32 encoders, ISO the ISO3 / ISO4 ones (their registers
// and code stay out of each other's kernels); PASSES is the encoders' cells (ISO: blocks) per thread
// (FP32: one).
template <bool PLAIN, bool ISO, int PASSES>
__global__ __launch_bounds__(256) void k_append(AppendArgs a, StoreArgs k, StoreArgs v, int D, float qw, float qx,
                                                float qy, float qz) {
  const StoreArgs& st = blockIdx.y == 0 ? k : v;
  // Workgroups are dealt to the 8 XCDs round robin.  Block b encodes logical block (b % 8) * per +
  // b / 8, so each XCD takes one contiguous run of a store's cells: the slots of a page, whose cells
  // share cache lines, are written through one L2, which merges the partial lines before they go to HBM.
  const long per = (st.blocks + 7) >> 3;           // this store's logical blocks per XCD
  const long j = blockIdx.x >> 3;
  const long lb = (long)(blockIdx.x & 7) * per + j;
  if (j >= per || lb >= st.blocks) return;
  if constexpr (PLAIN) {
    if (st.fmt == KVQ_FMT_INT8_G64) return append_int8<PASSES>(a, st.x, st.codes, st.scales, D, st.is_v != 0, (int)lb);
    if (st.fmt == KVQ_FMT_Q4_0_H256) return append_q4h<PASSES>(a, st.x, st.codes, st.scales, st.is_v != 0, (int)lb);
    if (st.fmt == KVQ_FMT_F32) return append_f32<1>(a, st.x, st.codes, D, st.is_v != 0, (int)lb);
  }
  if constexpr (ISO) {
    const float quat[4] = {qw, qx, qy, qz};
    if (st.fmt == KVQ_FMT_ISO4) append_iso<4, PASSES>(a, st.x, st.codes, st.scales, D, quat, (int)lb);
    else if (st.fmt == KVQ_FMT_ISO3) append_iso<3, PASSES>(a, st.x, st.codes, st.scales, D, quat, (int)lb);
  }
}

}  // namespace

hipError_t launch_append_kv(int fmt_k, const uint16_t* xk, uint8_t* codes_k, uint16_t* scales_k, int fmt_v,
                            const uint16_t* xv, uint8_t* codes_v, uint16_t* scales_v, int D, const float quat[4],
                            const AppendArgs& a, hipStream_t s) {
  const long cells = (long)a.n_tok * a.hkv;
  if (cells == 0 || (!xk && !xv)) return hipSuccess;
  // A multi-token append of more than about two rounds of the CUs at one cell (ISO: one 128-value
  // block per wave) per thread streams from HBM: then each int8 / q4_0 thread takes 4 cells with
  // all their loads in flight together (a cache fill of 131,072 tokens: 307 -> 212 us), and each
  // ISO wave 4 blocks whose latency-bound chains overlap.  A decode step's append keeps one cell
  // per thread, the shortest path.
  auto is_iso = [](int f) { return f == KVQ_FMT_ISO3 || f == KVQ_FMT_ISO4; };
  const long one_pass = (long)(xk ? blocks_for(fmt_k, D, cells, 1) : 0) + (xv ? blocks_for(fmt_v, D, cells, 1) : 0);
  const int passes = one_pass > 16L * device_cu_count() ? 4 : 1;
  StoreArgs k{fmt_k, 0, xk, codes_k, scales_k, xk ? blocks_for(fmt_k, D, cells, passes) : 0};
  StoreArgs v{fmt_v, 1, xv, codes_v, scales_v, xv ? blocks_for(fmt_v, D, cells, passes) : 0};
  const long gx = ((k.blocks > v.blocks ? k.blocks : v.blocks) + 7) / 8 * 8;   // whole rounds of the 8 XCDs
  dim3 grid((unsigned)gx, xv ? 2 : 1);
  if (!xk) {                                 // V only: make it the y == 0 slot
    k = v;
    grid.y = 1;
  }
  const bool iso = (xk && is_iso(fmt_k)) || (xv && is_iso(fmt_v));
  const bool plain = (xk && !is_iso(fmt_k)) || (xv && !is_iso(fmt_v));
  const float qw = quat[0], qx = quat[1], qy = quat[2], qz = quat[3];
  if (plain && iso) {
    if (passes == 4) k_append<true, true, 4><<<grid, dim3(256), 0, s>>>(a, k, v, D, qw, qx, qy, qz);
    else k_append<true, true, 1><<<grid, dim3(256), 0, s>>>(a, k, v, D, qw, qx, qy, qz);
  } else if (iso) {
    if (passes == 4) k_append<false, true, 4><<<grid, dim3(256), 0, s>>>(a, k, v, D, qw, qx, qy, qz);
    else k_append<false, true, 1><<<grid, dim3(256), 0, s>>>(a, k, v, D, qw, qx, qy, qz);
  } else {
    if (passes == 4) k_append<true, false, 4><<<grid, dim3(256), 0, s>>>(a, k, v, D, qw, qx, qy, qz);
    else k_append<true, false, 1><<<grid, dim3(256), 0, s>>>(a, k, v, D, qw, qx, qy, qz);
  }
  return hipGetLastError();
}

}  // namespace kvq
