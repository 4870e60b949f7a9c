// Dequant-gather: cells [start, start+count) of one sequence of one store -> contiguous values.
//
// The one-time dequantisation of a packed prefix (FreeToken PR #398, "What"), the dequantise-a-
// cache-range step of a prompt chunk (strata PR #2698, "What it does") and the gather half of the
// append/gather parity checks (strata PR #120, "Tests").  Built with -ffp-contract=off: the F32
// output equals the dequantised value of each format exactly:
//   INT8_G64   code * scale                            (exact in binary32)
//   Q4_0_H256  (code - 8) * d, rotated basis            (exact); with `unrotate`, H applied by
//              binary32 butterflies of spans 1..128 and a final x 1/16
//   ISO3/ISO4  conj(q) * centroid group (left to right), then times the norm
//   F32        the stored binary32 value
#include "kvq_internal.h"
#include "iso_levels.h"

namespace kvq {
namespace {

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ size_t tile_of(const GatherArgs& g, int i, int head, int& slot) {
  const int pos = clampi(g.start + i, 0, g.max_pages * KVQ_PAGE_SIZE - 1);
  const int page = clampi(g.bt[(size_t)g.seq * g.max_pages + pos / KVQ_PAGE_SIZE], 0, g.num_pages - 1);
  slot = pos % KVQ_PAGE_SIZE;
  return (size_t)page * g.hkv + head;
}

__device__ __forceinline__ void store4(void* out, size_t idx, const float v[4], int dtype) {
  if (dtype == KVQ_OUT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else if (dtype == KVQ_OUT_F16) {
    uint16_t* o = static_cast<uint16_t*>(out) + idx;
    for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[e]));
  } else {
    uint16_t* o = static_cast<uint16_t*>(out) + idx;
    for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[e]));
  }
}

// INT8_G64: one thread per 4 consecutive values of a cell.
__global__ __launch_bounds__(256) void k_gather_int8(GatherArgs g, const uint8_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ scales, int D, int is_v,
                                                     void* out, int dtype) {
  const int tpc = D / 4;
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long cells = (long)g.count * g.hkv;
  if (t >= cells * tpc) return;
  const long cell = t / tpc;
  const int part = (int)(t % tpc);
  const int i = (int)(cell / g.hkv), head = (int)(cell % g.hkv);
  int slot;
  const size_t tile = tile_of(g, i, head, slot);
  const float s = f16_bits_to_f32(scales[(tile * KVQ_PAGE_SIZE + slot) * (D / 64) + (4 * part) / 64]);
  float v[4];
  for (int e = 0; e < 4; ++e) {
    const int d = 4 * part + e;
    const size_t off = tile * KVQ_PAGE_SIZE * D + (is_v ? v_tile_offset(d, slot) : k_tile_offset(d, slot));
    v[e] = (float)(int8_t)codes[off] * s;
  }
  store4(out, ((size_t)i * g.hkv + head) * D + 4 * part, v, dtype);
}

// F32 (K or V tile order): one thread per 4 consecutive values of a cell.
__global__ __launch_bounds__(256) void k_gather_f32(GatherArgs g, const uint8_t* __restrict__ codes, int D, int is_v,
                                                    void* out, int dtype) {
  const int tpc = D / 4;
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long cells = (long)g.count * g.hkv;
  if (t >= cells * tpc) return;
  const long cell = t / tpc;
  const int part = (int)(t % tpc);
  const int i = (int)(cell / g.hkv), head = (int)(cell % g.hkv);
  int slot;
  const size_t tile = tile_of(g, i, head, slot);
  const uint8_t* base = codes + tile * KVQ_PAGE_SIZE * (4 * D);
  float v[4];
  if (!is_v) {
    const float4 q = *reinterpret_cast<const float4*>(base + k_tile_offset(16 * part, slot));
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
    for (int e = 0; e < 4; ++e) v[e] = *reinterpret_cast<const float*>(base + vf32_tile_offset(4 * (4 * part + e), slot));
  }
  store4(out, ((size_t)i * g.hkv + head) * D + 4 * part, v, dtype);
}

// Q4_0_H256 (K or V tile order): one wave per cell, lane l holds elements 4l .. 4l+3.
__global__ __launch_bounds__(256) void k_gather_q4h(GatherArgs g, const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales, int is_v, void* out,
                                                    int dtype, int unrotate) {
  const int lane = threadIdx.x & 63;
  const long cell = (long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const bool active = cell < (long)g.count * g.hkv;
  const long c = active ? cell : 0;
  const int i = (int)(c / g.hkv), head = (int)(c % g.hkv);
  int slot;
  const size_t tile = tile_of(g, i, head, slot);
  const uint8_t* base = codes + tile * KVQ_PAGE_SIZE * 128;
  const uint32_t b0 = base[is_v ? v_tile_offset(2 * lane, slot) : k4_tile_offset(2 * lane, slot)];
  const uint32_t b1 = base[is_v ? v_tile_offset(2 * lane + 1, slot) : k4_tile_offset(2 * lane + 1, slot)];
  const float d = f16_bits_to_f32(scales[(tile * KVQ_PAGE_SIZE + slot) * 8 + (lane >> 3)]);
  float y[4] = {(float)((int)(b0 & 15) - 8) * d, (float)((int)(b0 >> 4) - 8) * d, (float)((int)(b1 & 15) - 8) * d,
                (float)((int)(b1 >> 4) - 8) * d};
  if (unrotate) {
    float a0 = y[0] + y[1], a1 = y[0] - y[1], a2 = y[2] + y[3], a3 = y[2] - y[3];
    y[0] = a0 + a2; y[2] = a0 - a2; y[1] = a1 + a3; y[3] = a1 - a3;
    for (int o = 1; o < 64; o <<= 1) {
      const bool upper = (lane & o) != 0;
      for (int e = 0; e < 4; ++e) {
        const float other = __shfl_xor(y[e], o);
        y[e] = upper ? (other - y[e]) : (y[e] + other);
      }
    }
    for (int e = 0; e < 4; ++e) y[e] = y[e] * 0.0625f;
  }
  if (active) store4(out, ((size_t)i * g.hkv + head) * 256 + 4 * lane, y, dtype);
}


// ISO3 / ISO4: one thread per 4-value group; the group's 12 (16) code bits start at bit 12*g (16*g)
// of its block.
template <int BITS>
__global__ __launch_bounds__(256) void k_gather_iso(GatherArgs g, const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ norms, int D, float qw, float qx,
                                                    float qy, float qz, void* out, int dtype) {
  const int gpc = D / 4;                          // groups per cell
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long cells = (long)g.count * g.hkv;
  if (t >= cells * gpc) return;
  const long cell = t / gpc;
  const int grp = (int)(t % gpc);
  const int i = (int)(cell / g.hkv), head = (int)(cell % g.hkv);
  const int blk = grp / 32, gi = grp % 32;
  int slot;
  const size_t tile = tile_of(g, i, head, slot);
  const int nb = D / 128;
  float a, b, c, d, nrm;
  if constexpr (BITS == 3) {
    const uint8_t* cb = codes + (tile * KVQ_PAGE_SIZE + slot) * (nb * 48) + blk * 48;
    const int bit = 12 * gi;
    const uint32_t w16 = (uint32_t)cb[bit >> 3] | ((uint32_t)cb[(bit >> 3) + 1] << 8);
    const uint32_t bits = w16 >> (bit & 7);
    a = kIsoLevels[bits & 7]; b = kIsoLevels[(bits >> 3) & 7]; c = kIsoLevels[(bits >> 6) & 7];
    d = kIsoLevels[(bits >> 9) & 7];
    nrm = f16_bits_to_f32(norms[(tile * KVQ_PAGE_SIZE + slot) * nb + blk]);
  } else {
    const uint8_t* cb = codes + (tile * KVQ_PAGE_SIZE + slot) * (nb * 64) + blk * 64 + 2 * gi;
    const uint32_t bits = (uint32_t)cb[0] | ((uint32_t)cb[1] << 8);
    a = kIso4Levels[bits & 15]; b = kIso4Levels[(bits >> 4) & 15]; c = kIso4Levels[(bits >> 8) & 15];
    d = kIso4Levels[bits >> 12];
    nrm = reinterpret_cast<const float*>(norms)[(tile * KVQ_PAGE_SIZE + slot) * nb + blk];
  }
  // conjugate quaternion (w, -x, -y, -z), same evaluation order as the encoder's product
  const float w = qw, x = -qx, y = -qy, z = -qz;
  const float r0 = ((w * a - x * b) - y * c) - z * d;
  const float r1 = ((w * b + x * a) + y * d) - z * c;
  const float r2 = ((w * c - x * d) + y * a) + z * b;
  const float r3 = ((w * d + x * c) - y * b) + z * a;
  const float v[4] = {r0 * nrm, r1 * nrm, r2 * nrm, r3 * nrm};
  store4(out, ((size_t)i * g.hkv + head) * D + 4 * grp, v, dtype);
}

}  // namespace

hipError_t launch_gather(int fmt, bool is_v, const uint8_t* codes, const uint16_t* scales, int D,
                         const float quat[4], const GatherArgs& g, int out_dtype, bool unrotate, void* out,
                         hipStream_t s) {
  const long cells = (long)g.count * g.hkv;
  if (cells == 0) return hipSuccess;
  if (fmt == KVQ_FMT_INT8_G64) {
    const long threads = cells * (D / 4);
    k_gather_int8<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(g, codes, scales, D, is_v ? 1 : 0,
                                                                               out, out_dtype);
  } else if (fmt == KVQ_FMT_F32) {
    const long threads = cells * (D / 4);
    k_gather_f32<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(g, codes, D, is_v ? 1 : 0, out,
                                                                              out_dtype);
  } else if (fmt == KVQ_FMT_Q4_0_H256) {
    k_gather_q4h<<<dim3((unsigned)((cells + 3) / 4)), dim3(256), 0, s>>>(g, codes, scales, is_v ? 1 : 0, out,
                                                                          out_dtype, unrotate ? 1 : 0);
  } else if (fmt == KVQ_FMT_ISO4) {
    const long threads = cells * (D / 4);
    k_gather_iso<4><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(g, codes, scales, D, quat[0],
                                                                                 quat[1], quat[2], quat[3], out,
                                                                                 out_dtype);
  } else {
    const long threads = cells * (D / 4);
    k_gather_iso<3><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(g, codes, scales, D, quat[0],
                                                                                 quat[1], quat[2], quat[3], out,
                                                                                 out_dtype);
  }
  return hipGetLastError();
}

}  // namespace kvq
