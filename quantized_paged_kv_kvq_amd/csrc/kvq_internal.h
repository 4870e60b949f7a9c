// Library-internal declarations shared by the HIP translation units of libkvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// Byte order of code byte c of the cell in slot t inside one (page, KV head) tile (see kvq.h):
//   INT8_G64 K stores: 16-byte chunks, chunk-major -- a wave reads a contiguous kilobyte per load
//   INT8_G64 / Q4_0_H256 V stores: 4 consecutive slots of one code byte form a 32-bit word; the
//     words of code bytes c, c+16, c+32, c+48 (c % 64 < 16) form a 16-byte unit
//   Q4_0_H256 K stores: 16-byte units, unit (c/64, (c/4)%4, t) holds bytes 4w .. 4w+3 (w = (c/4)%4) of
//     the four 32-value groups c/64*4 .. +3 of slot t -- one wave load covers a contiguous kilobyte
//   ISO3 / ISO4 stores: token-major
//   F32 K stores: as INT8_G64 K (a 16-byte chunk holds 4 values); F32 V stores: head_dim-major, the 16
//     slots of one head_dim index are 64 contiguous bytes
__host__ __device__ inline int k_tile_offset(int c, int t) { return ((c >> 4) * 16 + t) * 16 + (c & 15); }
__host__ __device__ inline int k4_tile_offset(int c, int t) {
  return (((c >> 6) * 4 + ((c >> 2) & 3)) * 16 + t) * 16 + ((c >> 4) & 3) * 4 + (c & 3);
}
__host__ __device__ inline int vf32_tile_offset(int c, int t) { return ((c >> 2) * 16 + t) * 4 + (c & 3); }
__host__ __device__ inline int v_tile_offset(int c, int t) {
  return ((((c >> 6) << 4) | (c & 15)) * 4 + (t >> 2)) * 16 + ((c >> 4) & 3) * 4 + (t & 3);
}

// Where appended tokens go: the page table of a batch plus the per-token (sequence, position).
struct AppendArgs {
  const int32_t* tok_seq;   // [n_tok]
  const int32_t* tok_pos;   // [n_tok]
  const int32_t* bt;        // [batch][max_pages]
  int n_tok;
  int batch;
  int max_pages;
  int num_pages;
  int hkv;
  // Extend's deferred packing derives (seq, pos) from the chunk layout instead of tok_seq/tok_pos:
  // token i of the chunk belongs to the sequence b with cu_new[b] <= i < cu_new[b+1] and sits at
  // position seq_lens[b] + (i - cu_new[b]).
  const int32_t* cu_new;    // [batch + 1] or nullptr
  const int32_t* seq_lens;  // [batch] (only with cu_new)
};

// Encode n_tok tokens into the K store and/or the V store (x == nullptr skips a store), one launch.
hipError_t launch_append_kv(int fmt_k, const uint16_t* xk, uint8_t* codes_k, uint16_t* scales_k, int fmt_v,
                            const uint16_t* xv, uint8_t* codes_v, uint16_t* scales_v, int head_dim,
                            const float quat[4], const AppendArgs& a, hipStream_t s);

struct GatherArgs {
  const int32_t* bt;
  int max_pages;
  int num_pages;
  int hkv;
  int seq;
  int start;
  int count;
};

hipError_t launch_gather(int fmt, bool is_v, const uint8_t* codes, const uint16_t* scales,
                         int head_dim, const float quat[4], const GatherArgs& g, int out_dtype,
                         bool unrotate, void* out, hipStream_t s);

// Decode: one row per (query token, query head) of a KV head; rows of KV head j are
// head_list[head_off[j] .. head_off[j+1]) repeated for every query token.
struct DecodeArgs {
  const uint8_t* k_codes;
  const uint16_t* k_scales;
  const uint8_t* v_codes;
  const uint16_t* v_scales;
  const uint16_t* q;        // bf16 [batch][n_q][n_q_heads][head_dim]
  const int32_t* q_lens;    // [batch][n_q] or nullptr
  const int32_t* seq_lens;  // [batch]
  const int32_t* bt;        // [batch][max_pages]
  float* part;              // split partials
  float* out;               // fp32 [batch][n_q][n_q_heads][head_dim]
  int hkv;
  int num_pages;
  int max_pages;
  int batch;
  int n_q;
  int n_q_heads;
  int pages_per_split;
  int n_splits;
  float scale_log2;         // sm_scale * log2(e)
  int g_uniform;            // G when query head h reads KV head h / G (the default map), else 0
  int row_groups;           // workgroups per split: each takes 8 query rows of the KV head
  int row_alloc;            // rows of the partials per (sequence, KV head): 8 * row_groups
  int16_t head_off[KVQ_MAX_Q_HEADS + 1];
  int16_t head_list[KVQ_MAX_Q_HEADS];
  // fused quantize-on-write (INT8_G64 K; INT8_G64 or Q4_0_H256 V): new token t of sequence b, bf16
  // [batch][n_q][hkv][head_dim], is encoded into position seq_lens[b] - n_q + t before the
  // attention reads it; nullptr: plain decode
  const uint16_t* k_new;
  const uint16_t* v_new;
  float quat[4];            // ISO3 stores: the rotation quaternion (w, x, y, z)
};
constexpr int kDecodeMaxFused = 4;     // new tokens per sequence of a fused decode

// Output row (b, query token, query head) of row r of KV head kvh (G rows per token, heads from h0).
__device__ __forceinline__ int decode_out_row(const DecodeArgs& a, int b, int kvh, int r, int G, int h0) {
  const int t = r / G, i = r % G;
  const int hq = a.g_uniform > 0 ? kvh * a.g_uniform + i : a.head_list[h0 + i];
  return (b * a.n_q + t) * a.n_q_heads + hq;
}
constexpr int kIsoDecodeMaxRows = 16;  // query rows per KV head of an ISO3 decode

struct DecodePlan {
  int shape;            // launch shape (waves, pages per wave, prefetch depth)
  int rows;             // query rows of the widest KV head
  int row_groups;       // groups of 8 query rows per KV head
  int row_tiles;        // 0: one workgroup per row group of 8 (duplicated columns); else one
                        // workgroup per split holds all rows in this many row tiles of 16
  int waves;            // waves per workgroup
  int pages_per_split;
  int n_splits;
  size_t part_bytes;
};

DecodePlan plan_decode(int v_fmt, int head_dim, int hkv, int batch, int max_pages, int max_rows);
hipError_t launch_decode(int v_fmt, int head_dim, const DecodePlan& plan, const DecodeArgs& a,
                         hipStream_t s);
// k8v4 (INT8_G64 K, Q4_0_H256 V) with more than 8 rows per KV head: wave pairs splitting head_dim
// (row_tiles 1 or 2 tiles of 16 rows), then the combine
hipError_t launch_decode_verify(int row_tiles, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s);
// the log-sum-exp combine of the split partials (every decode kernel writes the same layout)
hipError_t launch_decode_combine(int head_dim, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s);
// ISO3 or ISO4 K and V stores (bits 3 or 4; head_dim 128 or 256, at most kIsoDecodeMaxRows rows per
// KV head)
DecodePlan plan_decode_iso(int head_dim, int hkv, int batch, int max_pages, int max_rows);
hipError_t launch_decode_iso(int bits, int head_dim, const DecodePlan& plan, const DecodeArgs& a, hipStream_t s);
// Q4_0_H256 K and V stores (head_dim 256, at most kQ4DecodeMaxRows rows per KV head)
constexpr int kQ4DecodeMaxRows = 16;
DecodePlan plan_decode_q4(int hkv, int batch, int max_pages, int max_rows);
hipError_t launch_decode_q4(const DecodePlan& plan, const DecodeArgs& a, hipStream_t s);
// K and V stores each INT8_G64 or F32, at least one F32 (head_dim 128 or 256, up to 32 rows per KV head)
DecodePlan plan_decode_f32(int head_dim, int hkv, int batch, int max_pages, int max_rows);
hipError_t launch_decode_f32(bool k_f32, bool v_f32, int head_dim, const DecodePlan& plan, const DecodeArgs& a,
                             hipStream_t s);

// Extend over an ISO3 or INT8_G64 prefix: one row per (new token, query head); rows of KV head j use
// the query heads head_list[head_off[j] .. head_off[j+1]).
struct ExtendArgs {
  const uint8_t* k_codes;
  const uint16_t* k_norms;    // the scales slabs: ISO3 norms, or INT8_G64 group scales
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  const uint16_t* q;          // bf16 [n_new][n_q_heads][head_dim]
  const uint16_t* k_new;      // bf16 [n_new][hkv][head_dim]
  const uint16_t* v_new;
  const int32_t* cu_new;      // [batch + 1]
  const int32_t* prefix_lens; // [batch]
  const int32_t* bt;          // [batch][max_pages]
  float* out;                 // fp32 [n_new][n_q_heads][head_dim]
  uint8_t* ws;                // tile images: [batch][hkv][pt_max] prefix tiles, then [batch][hkv][nt_max] chunk tiles
  int pt_max;                 // prefix tiles per (sequence, KV head): ceil(max_pages * page_size / 64)
  int nt_max;                 // chunk tiles per (sequence, KV head): ceil(max_new / 64)
  int hkv;
  int num_pages;
  int max_pages;
  int batch;
  int n_new;
  int n_q_heads;
  int g_pad;                  // power of two >= the largest group; a wave holds 32 / g_pad tokens
  float quat[4];
  float q_scale;              // sm_scale * log2(e) / S (rotated prefix phase); 1 for int8 (applied to the scores)
  int int8;                   // INT8_G64 K and V stores instead of ISO3
  float scale_log2;           // sm_scale * log2(e)
  int g_uniform;
  int16_t head_off[KVQ_MAX_Q_HEADS + 1];
  int16_t head_list[KVQ_MAX_Q_HEADS];
};

// Extend attention workgroups have 8 waves of 32 query rows; a row is (token, query head slot).
constexpr int kExtendWaves = 8;
inline int extend_tokens_per_block(int g_pad) { return kExtendWaves * (32 / g_pad); }
// One 64-key tile image: K [64][128] + V [128][64] 16-bit values (rows padded by 16 bytes), then
// 64 + 64 fp32 norms, rounded up to whole kilobytes.
constexpr int kExtendTileBytes = 36864;
inline size_t extend_workspace_bytes(int batch, int hkv, int pt_max, int nt_max) {
  return (size_t)batch * hkv * ((size_t)pt_max + nt_max) * kExtendTileBytes;
}
float extend_level_scale();
hipError_t launch_extend(const ExtendArgs& a, int tiles_per_seq, hipStream_t s);

int device_cu_count();
int decode_max_splits();
// this device's address of kvq_decode_attn_noalloc's scratch array (looked up once per device)
kvq_status noalloc_scratch(void** ptr);

}  // namespace kvq
