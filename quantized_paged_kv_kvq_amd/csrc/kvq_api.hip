// C ABI of libkvq: argument validation on the host (before any HIP call), format dispatch,
// workspace sizing and kernel launches.  Declarations and the contract of every entry point are
// in include/kvq.h.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "kvq_internal.h"

namespace kvq {

namespace {
thread_local char g_err[512] = "";

kvq_status fail(kvq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool fmt_known(int f) {
  return f == KVQ_FMT_INT8_G64 || f == KVQ_FMT_Q4_0_H256 || f == KVQ_FMT_ISO3 || f == KVQ_FMT_F32 ||
         f == KVQ_FMT_ISO4;
}

// Geometry rules of a store format (the pages validate head_dim at config time with a message).
kvq_status check_store_fmt(int fmt, int D, bool is_v) {
  if (!fmt_known(fmt)) return fail(KVQ_ERR_UNSUPPORTED, "unknown store format %d", fmt);
  if (fmt == KVQ_FMT_INT8_G64 && (D % 64 != 0 || D > KVQ_MAX_HEAD_DIM))
    return fail(KVQ_ERR_UNSUPPORTED, "INT8_G64 needs head_dim %% 64 == 0 and <= %d (got %d)", KVQ_MAX_HEAD_DIM, D);
  if (fmt == KVQ_FMT_Q4_0_H256 && D != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "Q4_0_H256 needs head_dim == 256 (got %d)", D);
  if (fmt == KVQ_FMT_ISO3 && (D % 128 != 0 || D > KVQ_MAX_HEAD_DIM))
    return fail(KVQ_ERR_UNSUPPORTED, "ISO3 needs head_dim %% 128 == 0 and <= %d (got %d)", KVQ_MAX_HEAD_DIM, D);
  if (fmt == KVQ_FMT_ISO4 && (D % 128 != 0 || D > KVQ_MAX_HEAD_DIM))
    return fail(KVQ_ERR_UNSUPPORTED, "ISO4 needs head_dim %% 128 == 0 and <= %d (got %d)", KVQ_MAX_HEAD_DIM, D);
  if (fmt == KVQ_FMT_F32 && (D % 64 != 0 || D > KVQ_MAX_HEAD_DIM))
    return fail(KVQ_ERR_UNSUPPORTED, "F32 needs head_dim %% 64 == 0 and <= %d (got %d)", KVQ_MAX_HEAD_DIM, D);
  return KVQ_OK;
}

kvq_status check_cache(const kvq_cache* c) {
  if (!c) return fail(KVQ_ERR_NULL, "cache descriptor is NULL");
  if (c->page_size != KVQ_PAGE_SIZE) return fail(KVQ_ERR_UNSUPPORTED, "page_size must be %d (got %d)", KVQ_PAGE_SIZE, c->page_size);
  if (c->n_kv_heads < 1 || c->n_kv_heads > KVQ_MAX_Q_HEADS) return fail(KVQ_ERR_SHAPE, "n_kv_heads %d out of range", c->n_kv_heads);
  if (c->head_dim < 1) return fail(KVQ_ERR_SHAPE, "head_dim %d out of range", c->head_dim);
  if (c->num_pages < 1) return fail(KVQ_ERR_SHAPE, "num_pages must be >= 1 (got %d)", c->num_pages);
  return KVQ_OK;
}

kvq_status check_store(const kvq_cache* c, const kvq_store& s, bool is_v) {
  kvq_status st = check_store_fmt(s.fmt, c->head_dim, is_v);
  if (st != KVQ_OK) return st;
  const bool scaled = s.fmt != KVQ_FMT_F32;          // an F32 store has no scales
  if (!s.codes || (scaled && !s.scales))
    return fail(KVQ_ERR_NULL, "%s store has a NULL codes or scales pointer", is_v ? "V" : "K");
  if (((uintptr_t)s.codes & 15) || (scaled && ((uintptr_t)s.scales & 15)))
    return fail(KVQ_ERR_SHAPE, "%s store slabs must be 16-byte aligned", is_v ? "V" : "K");
  return KVQ_OK;
}

kvq_status check_pages(const kvq_pages* p) {
  if (!p) return fail(KVQ_ERR_NULL, "pages descriptor is NULL");
  if (!p->block_table || !p->seq_lens) return fail(KVQ_ERR_NULL, "block_table or seq_lens is NULL");
  if (p->batch < 1 || p->batch > 65535) return fail(KVQ_ERR_SHAPE, "batch %d out of range [1, 65535]", p->batch);
  if (p->max_pages < 1) return fail(KVQ_ERR_SHAPE, "max_pages must be >= 1 (got %d)", p->max_pages);
  if ((long)p->max_pages * KVQ_PAGE_SIZE > (1L << 30)) return fail(KVQ_ERR_SHAPE, "max_pages %d too large", p->max_pages);
  return KVQ_OK;
}

kvq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVQ_OK;
  return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Rows per KV head for decode: builds head_off / head_list from an explicit or default map.
kvq_status build_head_lists(int hq, int hkv, const int32_t* head_map, int16_t* off, int16_t* list, int* max_g) {
  if (hq < 1 || hq > KVQ_MAX_Q_HEADS) return fail(KVQ_ERR_SHAPE, "n_q_heads %d out of range [1, %d]", hq, KVQ_MAX_Q_HEADS);
  std::vector<int> m(hq);
  if (head_map) {
    for (int h = 0; h < hq; ++h) {
      if (head_map[h] < 0 || head_map[h] >= hkv)
        return fail(KVQ_ERR_SHAPE, "head_map[%d] = %d outside [0, %d)", h, head_map[h], hkv);
      m[h] = head_map[h];
    }
  } else {
    if (hq % hkv) return fail(KVQ_ERR_SHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", hq, hkv);
    for (int h = 0; h < hq; ++h) m[h] = h / (hq / hkv);
  }
  int pos = 0;
  *max_g = 0;
  for (int j = 0; j < hkv; ++j) {
    off[j] = (int16_t)pos;
    int g = 0;
    for (int h = 0; h < hq; ++h)
      if (m[h] == j) { list[pos++] = (int16_t)h; ++g; }
    if (g > *max_g) *max_g = g;
  }
  off[hkv] = (int16_t)pos;
  // entries past the list are read (never used) for KV heads that serve no query head: keep them a
  // valid head index
  for (int i = pos; i < KVQ_MAX_Q_HEADS; ++i) list[i] = 0;
  return KVQ_OK;
}

}  // namespace

namespace {
// Scratch of kvq_decode_attn_noalloc: the split partials of one call, in device memory the library
// holds from module load until the process ends (one copy per GPU, at that GPU's own address).  Host
// code never passes the array's name to a kernel (on the host it is only a stand-in for the symbol):
// it takes each device's address once with hipGetSymbolAddress and uses that.
__device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// This device's address of the scratch array, looked up on the first call on each device (with that
// device current), then cached.
kvq_status noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVQ_ERR_HIP, "hipGetSymbolAddress of the decode scratch: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return KVQ_OK;
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> counts;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)counts.size() <= dev) counts.resize(dev + 1, 0);
  if (!counts[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

}  // namespace kvq

using namespace kvq;

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_last_error(void) { return g_err; }

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "null pointer";
    case KVQ_ERR_SHAPE: return "bad shape or size";
    case KVQ_ERR_UNSUPPORTED: return "unsupported format or geometry";
    case KVQ_ERR_WORKSPACE: return "workspace too small or misaligned";
    case KVQ_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int32_t kvq_cell_bytes(int32_t fmt, int32_t D, int32_t* code_bytes, int32_t* n_scales) {
  int cb = -1, ns = -1;
  if (fmt == KVQ_FMT_INT8_G64 && D > 0 && D % 64 == 0 && D <= KVQ_MAX_HEAD_DIM) { cb = D; ns = D / 64; }
  if (fmt == KVQ_FMT_Q4_0_H256 && D == 256) { cb = D / 2; ns = D / 32; }
  if (fmt == KVQ_FMT_ISO3 && D > 0 && D % 128 == 0 && D <= KVQ_MAX_HEAD_DIM) { cb = D / 128 * 48; ns = D / 128; }
  if (fmt == KVQ_FMT_F32 && D > 0 && D % 64 == 0 && D <= KVQ_MAX_HEAD_DIM) { cb = 4 * D; ns = 0; }
  if (fmt == KVQ_FMT_ISO4 && D > 0 && D % 128 == 0 && D <= KVQ_MAX_HEAD_DIM) { cb = D / 128 * 64; ns = D / 64; }
  if (cb < 0) return -1;
  if (code_bytes) *code_bytes = cb;
  if (n_scales) *n_scales = ns;
  return cb + 2 * ns;
}

kvq_status kvq_append(const kvq_cache* cache, const kvq_pages* pages, const void* k_new, const void* v_new,
                      const int32_t* tok_seq, const int32_t* tok_pos, int32_t n_tok, void* stream) {
  kvq_status st;
  if ((st = check_cache(cache)) != KVQ_OK) return st;
  if ((st = check_pages(pages)) != KVQ_OK) return st;
  if (n_tok < 0) return fail(KVQ_ERR_SHAPE, "n_tok must be >= 0 (got %d)", n_tok);
  if (k_new && (st = check_store(cache, cache->k, false)) != KVQ_OK) return st;
  if (v_new && (st = check_store(cache, cache->v, true)) != KVQ_OK) return st;
  if (n_tok == 0 || (!k_new && !v_new)) return KVQ_OK;
  if (!tok_seq || !tok_pos) return fail(KVQ_ERR_NULL, "tok_seq or tok_pos is NULL");
  if ((long)n_tok * cache->n_kv_heads > (1L << 31) / 4) return fail(KVQ_ERR_SHAPE, "n_tok %d too large", n_tok);
  AppendArgs a{tok_seq, tok_pos, pages->block_table, n_tok, pages->batch, pages->max_pages, cache->num_pages,
               cache->n_kv_heads, nullptr, nullptr};
  hipError_t e = launch_append_kv(cache->k.fmt, static_cast<const uint16_t*>(k_new),
                                  static_cast<uint8_t*>(cache->k.codes), static_cast<uint16_t*>(cache->k.scales),
                                  cache->v.fmt, static_cast<const uint16_t*>(v_new),
                                  static_cast<uint8_t*>(cache->v.codes), static_cast<uint16_t*>(cache->v.scales),
                                  cache->head_dim, cache->iso_quat, a, static_cast<hipStream_t>(stream));
  return hip_status(e, "append launch");
}

kvq_status kvq_dequant_gather(const kvq_cache* cache, const kvq_pages* pages, int32_t which, int32_t seq,
                              int32_t start, int32_t count, int32_t out_dtype, int32_t unrotate, void* out,
                              void* stream) {
  kvq_status st;
  if ((st = check_cache(cache)) != KVQ_OK) return st;
  if ((st = check_pages(pages)) != KVQ_OK) return st;
  if (which != 0 && which != 1) return fail(KVQ_ERR_SHAPE, "which must be 0 (K) or 1 (V), got %d", which);
  const kvq_store& sto = which ? cache->v : cache->k;
  if ((st = check_store(cache, sto, which == 1)) != KVQ_OK) return st;
  if (seq < 0 || seq >= pages->batch) return fail(KVQ_ERR_SHAPE, "seq %d outside [0, %d)", seq, pages->batch);
  if (start < 0 || count < 0 || (long)start + count > (long)pages->max_pages * KVQ_PAGE_SIZE)
    return fail(KVQ_ERR_SHAPE, "cells [%d, %d+%d) outside the page table's %d cells", start, start, count,
                pages->max_pages * KVQ_PAGE_SIZE);
  if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_F16 && out_dtype != KVQ_OUT_BF16)
    return fail(KVQ_ERR_SHAPE, "unknown out_dtype %d", out_dtype);
  if (count == 0) return KVQ_OK;
  if (!out) return fail(KVQ_ERR_NULL, "out is NULL");
  if ((uintptr_t)out & 15) return fail(KVQ_ERR_SHAPE, "out must be 16-byte aligned");
  GatherArgs g{pages->block_table, pages->max_pages, cache->num_pages, cache->n_kv_heads, seq, start, count};
  hipError_t e = launch_gather(sto.fmt, which == 1, static_cast<const uint8_t*>(sto.codes),
                               static_cast<const uint16_t*>(sto.scales), cache->head_dim, cache->iso_quat, g,
                               out_dtype, unrotate != 0, out, static_cast<hipStream_t>(stream));
  return hip_status(e, "gather launch");
}

static kvq_status decode_setup(const kvq_cache* cache, int32_t batch, int32_t max_pages, int32_t n_q,
                               int32_t n_q_heads, const int32_t* head_map, DecodeArgs* a, DecodePlan* plan) {
  kvq_status st;
  if ((st = check_cache(cache)) != KVQ_OK) return st;
  if ((st = check_store_fmt(cache->k.fmt, cache->head_dim, false)) != KVQ_OK) return st;
  if ((st = check_store_fmt(cache->v.fmt, cache->head_dim, true)) != KVQ_OK) return st;
  const bool iso = (cache->k.fmt == KVQ_FMT_ISO3 && cache->v.fmt == KVQ_FMT_ISO3) ||
                   (cache->k.fmt == KVQ_FMT_ISO4 && cache->v.fmt == KVQ_FMT_ISO4);
  const bool q4k = cache->k.fmt == KVQ_FMT_Q4_0_H256;
  const bool kf = cache->k.fmt == KVQ_FMT_F32, vf = cache->v.fmt == KVQ_FMT_F32;
  const bool f32 = kf || vf;      // single-store modes (and F32 for both)
  if (f32 && ((!kf && cache->k.fmt != KVQ_FMT_INT8_G64) || (!vf && cache->v.fmt != KVQ_FMT_INT8_G64)))
    return fail(KVQ_ERR_UNSUPPORTED, "decode with an F32 store needs the other store F32 or INT8_G64 (got formats %d / %d)",
                cache->k.fmt, cache->v.fmt);
  if (q4k && cache->v.fmt != KVQ_FMT_Q4_0_H256)
    return fail(KVQ_ERR_UNSUPPORTED, "decode over a Q4_0_H256 K store needs a Q4_0_H256 V store (got %d)",
                cache->v.fmt);
  if (!iso && !q4k && !f32 && cache->k.fmt != KVQ_FMT_INT8_G64)
    return fail(KVQ_ERR_UNSUPPORTED,
                "decode needs an INT8_G64 or Q4_0_H256 K store, or ISO3 / ISO4 K and V stores (got formats %d / %d)",
                cache->k.fmt, cache->v.fmt);
  if (!iso && (cache->k.fmt == KVQ_FMT_ISO3 || cache->k.fmt == KVQ_FMT_ISO4 || cache->v.fmt == KVQ_FMT_ISO3 ||
               cache->v.fmt == KVQ_FMT_ISO4))
    return fail(KVQ_ERR_UNSUPPORTED, "decode over ISO3 / ISO4 stores needs K and V of the same ISO format (got %d / %d)",
                cache->k.fmt, cache->v.fmt);
  const int D = cache->head_dim;
  if (iso && D != 128 && D != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "ISO3 / ISO4 decode supports head_dim 128 or 256 (got %d)", D);
  if (f32 && D != 128 && D != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "decode with an F32 store supports head_dim 128 or 256 (got %d)", D);
  if (D != 64 && D != 128 && D != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "decode supports head_dim 64, 128 or 256 (got %d)", D);
  if (batch < 1 || batch > 65535) return fail(KVQ_ERR_SHAPE, "batch %d out of range", batch);
  if (max_pages < 1) return fail(KVQ_ERR_SHAPE, "max_pages must be >= 1");
  if (n_q < 1) return fail(KVQ_ERR_SHAPE, "n_q must be >= 1 (got %d)", n_q);
  int max_g = 0;
  if ((st = build_head_lists(n_q_heads, cache->n_kv_heads, head_map, a->head_off, a->head_list, &max_g)) != KVQ_OK)
    return st;
  if ((long)n_q * max_g > KVQ_MAX_ROWS_PER_KV_HEAD)
    return fail(KVQ_ERR_UNSUPPORTED, "n_q * (query heads per KV head) = %d exceeds %d", n_q * max_g,
                KVQ_MAX_ROWS_PER_KV_HEAD);
  if (iso && (long)n_q * max_g > kIsoDecodeMaxRows)
    return fail(KVQ_ERR_UNSUPPORTED, "ISO3 / ISO4 decode: n_q * (query heads per KV head) = %d exceeds %d", n_q * max_g,
                kIsoDecodeMaxRows);
  if (q4k && (long)n_q * max_g > kQ4DecodeMaxRows)
    return fail(KVQ_ERR_UNSUPPORTED, "q4_0 K decode: n_q * (query heads per KV head) = %d exceeds %d", n_q * max_g,
                kQ4DecodeMaxRows);
  *plan = iso   ? plan_decode_iso(D, cache->n_kv_heads, batch, max_pages, n_q * max_g)
          : q4k ? plan_decode_q4(cache->n_kv_heads, batch, max_pages, n_q * max_g)
          : f32 ? plan_decode_f32(D, cache->n_kv_heads, batch, max_pages, n_q * max_g)
                : plan_decode(cache->v.fmt, D, cache->n_kv_heads, batch, max_pages, n_q * max_g);
  if (plan->n_splits > decode_max_splits())
    return fail(KVQ_ERR_UNSUPPORTED, "max_pages %d needs %d context splits; decode supports %d", max_pages,
                plan->n_splits, decode_max_splits());
  return KVQ_OK;
}

size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t max_pages, int32_t n_q,
                                  int32_t n_q_heads, const int32_t* head_map) {
  DecodeArgs a;
  DecodePlan plan;
  if (decode_setup(cache, batch, max_pages, n_q, n_q_heads, head_map, &a, &plan) != KVQ_OK) return 0;
  return plan.part_bytes;
}

// Validates every decode argument but the workspace and fills the kernel arguments and the launch plan
// (plan.part_bytes: the split partials the workspace must hold).
static kvq_status decode_prepare(const kvq_cache* cache, const kvq_pages* pages, const void* k_new,
                                 const void* v_new, const void* q, int32_t n_q, int32_t n_q_heads,
                                 const int32_t* q_lens, const int32_t* head_map, float sm_scale, float* out,
                                 DecodeArgs& a, DecodePlan& plan) {
  kvq_status st;
  if ((st = check_pages(pages)) != KVQ_OK) return st;
  if ((st = decode_setup(cache, pages->batch, pages->max_pages, n_q, n_q_heads, head_map, &a, &plan)) != KVQ_OK)
    return st;
  if ((st = check_store(cache, cache->k, false)) != KVQ_OK) return st;
  if ((st = check_store(cache, cache->v, true)) != KVQ_OK) return st;
  if (!q || !out) return fail(KVQ_ERR_NULL, "q or out is NULL");
  if (((uintptr_t)q & 15) || ((uintptr_t)out & 15)) return fail(KVQ_ERR_SHAPE, "q and out must be 16-byte aligned");
  if (!(sm_scale == sm_scale)) return fail(KVQ_ERR_SHAPE, "sm_scale is NaN");
  a.k_codes = static_cast<const uint8_t*>(cache->k.codes);
  a.k_scales = static_cast<const uint16_t*>(cache->k.scales);
  a.v_codes = static_cast<const uint8_t*>(cache->v.codes);
  a.v_scales = static_cast<const uint16_t*>(cache->v.scales);
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.q_lens = q_lens;
  a.seq_lens = pages->seq_lens;
  a.bt = pages->block_table;
  a.part = nullptr;
  a.out = out;
  a.hkv = cache->n_kv_heads;
  a.num_pages = cache->num_pages;
  a.max_pages = pages->max_pages;
  a.batch = pages->batch;
  a.n_q = n_q;
  a.n_q_heads = n_q_heads;
  a.pages_per_split = plan.pages_per_split;
  a.n_splits = plan.n_splits;
  a.row_groups = plan.row_groups;
  a.row_alloc = 8 * plan.row_groups;
  a.scale_log2 = sm_scale * 1.44269504088896340736f;
  for (int e = 0; e < 4; ++e) a.quat[e] = cache->iso_quat[e];
  // the default grouping (explicit maps that coincide with it included) lets kernels skip the lists
  a.g_uniform = n_q_heads % cache->n_kv_heads == 0 ? n_q_heads / cache->n_kv_heads : 0;
  for (int h = 0; h < n_q_heads && a.g_uniform; ++h)
    if (a.head_list[h] != h || (h % a.g_uniform == 0 && a.head_off[h / a.g_uniform] != h)) a.g_uniform = 0;
  return KVQ_OK;
}

// Launches the decode kernels of a prepared call with its split partials at `part`.
static kvq_status decode_launch(const kvq_cache* cache, const DecodePlan& plan, DecodeArgs& a, void* part,
                                void* stream) {
  a.part = static_cast<float*>(part);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (cache->k.fmt == KVQ_FMT_ISO3 || cache->k.fmt == KVQ_FMT_ISO4)
    return hip_status(launch_decode_iso(cache->k.fmt == KVQ_FMT_ISO4 ? 4 : 3, cache->head_dim, plan, a, hs),
                      "decode launch");
  if (cache->k.fmt == KVQ_FMT_Q4_0_H256) return hip_status(launch_decode_q4(plan, a, hs), "decode launch");
  if (cache->k.fmt == KVQ_FMT_F32 || cache->v.fmt == KVQ_FMT_F32)
    return hip_status(launch_decode_f32(cache->k.fmt == KVQ_FMT_F32, cache->v.fmt == KVQ_FMT_F32, cache->head_dim,
                                        plan, a, hs),
                      "decode launch");
  return hip_status(launch_decode(cache->v.fmt, cache->head_dim, plan, a, hs), "decode launch");
}

static kvq_status decode_impl(const kvq_cache* cache, const kvq_pages* pages, const void* k_new, const void* v_new,
                              const void* q, int32_t n_q, int32_t n_q_heads, const int32_t* q_lens,
                              const int32_t* head_map, float sm_scale, float* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  DecodeArgs a;
  DecodePlan plan;
  kvq_status st = decode_prepare(cache, pages, k_new, v_new, q, n_q, n_q_heads, q_lens, head_map, sm_scale, out, a,
                                 plan);
  if (st != KVQ_OK) return st;
  if (!workspace) return fail(KVQ_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", plan.part_bytes);
  if ((uintptr_t)workspace & 255) return fail(KVQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan.part_bytes)
    return fail(KVQ_ERR_WORKSPACE, "workspace has %zu bytes, decode needs %zu", workspace_bytes, plan.part_bytes);
  return decode_launch(cache, plan, a, workspace, stream);
}

kvq_status kvq_decode_attn(const kvq_cache* cache, const kvq_pages* pages, const void* q, int32_t n_q,
                           int32_t n_q_heads, const int32_t* q_lens, const int32_t* head_map, float sm_scale,
                           float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(cache, pages, nullptr, nullptr, q, n_q, n_q_heads, q_lens, head_map, sm_scale, out, workspace,
                     workspace_bytes, stream);
}

kvq_status kvq_decode_attn_noalloc(const kvq_cache* cache, const kvq_pages* pages, const void* q, int32_t n_q,
                                   int32_t n_q_heads, const int32_t* q_lens, const int32_t* head_map,
                                   float sm_scale, float* out, void* stream) {
  DecodeArgs a;
  DecodePlan plan;
  kvq_status st = decode_prepare(cache, pages, nullptr, nullptr, q, n_q, n_q_heads, q_lens, head_map, sm_scale, out,
                                 a, plan);
  if (st != KVQ_OK) return st;
  if (plan.part_bytes > (size_t)KVQ_NOALLOC_SCRATCH_BYTES)
    return fail(KVQ_ERR_WORKSPACE,
                "kvq_decode_attn_noalloc: this call's split partials need %zu bytes, more than the library's "
                "%zu-byte scratch (use kvq_decode_attn with a workspace)",
                plan.part_bytes, (size_t)KVQ_NOALLOC_SCRATCH_BYTES);
  void* part = nullptr;
  if ((st = noalloc_scratch(&part)) != KVQ_OK) return st;
  return decode_launch(cache, plan, a, part, stream);
}

kvq_status kvq_decode_attn_append(const kvq_cache* cache, const kvq_pages* pages, const void* k_new,
                                  const void* v_new, const void* q, int32_t n_q, int32_t n_q_heads,
                                  const int32_t* q_lens, const int32_t* head_map, float sm_scale, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  kvq_status st;
  if ((st = check_cache(cache)) != KVQ_OK) return st;
  const int fk = cache->k.fmt, fv = cache->v.fmt;
  const bool i8f32 = (fk == KVQ_FMT_INT8_G64 || fk == KVQ_FMT_F32) && (fv == KVQ_FMT_INT8_G64 || fv == KVQ_FMT_F32);
  const bool k8v4 = fk == KVQ_FMT_INT8_G64 && fv == KVQ_FMT_Q4_0_H256 && cache->head_dim == 256;
  if (!i8f32 && !k8v4)
    return fail(KVQ_ERR_UNSUPPORTED,
                "fused append + decode needs INT8_G64 or F32 K and V stores, or INT8_G64 K with a (head_dim 256) "
                "Q4_0_H256 V store (got formats %d / %d)",
                fk, fv);
  if (n_q < 1 || n_q > kDecodeMaxFused)
    return fail(KVQ_ERR_UNSUPPORTED, "fused append + decode takes 1..%d new tokens per sequence (got %d)",
                kDecodeMaxFused, n_q);
  if (!k_new || !v_new) return fail(KVQ_ERR_NULL, "k_new or v_new is NULL");
  if (((uintptr_t)k_new & 15) || ((uintptr_t)v_new & 15))
    return fail(KVQ_ERR_SHAPE, "k_new and v_new must be 16-byte aligned");
  return decode_impl(cache, pages, k_new, v_new, q, n_q, n_q_heads, q_lens, head_map, sm_scale, out, workspace,
                     workspace_bytes, stream);
}

static kvq_status extend_setup(const kvq_cache* cache, int32_t batch, int32_t max_pages, int32_t n_new,
                               int32_t max_new, int32_t n_q_heads, const int32_t* head_map, ExtendArgs* a,
                               int* tiles) {
  kvq_status st;
  if ((st = check_cache(cache)) != KVQ_OK) return st;
  if ((st = check_store_fmt(cache->k.fmt, cache->head_dim, false)) != KVQ_OK) return st;
  if ((st = check_store_fmt(cache->v.fmt, cache->head_dim, true)) != KVQ_OK) return st;
  const bool iso3 = cache->k.fmt == KVQ_FMT_ISO3 && cache->v.fmt == KVQ_FMT_ISO3;
  const bool int8 = cache->k.fmt == KVQ_FMT_INT8_G64 && cache->v.fmt == KVQ_FMT_INT8_G64;
  if (!iso3 && !int8)
    return fail(KVQ_ERR_UNSUPPORTED, "extend attention needs ISO3 or INT8_G64 K and V stores (got formats %d / %d)",
                cache->k.fmt, cache->v.fmt);
  a->int8 = int8 ? 1 : 0;
  if (cache->head_dim != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "extend attention supports head_dim 128 (got %d)", cache->head_dim);
  if (batch < 1 || batch > 65535) return fail(KVQ_ERR_SHAPE, "batch %d out of range", batch);
  if (max_pages < 1) return fail(KVQ_ERR_SHAPE, "max_pages must be >= 1");
  if (n_new < 0) return fail(KVQ_ERR_SHAPE, "n_new must be >= 0 (got %d)", n_new);
  if (max_new < 0 || max_new > n_new)
    return fail(KVQ_ERR_SHAPE, "max_new %d outside [0, n_new = %d]", max_new, n_new);
  int max_g = 0;
  if ((st = build_head_lists(n_q_heads, cache->n_kv_heads, head_map, a->head_off, a->head_list, &max_g)) != KVQ_OK)
    return st;
  if (max_g > 32)
    return fail(KVQ_ERR_UNSUPPORTED, "extend supports up to 32 query heads per KV head (got %d)", max_g);
  int g_pad = 1;
  while (g_pad < max_g) g_pad <<= 1;
  a->g_pad = g_pad;
  const int per_block = extend_tokens_per_block(g_pad);
  *tiles = (max_new + per_block - 1) / per_block;
  if ((long)*tiles * cache->n_kv_heads > 0x7fffffffL) return fail(KVQ_ERR_SHAPE, "n_new %d too large", n_new);
  if ((long)n_new * (n_q_heads > cache->n_kv_heads ? n_q_heads : cache->n_kv_heads) * cache->head_dim > 0x7fffffffL)
    return fail(KVQ_ERR_SHAPE, "n_new %d too large", n_new);
  a->pt_max = (int)(((long)max_pages * KVQ_PAGE_SIZE + 63) / 64);
  a->nt_max = (max_new + 63) / 64;
  if ((long)a->pt_max + a->nt_max > 0x7fffffffL) return fail(KVQ_ERR_SHAPE, "too many tiles");
  return KVQ_OK;
}

size_t kvq_extend_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t max_pages, int32_t n_new,
                                  int32_t max_new, int32_t n_q_heads) {
  (void)n_q_heads;   // the tile images depend on the KV heads only
  if (check_cache(cache) != KVQ_OK) return 0;
  const bool iso3 = cache->k.fmt == KVQ_FMT_ISO3 && cache->v.fmt == KVQ_FMT_ISO3;
  const bool int8 = cache->k.fmt == KVQ_FMT_INT8_G64 && cache->v.fmt == KVQ_FMT_INT8_G64;
  if ((!iso3 && !int8) || cache->head_dim != 128) return 0;
  if (batch < 1 || batch > 65535 || max_pages < 1 || n_new < 0 || max_new < 0 || max_new > n_new) return 0;
  const int pt_max = (int)(((long)max_pages * KVQ_PAGE_SIZE + 63) / 64), nt_max = (max_new + 63) / 64;
  return extend_workspace_bytes(batch, cache->n_kv_heads, pt_max, nt_max);
}

kvq_status kvq_extend_attn(const kvq_cache* cache, const kvq_pages* pages, const void* q, const void* k_new,
                           const void* v_new, const int32_t* cu_new, int32_t n_new, int32_t max_new,
                           int32_t n_q_heads, const int32_t* head_map, float sm_scale, float* out,
                           int32_t pack_after, void* workspace, size_t workspace_bytes, void* stream) {
  kvq_status st;
  if ((st = check_pages(pages)) != KVQ_OK) return st;
  ExtendArgs a;
  int tiles = 0;
  if ((st = extend_setup(cache, pages->batch, pages->max_pages, n_new, max_new, n_q_heads, head_map, &a, &tiles)) !=
      KVQ_OK)
    return st;
  if ((st = check_store(cache, cache->k, false)) != KVQ_OK) return st;
  if ((st = check_store(cache, cache->v, true)) != KVQ_OK) return st;
  if (!(sm_scale == sm_scale)) return fail(KVQ_ERR_SHAPE, "sm_scale is NaN");
  if (n_new == 0) return KVQ_OK;
  if (!q || !k_new || !v_new || !cu_new || !out) return fail(KVQ_ERR_NULL, "q, k_new, v_new, cu_new or out is NULL");
  if (((uintptr_t)q & 15) || ((uintptr_t)k_new & 15) || ((uintptr_t)v_new & 15) || ((uintptr_t)out & 15))
    return fail(KVQ_ERR_SHAPE, "q, k_new, v_new and out must be 16-byte aligned");
  const size_t need = extend_workspace_bytes(pages->batch, cache->n_kv_heads, a.pt_max, a.nt_max);
  if (tiles > 0) {
    if (!workspace) return fail(KVQ_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if ((uintptr_t)workspace & 255) return fail(KVQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(KVQ_ERR_WORKSPACE, "workspace has %zu bytes, extend needs %zu", workspace_bytes, need);
  }
  a.ws = static_cast<uint8_t*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  a.k_codes = static_cast<const uint8_t*>(cache->k.codes);
  a.k_norms = static_cast<const uint16_t*>(cache->k.scales);
  a.v_codes = static_cast<const uint8_t*>(cache->v.codes);
  a.v_norms = static_cast<const uint16_t*>(cache->v.scales);
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.cu_new = cu_new;
  a.prefix_lens = pages->seq_lens;
  a.bt = pages->block_table;
  a.out = out;
  a.hkv = cache->n_kv_heads;
  a.num_pages = cache->num_pages;
  a.max_pages = pages->max_pages;
  a.batch = pages->batch;
  a.n_new = n_new;
  a.n_q_heads = n_q_heads;
  for (int i = 0; i < 4; ++i) a.quat[i] = a.int8 ? (i == 0 ? 1.0f : 0.0f) : cache->iso_quat[i];
  a.scale_log2 = sm_scale * 1.44269504088896340736f;
  a.q_scale = a.int8 ? 1.0f : a.scale_log2 / extend_level_scale();   // int8: the scale goes to the scores
  a.g_uniform = n_q_heads % cache->n_kv_heads == 0 ? n_q_heads / cache->n_kv_heads : 0;
  for (int h = 0; h < n_q_heads && a.g_uniform; ++h)
    if (a.head_list[h] != h || (h % a.g_uniform == 0 && a.head_off[h / a.g_uniform] != h)) a.g_uniform = 0;
  if (tiles > 0 && (st = hip_status(launch_extend(a, tiles, s), "extend launch")) != KVQ_OK) return st;
  if (!pack_after) return KVQ_OK;
  // deferred packing: token i of sequence b goes to cell seq_lens[b] + (i - cu_new[b])
  AppendArgs ap{nullptr, nullptr, pages->block_table, n_new, pages->batch, pages->max_pages, cache->num_pages,
                cache->n_kv_heads, cu_new, pages->seq_lens};
  return hip_status(launch_append_kv(cache->k.fmt, static_cast<const uint16_t*>(k_new),
                                     static_cast<uint8_t*>(cache->k.codes), static_cast<uint16_t*>(cache->k.scales),
                                     cache->v.fmt, static_cast<const uint16_t*>(v_new),
                                     static_cast<uint8_t*>(cache->v.codes), static_cast<uint16_t*>(cache->v.scales),
                                     cache->head_dim, cache->iso_quat, ap, s),
                    "extend pack launch");
}

}  // extern "C"
