/*
 * kvq.h -- C ABI of the quantized paged KV-cache library (MI355X / gfx950).
 *
 * The hot path: new bf16 K/V tokens are quantised as they are written into a
 * paged cache of packed cells (quantize-on-write), and attention then reads the
 * codes and their FP16 scales page by page and dequantises them inside the
 * attention loop.
 *
 * Sources (the pages this library implements):
 *   [FT398]  FreeToken PR #398, "feat(kvcache): add ISO3/ISO4 KV-cache quantization
 *            (--kv-cache-iso)" -- sections "What", "Correctness", "Caveats".
 *   [ST2698] strata PR #2698, "qwen35/q36: --kv - int8 K/V caches (codes + a FP16
 *            scale per 64 values)" -- sections "What it does", "Not in this PR".
 *   [ST120]  strata PR #120, "--kv k8v4: hybrid KV cache -- INT8 K + Hadamard-rotated
 *            Q4_0 V (816 B/cell)" -- sections "What", "How", "Tests".
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every buffer (cache slabs, page tables, lengths,
 *     q/k/v, outputs, workspaces).  The library allocates nothing and keeps no
 *     per-call state; it only caches per-device properties.  The one exception is
 *     kvq_decode_attn_noalloc's scratch, a fixed device array of the library's own
 *     (see there).
 *   - Pointers marked "device" are HIP device pointers; "host" pointers are read
 *     during the call only.  Nothing is retained after a call returns.
 *   - Execution: every call enqueues its kernels on `stream` (a hipStream_t; NULL =
 *     the legacy default stream) and returns without synchronising.
 *   - Errors: arguments are validated on the host BEFORE any HIP call; on failure
 *     the call returns a status, enqueues nothing, and kvq_last_error() gives a
 *     thread-local message.  Unsupported combinations are refused, never silently
 *     downgraded (the pages refuse unsupported modes with a message at config
 *     time: [ST2698] "What it does"/"Not in this PR", [FT398] "Caveats").
 *     A failed launch returns KVQ_ERR_HIP.
 *   - Device-side data (page-table entries, lengths, token positions) cannot be
 *     checked without a synchronisation.  Kernels clamp page ids to
 *     [0, num_pages) and lengths to [0, max_pages * page_size), so bad device
 *     data yields wrong values but never an out-of-bounds access.
 *
 * Cache layout (one "store" = the K side or the V side)
 *   scales : float16 [num_pages][n_kv_heads][page_size][n_scales]
 *   codes  : uint8 [num_pages][n_kv_heads] tiles of page_size * code_bytes bytes.  Inside a tile,
 *            code byte c (0 <= c < code_bytes) of the cell in slot t (0 <= t < 16) sits at
 *     INT8_G64 K store            ((c / 16) * 16 + t) * 16 + c % 16
 *                                 (16-byte chunks, chunk-major: one wave load of 16 bytes per
 *                                 lane covers a contiguous kilobyte of chunks 0..3 of 16 slots);
 *     INT8_G64 / Q4_0_H256 V store (((c / 64) * 16 + c % 16) * 4 + t / 4) * 16
 *                                 + ((c / 16) % 4) * 4 + t % 4
 *                                 (attention contracts V over tokens: 4 consecutive slots of one
 *                                 code byte form a 32-bit word, and the words of code bytes c,
 *                                 c+16, c+32, c+48 form one 16-byte unit);
 *     Q4_0_H256 K store           (((c / 64) * 4 + (c / 4) % 4) * 16 + t) * 16
 *                                 + ((c / 16) % 4) * 4 + c % 4
 *                                 (attention contracts K over head_dim in 32-value scale groups:
 *                                 one 16-byte unit holds, for slot t, bytes 4w .. 4w+3 of four
 *                                 consecutive groups; a wave load covers a contiguous kilobyte);
 *     ISO3 / ISO4 store (K or V)  t * code_bytes + c   (token-major).
 *     F32 K store                 as INT8_G64 K (16-byte chunks of 4 values, chunk-major)
 *     F32 V store                 ((c / 4) * 16 + t) * 4 + c % 4
 *                                 (head_dim-major: the 16 slots' values of one head_dim
 *                                 index are 64 contiguous bytes, so 4 slots form 16 bytes).
 *   An F32 store has no scales (its scales pointer may be NULL) and holds the values
 *   themselves, which must be finite like the scales.
 *   Every fp16 scale in the slabs must be finite, including those of slots no append has
 *   written yet (zero-initialise new slabs): attention weighs cells past a sequence's length
 *   by exact zeros, which a NaN or infinite scale would turn into NaN.
 *   Logical token j of sequence b is the cell (page = block_table[b][j / page_size],
 *   slot = j % page_size).  Codes and scales are separate slabs ([ST2698] "What it
 *   does"); the page table may be any mapping ([ST120] "Tests" checks a
 *   non-identity one).  page_size must be 16.
 *
 * Formats (code_bytes / n_scales per (token, KV head) cell of one store, D = head_dim)
 *   KVQ_FMT_INT8_G64  D / D/64.  int8 two's-complement codes; scale = fp16(absmax/127)
 *                     of each 64 consecutive values; code = clamp(rint(x / (absmax/127)),
 *                     -127, 127) with the binary32 divisor, ties to even; an all-zero
 *                     group stores scale +0 and codes 0.  D % 64 == 0, D <= 512.
 *                     ([ST2698] "What it does"; ties-to-even: [ST120] "Tests".)
 *   KVQ_FMT_Q4_0_H256 D/2 / D/32.  K or V.  The vector is rotated by the orthonormal
 *                     Walsh-Hadamard transform H = H_256/16 (Sylvester order; binary32
 *                     butterflies of span 1, 2, ..., 128, then x 1/16), then q4_0: per
 *                     32 values d = m / -8 with m the first value of largest magnitude,
 *                     stored fp16; code = clamp(rint(z / d) + 8, 0, 15); byte j holds
 *                     code 2j (low nibble) and 2j+1 (high nibble); a zero block stores
 *                     d = +0, codes 8.  Values stay in the rotated basis; attention
 *                     rotates its output back, and with a Q4_0_H256 K store rotates q
 *                     (<q, k> = <Hq, Hk>).  D == 256.
 *                     ([ST120] "What"/"How"; [ST2698] "Not in this PR".)
 *   KVQ_FMT_ISO3      D/128*48 / D/128.  Per 128 values: n = ||x|| (binary32 pairwise
 *                     halving sum of squares, then sqrt); u = x / n; each 4-group
 *                     (w,x,y,z) is left-multiplied by the unit quaternion iso_quat; each
 *                     value takes the index of the nearest of the 8 Lloyd-Max centroids
 *                     {+-0.2451, +-0.7560, +-1.3440, +-2.1520}/sqrt(128) (binary32
 *                     distances, lowest index on ties); the stored norm is
 *                     fp16(n / ||chosen centroids||).  Codes are a little-endian 3-bit
 *                     stream (code i in bits 3i..3i+2, 8 codes per 3 bytes).
 *                     Dequant: conj(iso_quat) * centroid group, times the norm.
 *                     D % 128 == 0, D <= 512.  ([FT398] "What".)
 *   KVQ_FMT_ISO4      D/128*64 / 2*D/128.  ISO3's steps with the sixteen levels of the 16-level
 *                     Lloyd-Max quantiser of a standard normal variable
 *                     {+-0.1284, +-0.3880, +-0.6568, +-0.9423, +-1.2562, +-1.6180, +-2.0690,
 *                     +-2.7326}/sqrt(128) (the page gives only the size: 4.25 bits per value,
 *                     68 B per 128-value block); 4-bit codes, code i in bits 4i..4i+3 (byte j:
 *                     code 2j in the low nibble); the corrected norm n / ||chosen centroids||
 *                     is kept in binary32, its bytes in the block's two 16-bit scale slots
 *                     (low half first).  D % 128 == 0, D <= 512.  ([FT398] "What".)
 *   KVQ_FMT_F32       4*D / 0.  Unquantised: value d of the cell as binary32 in code bytes
 *                     4d .. 4d+3 (little-endian); written from bf16 inputs, the bf16 value
 *                     exactly.  With an INT8_G64 store for the other side this is the
 *                     single-store mode k8v32 (K int8, V FP32) or k32v8 (K FP32, V int8).
 *                     D % 64 == 0, D <= 512.  ([ST2698] intro: FP32 caches of 2 KiB per
 *                     cell per store; "What it does": `k8v32` / `k32v8` quantise one store.)
 *
 * Arithmetic contract of the encoders and of kvq_dequant_gather (F32 output):
 * binary32, one rounding per operation (no fused multiply-add), correctly rounded
 * division and square root, round-half-even, binary16 subnormals kept.  Under it
 * the library's codes, scales and norms are a pure function of the inputs.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 1
#define KVQ_PAGE_SIZE 16
#define KVQ_MAX_HEAD_DIM 512
#define KVQ_MAX_Q_HEADS 256
#define KVQ_MAX_ROWS_PER_KV_HEAD 32   /* n_q * (query heads of one KV head) in decode */

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,         /* a required pointer is NULL */
  KVQ_ERR_SHAPE = 2,        /* a count or size is out of range or inconsistent */
  KVQ_ERR_UNSUPPORTED = 3,  /* a format / head_dim / path combination the library refuses */
  KVQ_ERR_WORKSPACE = 4,    /* workspace missing, too small or misaligned */
  KVQ_ERR_HIP = 5           /* a HIP runtime call or a kernel launch failed */
} kvq_status;

typedef enum {
  KVQ_FMT_INT8_G64 = 1,
  KVQ_FMT_Q4_0_H256 = 2,
  KVQ_FMT_ISO3 = 3,
  KVQ_FMT_F32 = 4,
  KVQ_FMT_ISO4 = 5
} kvq_fmt;

typedef enum { KVQ_OUT_F32 = 0, KVQ_OUT_F16 = 1, KVQ_OUT_BF16 = 2 } kvq_out_dtype;

/* One store.  Both pointers are device pointers, 16-byte aligned; the byte order of
 * `codes` follows from the store's role and format (see "Cache layout"). */
typedef struct {
  int32_t fmt;     /* kvq_fmt */
  void* codes;     /* uint8 [num_pages][n_kv_heads] tiles of page_size * code_bytes */
  void* scales;    /* fp16  [num_pages][n_kv_heads][page_size][n_scales]; unused (may be NULL)
                      for an F32 store */
} kvq_store;

/* The cache: geometry plus the K and V stores ([ST120] "How": separate K/V pointers). */
typedef struct {
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t page_size;      /* must be KVQ_PAGE_SIZE */
  int32_t num_pages;
  kvq_store k;
  kvq_store v;
  float iso_quat[4];      /* (w, x, y, z) used by ISO3 stores; ignored otherwise */
} kvq_cache;

/* Page table and lengths of a batch of sequences (device pointers). */
typedef struct {
  const int32_t* block_table;  /* int32 [batch][max_pages] */
  const int32_t* seq_lens;     /* int32 [batch]: cells of each sequence that attention reads */
  int32_t batch;
  int32_t max_pages;
} kvq_pages;

/* Quantize-on-write ([FT398] section What: a decode step stores each new token already
 * quantised; [ST2698] section What it does).  Encodes n_tok bf16 vectors per store and writes each into
 * the cell of (tok_seq[i], tok_pos[i]) through pages->block_table.  seq_lens is not read
 * or changed: the caller advances it.
 *   k_new, v_new : device bf16 [n_tok][n_kv_heads][head_dim]; either may be NULL to skip
 *                  that store.
 *   tok_seq      : device int32 [n_tok], sequence index in [0, batch)
 *   tok_pos      : device int32 [n_tok], logical position in [0, max_pages*page_size)
 * Out-of-range device indices are clamped (see the conventions above).  Two tokens
 * writing the same cell in one call race.  n_tok == 0 is a no-op. */
kvq_status kvq_append(const kvq_cache* cache, const kvq_pages* pages,
                      const void* k_new, const void* v_new,
                      const int32_t* tok_seq, const int32_t* tok_pos,
                      int32_t n_tok, void* stream);

/* Decode / MTP-verify attention over the packed cache, dequantising K and V inside the
 * attention loop ([ST2698] "What it does": decode and verify windows dequantise on the
 * fly; [ST120] "How"/"Tests": per-query step arrays for verify; k8v4 rotates V and the
 * output only, never q).  Split-K over the context with a log-sum-exp combine.
 *   q        : device bf16 [batch][n_q][n_q_heads][head_dim]
 *   q_lens   : device int32 [batch][n_q], cells visible to each query token, or NULL
 *              (every query token of sequence b sees seq_lens[b] cells)
 *   head_map : host int32 [n_q_heads], KV head of each query head, or NULL for
 *              h / (n_q_heads / n_kv_heads) (then n_q_heads % n_kv_heads == 0)
 *   sm_scale : softmax scale (the caller's 1/sqrt(head_dim) for plain attention)
 *   out      : device fp32 [batch][n_q][n_q_heads][head_dim]; a query with no visible
 *              cell gets zeros.  With a Q4_0_H256 V store the output is rotated back.
 *   workspace: device, >= kvq_decode_workspace_bytes(...) bytes, 256-byte aligned.
 * Requires n_q * (largest number of query heads of one KV head) <= 32, head_dim 64,
 * 128 or 256, and a K store of format INT8_G64 (the V store may be INT8_G64 or
 * Q4_0_H256); or ISO3 K and V stores ([FT398] section What: the ISO attention backend runs its
 * own kernels over the packed cells, which its file table lists as the ISO attention source) with
 * head_dim 128 or 256 and n_q * (largest number
 * of query heads of one KV head) <= 16, or likewise ISO4 K and V stores (norms up to 65504).
 * ISO3 / ISO4 outputs are in the original basis.  A
 * Q4_0_H256 K store needs a Q4_0_H256 V store and the same <= 16 rows ([ST2698] "Not in this
 * PR": q4_0 K and V, rotated, with the queries rotated).  K and V stores that are each
 * INT8_G64 or F32, at least one F32 ([ST2698] "What it does": k8v32 / k32v8, and the FP32
 * default), take head_dim 128 or 256 and up to 32 rows. */
kvq_status kvq_decode_attn(const kvq_cache* cache, const kvq_pages* pages,
                           const void* q, int32_t n_q, int32_t n_q_heads,
                           const int32_t* q_lens, const int32_t* head_map,
                           float sm_scale, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* A decode step in one launch: quantize-on-write of the step's tokens ([FT398] section What:
 * a decode step stores each new token already quantised) and decode attention over the cache that
 * includes them ([ST2698] "What it does").  Same result as kvq_append of the n_q new tokens
 * of every sequence into cells seq_lens[b] - n_q .. seq_lens[b] - 1 followed by
 * kvq_decode_attn with the same arguments: the cells are encoded exactly as kvq_append
 * encodes them, written to the cache, and the attention reads them as stored.
 *   k_new, v_new : device bf16 [batch][n_q][n_kv_heads][head_dim], 16-byte aligned; token t
 *                  of sequence b goes to position seq_lens[b] - n_q + t
 *   seq_lens     : already counts the new tokens; a sequence with seq_lens[b] < n_q has no cell
 *                  for its tokens t < n_q - seq_lens[b], which are skipped (never written)
 * Other arguments, workspace and limits as for kvq_decode_attn (same workspace size).
 * Requires INT8_G64 or F32 K and V stores (the single-store modes included), or an INT8_G64
 * K store with a Q4_0_H256 V store at head_dim 256 (k8v4: [ST120] "How"), and 1 <= n_q <= 4.  A page holding new cells must not
 * be read by another sequence of the batch in the same call (pages written by a step are
 * owned by their sequence). */
kvq_status kvq_decode_attn_append(const kvq_cache* cache, const kvq_pages* pages,
                                  const void* k_new, const void* v_new,
                                  const void* q, int32_t n_q, int32_t n_q_heads,
                                  const int32_t* q_lens, const int32_t* head_map,
                                  float sm_scale, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* kvq_decode_attn for callers that cannot allocate device memory: code under HIP graph capture,
 * serving loops that forbid allocation, harnesses that cannot call hipMalloc.  It takes no workspace:
 * the split partials go to a scratch array the library keeps in device memory, one copy of
 * KVQ_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU it runs on, held from module load until the process
 * ends.  The call itself allocates nothing (the first call on a device looks up that device's
 * address of the array once).  Arguments, results and limits are those of kvq_decode_attn; a call
 * whose partials would exceed the scratch (kvq_decode_workspace_bytes(...) > KVQ_NOALLOC_SCRATCH_BYTES)
 * returns KVQ_ERR_WORKSPACE and enqueues nothing.  Every call on one GPU shares that GPU's scratch,
 * which keeps the last call's partials (nothing in it needs clearing between calls): calls that
 * overlap in time on one GPU (different streams, or host threads without ordering between them)
 * race and give wrong results.  Calls on one stream are ordered and safe. */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_decode_attn_noalloc(const kvq_cache* cache, const kvq_pages* pages,
                                   const void* q, int32_t n_q, int32_t n_q_heads,
                                   const int32_t* q_lens, const int32_t* head_map,
                                   float sm_scale, float* out, void* stream);

/* Workspace bytes kvq_decode_attn needs for this geometry (0 on invalid arguments). */
size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t max_pages,
                                  int32_t n_q, int32_t n_q_heads, const int32_t* head_map);

/* Extend (prefill chunk) attention ([FT398] "What"): new token i of sequence b sits at
 * position seq_lens[b] + i and attends the seq_lens[b] packed cells (dequantised) plus
 * new tokens 0..i of its own sequence unquantised (bf16).  With pack_after != 0 the new
 * tokens are quantised into cells seq_lens[b] + i after the attention, on the same
 * stream (deferred packing: the chunk never reads its own quantised K/V).  The caller
 * then advances seq_lens.
 *   q            : device bf16 [n_new][n_q_heads][head_dim]
 *   k_new, v_new : device bf16 [n_new][n_kv_heads][head_dim]
 *   cu_new       : device int32 [batch + 1], offsets of each sequence's new tokens;
 *                  cu_new[0] = 0 <= cu_new[1] <= ... <= cu_new[batch] = n_new
 *   max_new      : host bound, >= cu_new[b+1] - cu_new[b] for every b and <= n_new
 *                  (sizes the grid; tokens past it are not computed)
 *   head_map     : as for decode; at most 32 query heads per KV head
 *   out          : device fp32 [n_new][n_q_heads][head_dim]
 *   workspace    : device, >= kvq_extend_workspace_bytes(...) bytes, 256-byte aligned:
 *                  every 64-cell tile of every prefix and chunk is staged there once as
 *                  the attention kernel's tile image (about 33 KB per tile and KV head)
 * Requires ISO3 K and V stores, or INT8_G64 K and V stores ([ST2698] "What it does": the
 * prompt chunk reads the int8 cache dequantised), and head_dim 128.  ISO3 prefix attention
 * runs in the quaternion-rotated basis (the query rotated once, the accumulator rotated back
 * once); int8 prefix attention weights each 64-value group's partial sums by its scale;
 * the cells of a chunk's pages must not be written by pack_after of another sequence
 * in the same call. */
kvq_status kvq_extend_attn(const kvq_cache* cache, const kvq_pages* pages,
                           const void* q, const void* k_new, const void* v_new,
                           const int32_t* cu_new, int32_t n_new, int32_t max_new,
                           int32_t n_q_heads, const int32_t* head_map,
                           float sm_scale, float* out, int32_t pack_after,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes kvq_extend_attn needs for this geometry (0 on invalid arguments):
 * batch * n_kv_heads * (ceil(max_pages * page_size / 64) + ceil(max_new / 64)) tiles. */
size_t kvq_extend_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t max_pages,
                                  int32_t n_new, int32_t max_new, int32_t n_q_heads);

/* Dequantise cells [start, start+count) of sequence `seq` of one store into a contiguous
 * buffer ([ST120] "Tests": gather through the page table; [FT398] "What": the one-time
 * dequant of a packed prefix into a bf16 scratch; [ST2698] "What it does": dequantise a
 * cache range for a prompt chunk).
 *   which     : 0 = K store, 1 = V store
 *   out_dtype : kvq_out_dtype; F32 output is exact (it equals the encoder contract's
 *               dequantised value), F16/BF16 round it to nearest even
 *   unrotate  : for a Q4_0_H256 store, nonzero applies H (binary32 butterflies) so the
 *               output is in the original basis; otherwise the rotated values.
 *   out       : device [count][n_kv_heads][head_dim] of out_dtype
 * Requires 0 <= seq < batch, start >= 0, start + count <= max_pages * page_size. */
kvq_status kvq_dequant_gather(const kvq_cache* cache, const kvq_pages* pages, int32_t which,
                              int32_t seq, int32_t start, int32_t count, int32_t out_dtype,
                              int32_t unrotate, void* out, void* stream);

/* Bytes of one (token, KV head) cell of one store: returns code_bytes + 2 * n_scales and
 * writes the two parts if the pointers are non-NULL; -1 if fmt/head_dim are unsupported. */
int32_t kvq_cell_bytes(int32_t fmt, int32_t head_dim, int32_t* code_bytes, int32_t* n_scales);

const char* kvq_status_str(kvq_status status);
const char* kvq_last_error(void);   /* thread-local message of the last failed call */
int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
