// Page-stream probe: the memory access pattern of the int8 split-K decode kernel without its
// attention arithmetic, as a floor for that kernel's HBM time.  A measurement tool, built into its
// own library (libkvq_probe.so) and used by bench.py only; nothing in libkvq calls it.
//
// Grid (splits, n_kv_heads, 1) of `waves` waves; wave w of split s streams pages s * waves * ppw + w,
// + waves, ... (at most ppw of them, through the page table) of one KV head, keeping `depth` pages in
// flight, with the decode kernel's loads: per page and head the K code tile (16 B per lane, head_dim / 64
// loads), the V code tile (likewise), and unless `no_scales` the two 16-lane-strided scale loads.  The
// loaded words are folded with xor into one word per wave, written to `sink`, so no load is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxDepth = 4;
constexpr int kMaxGroups = 4;          // head_dim / 64 up to 256

struct ProbeArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_scales;
  const uint16_t* v_scales;
  const int32_t* block_table;          // one sequence: [max_pages]
  uint32_t* sink;                      // [splits * n_kv_heads * waves]
  int max_pages, num_pages, hkv, head_dim, waves, ppw, depth, no_scales;
};

struct Page {
  uint4 k[kMaxGroups], v[kMaxGroups];
  uint4 ks[2], vs[2];
};

__device__ __forceinline__ uint4 nt_load(const void* p) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int NG>
__device__ __forceinline__ void load(Page& pg, const ProbeArgs& a, int page, int kvh, int lane) {
  const size_t tile = (size_t)page * a.hkv + kvh;
  const uint4* kb = reinterpret_cast<const uint4*>(a.k_codes + tile * (16 * 64 * NG)) + lane;
  const uint4* vb = reinterpret_cast<const uint4*>(a.v_codes + tile * (16 * 64 * NG)) + lane;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    pg.k[g] = nt_load(kb + 64 * g);
    pg.v[g] = nt_load(vb + 64 * g);
  }
  if (!a.no_scales) {
    // the scales of tokens 4 (lane / 16) .. + 3, all groups: 8 B (head_dim 64), 16 B or 32 B per lane
    const uint16_t* ks = a.k_scales + (tile * 16 + 4 * (lane >> 4)) * NG;
    const uint16_t* vs = a.v_scales + (tile * 16 + 4 * (lane >> 4)) * NG;
    if constexpr (NG == 1) {
      const uint2 k2 = *reinterpret_cast<const uint2*>(ks), v2 = *reinterpret_cast<const uint2*>(vs);
      pg.ks[0] = make_uint4(k2.x, k2.y, 0u, 0u);
      pg.vs[0] = make_uint4(v2.x, v2.y, 0u, 0u);
    } else {
      pg.ks[0] = nt_load(ks); pg.vs[0] = nt_load(vs);
      if constexpr (NG > 2) { pg.ks[1] = nt_load(ks + 8); pg.vs[1] = nt_load(vs + 8); }
    }
  }
}

__device__ __forceinline__ uint32_t fold(const uint4& x) { return x.x ^ x.y ^ x.z ^ x.w; }

template <int NG, int PD>
__global__ __launch_bounds__(512) void k_page_probe(const ProbeArgs a) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, kvh = blockIdx.y;
  const int p_begin = split * a.waves * a.ppw;
  const int p0 = p_begin + wv;
  const int p_cap = min(p_begin + a.waves * a.ppw, a.max_pages) - 1;
  if (p0 > p_cap) return;
  const int n_mine = (p_cap - p0) / a.waves + 1;
  auto page_id = [&](int i) {
    const int p = min(p0 + min(i, n_mine - 1) * a.waves, p_cap);
    const int id = a.block_table[p];
    return id < 0 ? 0 : (id >= a.num_pages ? a.num_pages - 1 : id);
  };
  Page ring[PD + 1];
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < PD; ++i) load<NG>(ring[i], a, page_id(i), kvh, lane);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + PD < 16) load<NG>(ring[(i + PD) % (PD + 1)], a, page_id(i + PD), kvh, lane);
    const Page& pg = ring[i % (PD + 1)];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc ^= fold(pg.k[g]) ^ fold(pg.v[g]);
    if (!a.no_scales) acc ^= fold(pg.ks[0]) ^ fold(pg.vs[0]) ^ (NG > 2 ? fold(pg.ks[1]) ^ fold(pg.vs[1]) : 0u);
    if (i + 1 >= n_mine) break;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane == 0) a.sink[((size_t)split * a.hkv + kvh) * a.waves + wv] = acc;
}

template <int NG>
hipError_t launch_ng(const ProbeArgs& a, int splits, hipStream_t s) {
  const dim3 grid((unsigned)splits, (unsigned)a.hkv), block(64 * a.waves);
  switch (a.depth) {
    case 1: k_page_probe<NG, 1><<<grid, block, 0, s>>>(a); break;
    case 2: k_page_probe<NG, 2><<<grid, block, 0, s>>>(a); break;
    case 3: k_page_probe<NG, 3><<<grid, block, 0, s>>>(a); break;
    default: k_page_probe<NG, 4><<<grid, block, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Streams pages [0, max_pages) of one sequence for every KV head with the int8 decode kernel's loads
// (int8-g64 K and V tiles, head_dim 64 / 128 / 256); waves (1..8) per workgroup, ppw (1..16) pages
// per wave, depth (1..4) pages in flight.  Returns 0, or -1 on bad arguments, or the HIP error code.
int kvq_probe_page_stream(const void* k_codes, const void* v_codes, const void* k_scales, const void* v_scales,
                          const int32_t* block_table, int32_t max_pages, int32_t num_pages, int32_t n_kv_heads,
                          int32_t head_dim, int32_t waves, int32_t ppw, int32_t depth, int32_t no_scales,
                          uint32_t* sink, void* stream) {
  if (!k_codes || !v_codes || !k_scales || !v_scales || !block_table || !sink) return -1;
  if (max_pages < 1 || num_pages < 1 || n_kv_heads < 1 || waves < 1 || waves > 8 || ppw < 1 || ppw > 16 ||
      depth < 1 || depth > kMaxDepth)
    return -1;
  const ProbeArgs a{static_cast<const uint8_t*>(k_codes), static_cast<const uint8_t*>(v_codes),
                    static_cast<const uint16_t*>(k_scales), static_cast<const uint16_t*>(v_scales),
                    block_table, sink, max_pages, num_pages, n_kv_heads, head_dim, waves, ppw, depth, no_scales};
  const int splits = (max_pages + waves * ppw - 1) / (waves * ppw);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (head_dim) {
    case 64: e = launch_ng<1>(a, splits, s); break;
    case 128: e = launch_ng<2>(a, splits, s); break;
    case 256: e = launch_ng<4>(a, splits, s); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : (int)e;
}

// Workgroups of one probe launch (the sink needs splits * n_kv_heads * waves words).
int kvq_probe_sink_words(int32_t max_pages, int32_t n_kv_heads, int32_t waves, int32_t ppw) {
  if (max_pages < 1 || n_kv_heads < 1 || waves < 1 || ppw < 1) return -1;
  return (max_pages + waves * ppw - 1) / (waves * ppw) * n_kv_heads * waves;
}

}  // extern "C"
