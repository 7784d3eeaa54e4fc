// C-ABI entry points of helixdecode: argument checks on the host, geometry,
// the split policy, and the launches.  Nothing here allocates device memory.

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "hx_cache.h"

namespace hx {

static thread_local char g_err[512] = "";

hx_status fail(hx_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = 0; }

hx_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return HX_OK;
  return fail(HX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------- launch trace
// While a trace is open (hx_trace_begin .. hx_trace_end), every kernel the
// library launches is followed by a HIP event recorded on its stream, so the
// events bracket the launches.
struct Trace {
  std::mutex mu;
  bool open = false, overflow = false;
  int cap = 0, n = 0;
  hipEvent_t start = nullptr;
  std::vector<hipEvent_t> ev;
  std::vector<char> names;   // [cap][kTraceName]
};
constexpr int kTraceName = 32;
static Trace g_trace;
static std::atomic<bool> g_trace_open{false};

static void trace_mark(const char* name, hipStream_t st) {
  if (!g_trace_open.load(std::memory_order_acquire)) return;
  std::lock_guard<std::mutex> lk(g_trace.mu);
  if (!g_trace.open) return;
  if (g_trace.n >= g_trace.cap) {
    g_trace.overflow = true;
    return;
  }
  if (hipEventRecord(g_trace.ev[g_trace.n], st) != hipSuccess) {
    g_trace.overflow = true;
    return;
  }
  snprintf(&g_trace.names[(size_t)g_trace.n * kTraceName], kTraceName, "%s", name);
  ++g_trace.n;
}

// Plane and tile sizes for `units` chunk tiles per plane (one plane for a
// packed cache: its tiles hold all four parts).
static void plane_sizes(const Geometry& g, int64_t units, hx_kv_layout_info* out) {
  if (g.packed) {
    out->k_tile_bytes = (size_t)g.packed_tile;
    out->v_tile_bytes = 0;
    out->k_bytes = (size_t)(units * g.packed_tile);
    out->v_bytes = out->k_scale_bytes = out->v_scale_bytes = 0;
    return;
  }
  out->k_tile_bytes = (size_t)g.k_tile;
  out->v_tile_bytes = (size_t)g.v_tile;
  out->k_bytes = (size_t)(units * g.k_tile);
  out->v_bytes = (size_t)(units * g.v_tile);
  out->k_scale_bytes = (size_t)(units * g.ks_tile);
  out->v_scale_bytes = (size_t)(units * g.vs_tile);
}

// The cache as the kernels address it: base pointer and bytes between
// consecutive chunk tiles of the K codes, V codes, K scales and V scales.
// A packed (MXFP4) cache is one plane passed as `k`, its tiles holding the
// four parts in that order; an aliased (MLA) cache reads V from the K plane.
// Checks which planes must and must not be given, and their alignment.
struct PlaneRefs {
  uint8_t* base[4];
  int64_t stride[4];
};

static hx_status plane_refs(const hx_kv_desc& d, const Geometry& g, const hx_kv_cache* c, PlaneRefs* out) {
  PlaneRefs p{};
  if (!c->k) return fail(HX_EINVAL, "null K plane");
  if (g.packed) {
    if (c->v || c->k_scale || c->v_scale)
      return fail(HX_EINVAL, "a packed cache (MXFP4, or a quantised MLA cache) is one plane: pass it as k and leave "
                  "v, k_scale and v_scale NULL");
    // aliased (MLA): V codes and scales are the K ones
    const int64_t off[4] = {0, d.v_alias_k ? 0 : g.k_tile, g.k_tile + g.v_tile,
                            d.v_alias_k ? g.k_tile : g.k_tile + g.v_tile + g.ks_tile};
    for (int i = 0; i < 4; ++i) {
      p.base[i] = (uint8_t*)c->k + off[i];
      p.stride[i] = g.packed_tile;
    }
  } else {
    if (d.v_alias_k && c->v) return fail(HX_EINVAL, "cache->v must be NULL when v_alias_k = 1");
    if (!d.v_alias_k && !c->v) return fail(HX_EINVAL, "null V plane");
    if (d.dtype != HX_KV_BF16 && (!c->k_scale || (!d.v_alias_k && !c->v_scale)))
      return fail(HX_EINVAL, "null scale plane");
    p.base[0] = (uint8_t*)c->k;
    p.base[1] = (uint8_t*)(d.v_alias_k ? c->k : c->v);
    p.base[2] = (uint8_t*)c->k_scale;
    p.base[3] = (uint8_t*)(d.v_alias_k ? c->k_scale : c->v_scale);
    p.stride[0] = g.k_tile;
    p.stride[1] = d.v_alias_k ? g.k_tile : g.v_tile;
    p.stride[2] = g.ks_tile;
    p.stride[3] = d.v_alias_k ? g.ks_tile : g.vs_tile;
  }
  const void* ptrs[4] = {c->k, c->v, c->k_scale, c->v_scale};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(HX_EINVAL, "device pointers must be 16-byte aligned");
  *out = p;
  return HX_OK;
}

hx_status geometry(const hx_kv_desc& d, Geometry* g) {
  if (d.P < 1 || d.P > 64) return fail(HX_EINVAL, "P=%d must be in 1..64", d.P);
  if (d.B < 1) return fail(HX_EINVAL, "B=%d must be >= 1", d.B);
  if (d.Hkv < 1) return fail(HX_EINVAL, "Hkv=%d must be >= 1", d.Hkv);
  if (d.cap < kChunk || d.cap % kChunk) return fail(HX_EINVAL, "cap=%lld must be a positive multiple of 16", (long long)d.cap);
  if (d.flags & ~HX_FLAG_P_BF16) return fail(HX_EINVAL, "unknown flags 0x%x", d.flags);
  if (d.dtype < HX_KV_BF16 || d.dtype > HX_KV_MXFP4) return fail(HX_EINVAL, "unknown dtype %d", d.dtype);
  if (d.v_alias_k != 0 && d.v_alias_k != 1) return fail(HX_EINVAL, "v_alias_k must be 0 or 1");
  if (d.Dk < 1 || d.Dv < 1) return fail(HX_EINVAL, "Dk and Dv must be positive");
  Geometry t{};
  if (d.Dk == 128 && d.Dv == 128 && !d.v_alias_k) {
    t.kind = 0;
    if (d.dtype == HX_KV_BF16) {
      t.lay_k = kLayGqaBf16K; t.lay_v = kLayGqaBf16V; t.ebits = 16;
      t.k_tile = t.v_tile = 4096; t.ks_tile = t.vs_tile = 0;
    } else if (d.dtype == HX_KV_FP8_E4M3) {
      t.lay_k = kLayGqaFp8K; t.lay_v = kLayGqaFp8V; t.ebits = 8;
      t.k_tile = t.v_tile = 2048; t.ks_tile = t.vs_tile = 4;
    } else {
      t.lay_k = kLayGqaFp4K; t.lay_v = kLayGqaFp4V; t.ebits = 4;
      t.k_tile = t.v_tile = 1024; t.ks_tile = t.vs_tile = 16 * (128 / 32);
      t.packed = true;
      t.packed_tile = t.k_tile + t.v_tile + t.ks_tile + t.vs_tile;   // 2,176 B
    }
  } else if (d.Dk == 576 && d.Dv == 512 && d.v_alias_k) {
    t.kind = 1;
    t.lay_v = -1;
    t.v_tile = 0;
    t.vs_tile = 0;
    if (d.dtype == HX_KV_BF16) {
      t.lay_k = kLayMlaBf16; t.ebits = 16;
      t.k_tile = (int64_t)kChunk * 576 * 2; t.ks_tile = 0;
    } else {
      // quantised latent rows: one plane of packed tiles, the codes (row-major)
      // then the scales, so a workgroup streams one contiguous run; fp8: the
      // group's fp32 scale padded to 16 bytes; MXFP4: 16 rows x 18 e8m0 bytes
      t.packed = true;
      if (d.dtype == HX_KV_FP8_E4M3) {
        t.lay_k = kLayRowU8; t.ebits = 8;
        t.k_tile = (int64_t)kChunk * 576; t.ks_tile = 16;
      } else {
        t.lay_k = kLayRowU4; t.ebits = 4;
        t.k_tile = (int64_t)kChunk * 576 / 2; t.ks_tile = (int64_t)kChunk * (576 / 32);
      }
      t.packed_tile = t.k_tile + t.ks_tile;   // 9,232 B (fp8), 4,896 B (MXFP4)
    }
  } else {
    return fail(HX_EUNSUPPORTED, "unsupported cache: Dk=%d Dv=%d v_alias_k=%d dtype=%d", d.Dk, d.Dv, d.v_alias_k,
                d.dtype);
  }
  const double tiles = (double)d.P * d.B * d.Hkv * (double)(d.cap / kChunk);
  if (tiles * (double)(t.packed ? t.packed_tile : t.k_tile) > 9.0e18) return fail(HX_EINVAL, "cache too large");
  t.tiles = (int64_t)d.P * d.B * d.Hkv * (d.cap / kChunk);
  *g = t;
  return HX_OK;
}

// ---------------------------------------------------------------- split policy
static int env_int(const char* name, int dflt, int lo, int hi) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  const int v = atoi(s);
  return v < lo ? lo : (v > hi ? hi : v);
}

static int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

constexpr int64_t kShortSliceChunks = 64;   // 1,024 rows per slice

int target_wgs(int kind, int dtype, int G) {
  // Workgroups per CU for one launch, measured on MI355X at 1M-token contexts:
  // bf16 / fp8 tiles stream best with two workgroups per CU (one round, all
  // resident); MXFP4 splits are short in time (a quarter of the bf16 bytes
  // per row) and three workgroups fit per CU, so eight per CU keep the
  // rounds even (measured: 475 us at four, 445 us at eight on the ragged
  // 16-request cache).  The MLA kernel holds 144 KiB of LDS: one workgroup
  // of four waves per CU.  HX_WGS_PER_CU overrides (tuning knob).
  // Wide GQA groups (LDS-shared tile pairs, decode_gqa_wide.hip) run best
  // with four workgroups per CU for bf16 and eight for fp8 and MXFP4 pairs.
  const bool wide = kind == 0 && G > kGqaNarrowMaxHeads;
  const int dflt = kind != 0 ? 1 : (dtype == HX_KV_MXFP4 ? 8 : (wide ? (dtype == HX_KV_BF16 ? 4 : 8) : 2));
  const int per_cu = env_int("HX_WGS_PER_CU", dflt, 1, 8);
  const int bound = kind == 0 ? kGqaTargetWgs : kMlaTargetWgs;
  return std::min(bound, device_cus() * per_cu);
}

// Workgroups per launch for a batch whose one-round plan above overflows its
// round (ragged contexts: each slice's last split is short, so the slices
// need more splits in all than the target): narrow bf16 and fp8 groups then
// take eight workgroups per CU, several rounds whose shorter workgroups
// (dispatched last) fill the end of the launch.  Measured on 16 requests of
// 4K-2M tokens: bf16 1,492 -> 1,438 us, fp8 768 -> 741 us (four per CU); on
// uniform contexts one round stays best (1M tokens: 652 us at two per CU,
// 657 at four).  0: no such re-plan (other kernels, or HX_WGS_PER_CU set).
int overflow_target_wgs(int kind, int dtype, int G) {
  if (kind != 0 || G > kGqaNarrowMaxHeads || dtype == HX_KV_MXFP4 || getenv("HX_WGS_PER_CU")) return 0;
  return std::min(kGqaTargetWgs, device_cus() * 8);
}

// Smallest split (chunk tiles per workgroup): GQA waves each take one tile in
// turn, so four per wave keep their loads pipelined; MLA tiles come in pairs.
// HX_MIN_CHUNKS_PER_WG overrides (tuning knob).
int min_chunks_per_wg(int kind) {
  const int dflt = kind == 0 ? 4 * kGqaWavesPerWg : 4;
  const int v = env_int("HX_MIN_CHUNKS_PER_WG", dflt, 1, 1 << 20);
  return kind == 1 ? v + (v & 1) : v;
}

static int64_t ws_records(const hx_kv_desc& d, int kind) {
  const int bound = kind == 0 ? kGqaTargetWgs : kMlaTargetWgs;
  return (int64_t)bound + (int64_t)d.Hkv * d.P * std::min(d.B, kMaxBatchPerLaunch);
}

static int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// Workspace: one record per workgroup of a launch, [records][G][Dv] partial
// outputs then [records][G] LSEs.
struct WsLayout {
  int64_t o_off, lse_off;         // split records
  int64_t opart_off, lpart_off;   // slice partials of hx_decode_attn
  int64_t total;
};

// `recs` split records: ws_records (the bound hx_workspace_size reports),
// or the count one call actually uses (the fixed scratch of
// hx_decode_attn_noalloc).
static WsLayout ws_layout(const hx_kv_desc& d, int G, int64_t recs) {
  WsLayout w;
  const int64_t Hq = (int64_t)G * d.Hkv;
  w.o_off = 0;
  w.lse_off = align256(recs * G * d.Dv * 4);
  w.opart_off = w.lse_off + align256(recs * G * 4);
  w.lpart_off = w.opart_off + align256((int64_t)d.P * d.B * Hq * d.Dv * 4);
  w.total = w.lpart_off + align256((int64_t)d.P * d.B * Hq * 4);
  return w;
}

}  // namespace hx

using namespace hx;

extern "C" {

const char* hx_last_error(void) { return g_err; }

const char* hx_version(void) { return "helixdecode 0.1 (gfx950)"; }

hx_status hx_kv_layout(const hx_kv_desc* desc, hx_kv_layout_info* out) {
  g_err[0] = 0;
  if (!desc || !out) return fail(HX_EINVAL, "null argument");
  Geometry g;
  hx_status s = geometry(*desc, &g);
  if (s) return s;
  plane_sizes(g, g.tiles, out);
  out->n_max = (int64_t)desc->P * desc->cap;
  return HX_OK;
}

hx_status hx_slot(int64_t t, int32_t P, int32_t* r, int64_t* j) {
  g_err[0] = 0;
  if (!r || !j) return fail(HX_EINVAL, "null argument");
  if (t < 0 || P < 1) return fail(HX_EINVAL, "t=%lld must be >= 0 and P=%d >= 1", (long long)t, P);
  const int64_t c = t / kChunk;
  *r = (int32_t)(c % P);
  *j = (c / P) * kChunk + t % kChunk;
  return HX_OK;
}

hx_status hx_slice_len(int64_t n, int32_t P, int32_t r, int64_t* len) {
  g_err[0] = 0;
  if (!len) return fail(HX_EINVAL, "null argument");
  if (n < 0 || P < 1 || r < 0 || r >= P) return fail(HX_EINVAL, "need n >= 0, P >= 1, 0 <= r < P");
  *len = slice_len(n, P, r);
  return HX_OK;
}

hx_status hx_kv_tile_offset(const hx_kv_desc* desc, int32_t which, int32_t m, int32_t d, int64_t* off2) {
  g_err[0] = 0;
  if (!desc || !off2) return fail(HX_EINVAL, "null argument");
  Geometry g;
  hx_status s = geometry(*desc, &g);
  if (s) return s;
  if (which < 0 || which > 3) return fail(HX_EINVAL, "which must be 0 (K), 1 (V), 2 (K scale) or 3 (V scale)");
  const bool is_v = which == 1 || which == 3;
  if (is_v && desc->v_alias_k) return fail(HX_EINVAL, "an aliased cache has no V plane");
  const int width = is_v ? desc->Dv : desc->Dk;
  if (m < 0 || m >= kChunk || d < 0 || d >= width) return fail(HX_EINVAL, "element out of the tile");
  if (which < 2) {
    // a packed tile holds the V codes after the K codes
    *off2 = tile_off2(is_v ? g.lay_v : g.lay_k, desc->Dk, m, d) + (g.packed && is_v ? 2 * g.k_tile : 0);
    return HX_OK;
  }
  if (desc->dtype == HX_KV_BF16) return fail(HX_EINVAL, "bf16 caches have no scales");
  // fp8: the tile's one float; MXFP4: the e8m0 byte of row m, 32-column block d / 32 (after the codes when packed)
  const int64_t byte = desc->dtype == HX_KV_FP8_E4M3 ? 0 : (int64_t)m * (width / 32) + d / 32;
  const int64_t base = g.packed ? g.k_tile + g.v_tile + (is_v ? g.ks_tile : 0) : 0;
  *off2 = 2 * (base + byte);
  return HX_OK;
}

}  // extern "C"

namespace hx {

// A block pool's table and size; {nullptr, 0} for a dense cache.
struct PoolRef {
  const int32_t* table;
  int32_t num_blocks;
};

static hx_status check_pool(const hx_kv_desc* desc, const hx_kv_pool* pool, PoolRef* ref) {
  if (!desc || !pool) return fail(HX_EINVAL, "null argument");
  if (!pool->block_table || !aligned16(pool->block_table))
    return fail(HX_EINVAL, "block_table must be a non-null 16-byte aligned device pointer");
  if (pool->num_blocks < 1) return fail(HX_EINVAL, "num_blocks=%d must be >= 1", pool->num_blocks);
  if (pool->reserved != 0) return fail(HX_EINVAL, "reserved must be 0");
  Geometry g;
  hx_status s = geometry(*desc, &g);
  if (s) return s;
  if ((double)pool->num_blocks * desc->Hkv * (double)(g.packed ? g.packed_tile : g.k_tile) > 9.0e18)
    return fail(HX_EINVAL, "pool too large");
  *ref = PoolRef{pool->block_table, pool->num_blocks};
  return HX_OK;
}

// Checks an append's arguments and fills the plane fields of `a` (every
// request; per-launch fields are set by append_batch).
static hx_status append_setup(const hx_kv_desc* desc, const hx_kv_cache* cache, PoolRef pool, const void* k_new,
                              const void* v_new, const void* k_scale_new, const void* v_scale_new, const int64_t* pos,
                              const int32_t* count, int32_t n_new, AppendArgs* out) {
  if (!desc || !cache || !pos) return fail(HX_EINVAL, "null argument");
  Geometry g;
  hx_status s = geometry(*desc, &g);
  if (s) return s;
  const hx_kv_desc& d = *desc;
  if (n_new < 1) return fail(HX_EINVAL, "n_new=%d must be >= 1", n_new);
  const bool alias = d.v_alias_k;
  const bool scaled = d.dtype != HX_KV_BF16;
  PlaneRefs pr;
  s = plane_refs(d, g, cache, &pr);
  if (s) return s;
  if (!k_new) return fail(HX_EINVAL, "null k_new");
  if (!alias && !v_new) return fail(HX_EINVAL, "null v_new");
  if (alias && v_new) return fail(HX_EINVAL, "v_new must be NULL when v_alias_k = 1");
  if (scaled && (!k_scale_new || (!alias && !v_scale_new))) return fail(HX_EINVAL, "null scale input");
  if (!scaled && (k_scale_new || v_scale_new)) return fail(HX_EINVAL, "bf16 caches take no scales");
  const void* ptrs[4] = {k_new, v_new, k_scale_new, v_scale_new};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(HX_EINVAL, "device pointers must be 16-byte aligned");
  const int64_t nmax = (int64_t)d.P * d.cap;
  for (int b = 0; b < d.B; ++b) {
    const int32_t cnt = count ? count[b] : n_new;
    if (cnt < 0 || cnt > n_new) return fail(HX_EINVAL, "request %d: count=%d must be in [0, n_new=%d]", b, cnt, n_new);
    if (pos[b] < 0 || pos[b] + cnt > nmax)
      return fail(HX_EINVAL, "request %d: pos=%lld, count=%d exceeds P*cap=%lld", b, (long long)pos[b], cnt,
                  (long long)nmax);
  }

  AppendArgs a{};
  int np = 0;
  // plane i of pr: 0 K codes, 1 V codes, 2 K scales, 3 V scales
  auto add = [&](const void* src, int i, int lay, int width, int ebits, int64_t row_bytes, int64_t tile_bytes) {
    a.src[np] = (const uint8_t*)src;
    a.dst[np] = pr.base[i];
    a.lay[np] = lay;
    a.width[np] = width;
    a.ebits[np] = ebits;
    a.src_row_bytes[np] = row_bytes;
    a.tile_bytes[np] = tile_bytes;
    a.tile_stride[np] = pr.stride[i];
    ++np;
  };
  add(k_new, 0, g.lay_k, d.Dk, g.ebits, (int64_t)d.Dk * g.ebits / 8, g.k_tile);
  if (!alias) add(v_new, 1, g.lay_v, d.Dv, g.ebits, (int64_t)d.Dv * g.ebits / 8, g.v_tile);
  if (d.dtype == HX_KV_FP8_E4M3) {
    add(k_scale_new, 2, kLayRowU8, 1, 32, 4, 4);
    if (!alias) add(v_scale_new, 3, kLayRowU8, 1, 32, 4, 4);
  } else if (d.dtype == HX_KV_MXFP4) {
    add(k_scale_new, 2, kLayRowU8, d.Dk / 32, 8, d.Dk / 32, g.ks_tile);
    if (!alias) add(v_scale_new, 3, kLayRowU8, d.Dv / 32, 8, d.Dv / 32, g.vs_tile);
  }
  a.nplanes = np;
  a.P = d.P;
  a.B = d.B;
  a.Hkv = d.Hkv;
  a.cap_chunks = d.cap / kChunk;
  a.table = pool.table;
  a.num_blocks = pool.num_blocks;
  a.n_new = n_new;
  *out = a;
  return HX_OK;
}

// The per-launch fields of an append for requests b0 .. b0 + nb - 1 (`base`
// as append_setup left it: its src are the first request's rows).
static AppendArgs append_batch(const AppendArgs& base, const int64_t* pos, const int32_t* count, int b0, int nb) {
  AppendArgs a = base;
  int maxc = 0;
  for (int i = 0; i < nb; ++i) {
    const int64_t p0 = pos[b0 + i];
    const int32_t cnt = count ? count[b0 + i] : base.n_new;
    a.pos[i] = p0;
    a.count[i] = cnt;
    if (cnt > 0) maxc = std::max(maxc, (int)((p0 + cnt - 1) / kChunk - p0 / kChunk + 1));
  }
  a.max_chunks = maxc;
  a.b0 = b0;
  for (int p = 0; p < a.nplanes; ++p) a.src[p] = base.src[p] + (int64_t)b0 * a.Hkv * a.n_new * a.src_row_bytes[p];
  return a;
}

static hx_status kv_append(const hx_kv_desc* desc, const hx_kv_cache* cache, PoolRef pool, const void* k_new,
                           const void* v_new, const void* k_scale_new, const void* v_scale_new, const int64_t* pos,
                           const int32_t* count, int32_t n_new, void* stream) {
  AppendArgs base;
  hx_status s = append_setup(desc, cache, pool, k_new, v_new, k_scale_new, v_scale_new, pos, count, n_new, &base);
  if (s) return s;
  for (int b0 = 0; b0 < desc->B; b0 += kMaxBatchPerLaunch) {
    const int nb = std::min(kMaxBatchPerLaunch, desc->B - b0);
    const AppendArgs a = append_batch(base, pos, count, b0, nb);
    s = check_hip(launch_append(a, nb, (hipStream_t)stream), "kv_append launch");
    if (s) return s;
    if (a.max_chunks > 0) trace_mark("append", (hipStream_t)stream);
  }
  return HX_OK;
}

static hx_status kv_append_bf16(const hx_kv_desc* desc, const hx_kv_cache* cache, PoolRef pool, const void* k_new,
                                const void* v_new, const int64_t* pos, const int32_t* count, int32_t n_new,
                                void* stream) {
  if (!desc || !cache || !pos) return fail(HX_EINVAL, "null argument");
  Geometry g;
  hx_status s = geometry(*desc, &g);
  if (s) return s;
  const hx_kv_desc& d = *desc;
  if (d.dtype == HX_KV_BF16) return kv_append(desc, cache, pool, k_new, v_new, nullptr, nullptr, pos, count, n_new, stream);
  if (n_new < 1) return fail(HX_EINVAL, "n_new=%d must be >= 1", n_new);
  PlaneRefs pr;
  s = plane_refs(d, g, cache, &pr);
  if (s) return s;
  const bool alias = d.v_alias_k;   // MLA latent rows: K only
  if (!k_new || (!alias && !v_new)) return fail(HX_EINVAL, "null k_new or v_new");
  if (alias && v_new) return fail(HX_EINVAL, "v_new must be NULL when v_alias_k = 1");
  if (!aligned16(k_new) || (v_new && !aligned16(v_new))) return fail(HX_EINVAL, "device pointers must be 16-byte aligned");
  const int64_t nmax = (int64_t)d.P * d.cap;
  for (int b = 0; b < d.B; ++b) {
    const int32_t cnt = count ? count[b] : n_new;
    if (cnt < 0 || cnt > n_new) return fail(HX_EINVAL, "request %d: count=%d must be in [0, n_new=%d]", b, cnt, n_new);
    if (pos[b] < 0 || pos[b] + cnt > nmax)
      return fail(HX_EINVAL, "request %d: pos=%lld, count=%d exceeds P*cap=%lld", b, (long long)pos[b], cnt,
                  (long long)nmax);
  }
  QAppendArgs a{};
  a.dst[0] = pr.base[0];
  a.dst[1] = pr.base[1];
  a.sc[0] = pr.base[2];
  a.sc[1] = pr.base[3];
  a.lay[0] = g.lay_k;
  a.lay[1] = g.lay_v;
  a.nplanes = alias ? 1 : 2;
  a.dtype = d.dtype;
  a.D = d.Dk;
  a.P = d.P;
  a.B = d.B;
  a.Hkv = d.Hkv;
  a.cap_chunks = d.cap / kChunk;
  a.table = pool.table;
  a.num_blocks = pool.num_blocks;
  a.tile_stride = pr.stride[0];      // K and V code planes share it
  a.sc_tile_stride = pr.stride[2];   // and so do the scale planes
  a.n_new = n_new;
  for (int b0 = 0; b0 < d.B; b0 += kMaxBatchPerLaunch) {
    const int nb = std::min(kMaxBatchPerLaunch, d.B - b0);
    int maxc = 0;
    for (int i = 0; i < nb; ++i) {
      const int64_t p0 = pos[b0 + i];
      const int32_t cnt = count ? count[b0 + i] : n_new;
      a.pos[i] = p0;
      a.count[i] = cnt;
      if (cnt > 0) maxc = std::max(maxc, (int)((p0 + cnt - 1) / kChunk - p0 / kChunk + 1));
    }
    if (maxc == 0) continue;
    a.max_chunks = maxc;
    a.b0 = b0;
    const int64_t off = (int64_t)b0 * d.Hkv * n_new * d.Dk;
    a.src[0] = (const uint16_t*)k_new + off;
    a.src[1] = alias ? nullptr : (const uint16_t*)v_new + off;
    s = check_hip(launch_quant_append(a, nb, (hipStream_t)stream), "kv_append_bf16 launch");
    if (s) return s;
    trace_mark("quant_append", (hipStream_t)stream);
  }
  return HX_OK;
}

static hx_status kv_dequant(const hx_kv_desc* desc, const hx_kv_cache* cache, PoolRef pool, int32_t r, int32_t b,
                            int32_t g, int64_t j0, int64_t n, float* k_out, float* v_out, void* stream) {
  if (!desc || !cache || !k_out) return fail(HX_EINVAL, "null argument");
  Geometry geo;
  hx_status s = geometry(*desc, &geo);
  if (s) return s;
  const hx_kv_desc& d = *desc;
  if (r < 0 || r >= d.P || b < 0 || b >= d.B || g < 0 || g >= d.Hkv) return fail(HX_EINVAL, "(r, b, g) out of range");
  if (j0 < 0 || n < 0 || j0 + n > d.cap) return fail(HX_EINVAL, "rows [j0, j0+n) must lie in [0, cap)");
  PlaneRefs pr;
  s = plane_refs(d, geo, cache, &pr);
  if (s) return s;
  if (!aligned16(k_out) || (v_out && !aligned16(v_out))) return fail(HX_EINVAL, "device pointers must be 16-byte aligned");
  DequantArgs a{};
  a.k = pr.base[0];
  a.v = pr.base[1];
  a.ks = pr.base[2];
  a.vs = pr.base[3];
  a.k_out = k_out;
  a.v_out = v_out;
  a.dtype = d.dtype;
  a.lay_k = geo.lay_k;
  a.lay_v = geo.lay_v;
  a.Dk = d.Dk;
  a.Dv = d.Dv;
  a.v_alias = d.v_alias_k;
  a.k_tile = pr.stride[0];
  a.v_tile = pr.stride[1];
  a.ks_tile = pr.stride[2];
  a.vs_tile = pr.stride[3];
  a.map = TileMap{pool.table, pool.num_blocks, d.P, d.B, d.Hkv, d.cap / kChunk};
  a.r = r;
  a.b = b;
  a.g = g;
  a.j0 = j0;
  a.n = n;
  s = check_hip(launch_dequant(a, (hipStream_t)stream), "kv_dequant launch");
  if (!s && n > 0) trace_mark("dequant", (hipStream_t)stream);
  return s;
}

}  // namespace hx

extern "C" {

hx_status hx_kv_append(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* k_new, const void* v_new,
                       const void* k_scale_new, const void* v_scale_new, const int64_t* pos, const int32_t* count,
                       int32_t n_new, void* stream) {
  g_err[0] = 0;
  return kv_append(desc, cache, PoolRef{nullptr, 0}, k_new, v_new, k_scale_new, v_scale_new, pos, count, n_new, stream);
}

hx_status hx_kv_append_bf16(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* k_new, const void* v_new,
                            const int64_t* pos, const int32_t* count, int32_t n_new, void* stream) {
  g_err[0] = 0;
  return kv_append_bf16(desc, cache, PoolRef{nullptr, 0}, k_new, v_new, pos, count, n_new, stream);
}

hx_status hx_kv_dequant(const hx_kv_desc* desc, const hx_kv_cache* cache, int32_t r, int32_t b, int32_t g,
                        int64_t j0, int64_t n, float* k_out, float* v_out, void* stream) {
  g_err[0] = 0;
  return kv_dequant(desc, cache, PoolRef{nullptr, 0}, r, b, g, j0, n, k_out, v_out, stream);
}

hx_status hx_kv_append_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* k_new, const void* v_new,
                             const void* k_scale_new, const void* v_scale_new, const int64_t* pos,
                             const int32_t* count, int32_t n_new, void* stream) {
  g_err[0] = 0;
  PoolRef ref;
  hx_status s = check_pool(desc, pool, &ref);
  if (s) return s;
  return kv_append(desc, &pool->planes, ref, k_new, v_new, k_scale_new, v_scale_new, pos, count, n_new, stream);
}

hx_status hx_kv_append_bf16_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* k_new,
                                  const void* v_new, const int64_t* pos, const int32_t* count, int32_t n_new,
                                  void* stream) {
  g_err[0] = 0;
  PoolRef ref;
  hx_status s = check_pool(desc, pool, &ref);
  if (s) return s;
  return kv_append_bf16(desc, &pool->planes, ref, k_new, v_new, pos, count, n_new, stream);
}

hx_status hx_kv_dequant_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, int32_t r, int32_t b, int32_t g,
                              int64_t j0, int64_t n, float* k_out, float* v_out, void* stream) {
  g_err[0] = 0;
  PoolRef ref;
  hx_status s = check_pool(desc, pool, &ref);
  if (s) return s;
  return kv_dequant(desc, &pool->planes, ref, r, b, g, j0, n, k_out, v_out, stream);
}

hx_status hx_pool_layout(const hx_kv_desc* desc, int32_t num_blocks, hx_kv_layout_info* out) {
  g_err[0] = 0;
  if (!desc || !out) return fail(HX_EINVAL, "null argument");
  Geometry g;
  hx_status s = geometry(*desc, &g);
  if (s) return s;
  if (num_blocks < 1) return fail(HX_EINVAL, "num_blocks=%d must be >= 1", num_blocks);
  const double tiles = (double)num_blocks * desc->Hkv;
  if (tiles * (double)(g.packed ? g.packed_tile : g.k_tile) > 9.0e18) return fail(HX_EINVAL, "pool too large");
  plane_sizes(g, (int64_t)num_blocks * desc->Hkv, out);
  out->n_max = (int64_t)desc->P * desc->cap;
  return HX_OK;
}

}  // extern "C"

namespace hx {

static hx_status check_heads(const hx_kv_desc& d, const Geometry& geo, int32_t Hq) {
  if (Hq < 1 || Hq % d.Hkv) return fail(HX_EINVAL, "Hq=%d must be a positive multiple of Hkv=%d", Hq, d.Hkv);
  const int G = Hq / d.Hkv;
  if (geo.kind == 0 && G > kGqaWideMaxHeads)
    return fail(HX_EUNSUPPORTED, "GQA kernels take at most %d query heads per KV head (G=%d)", kGqaWideMaxHeads, G);
  if (geo.kind == 1 && G != 128) return fail(HX_EUNSUPPORTED, "MLA kernel takes 128 query heads per latent head (G=%d)", G);
  return HX_OK;
}

}  // namespace hx

extern "C" {

hx_status hx_workspace_size(const hx_kv_desc* desc, int32_t Hq, size_t* bytes) {
  g_err[0] = 0;
  if (!desc || !bytes) return fail(HX_EINVAL, "null argument");
  Geometry geo;
  hx_status s = geometry(*desc, &geo);
  if (s) return s;
  s = check_heads(*desc, geo, Hq);
  if (s) return s;
  *bytes = (size_t)ws_layout(*desc, Hq / desc->Hkv, ws_records(*desc, geo.kind)).total;
  return HX_OK;
}

hx_status hx_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!ws || !aligned16(ws)) return fail(HX_EINVAL, "workspace must be a non-null 16-byte aligned pointer");
  return check_hip(hipMemsetAsync(ws, 0, ws_bytes, (hipStream_t)stream), "workspace memset");
}

}  // extern "C"

namespace hx {

// The partial pass of a decode step.  With o_final / lse_final (hx_decode_attn)
// the slice partials go to workspace scratch and one more kernel folds every
// slice's partial or split records straight into the final output.
// With `fuse` (an append_setup result) and its host positions, the partial
// kernels first append those rows into the tiles they own (hx_decode_step).
// Split plan of the requests b0 .. b0 + nb - 1 of one launch: fills a.n,
// a.cpw, a.waves, a.nsplit, a.wg_begin and a.fold_begin; returns the number
// of workgroups (= split records) of the launch.  `final_out`: the one-call
// forms, which fold every record in their second launch.
static int plan_launch(const hx_kv_desc& d, const Geometry& geo, const int64_t* ctx_len, int b0, int nb, int G,
                       bool final_out, PartialArgs& a) {
  const int target = target_wgs(geo.kind, d.dtype, G);
  // the one-call forms (fold launched anyway) take splits half as long:
  // two tiles per wave (measured on the 4,096-token step: 30.2 -> 29.3 us)
  const int minc = final_out ? std::max(1, min_chunks_per_wg(geo.kind) / 2) : min_chunks_per_wg(geo.kind);
  int64_t W = 0;
  int64_t nch[kMaxBatchPerLaunch];
  for (int i = 0; i < nb; ++i) {
    a.n[i] = ctx_len[b0 + i];
    nch[i] = (slice_len(a.n[i], d.P, 0) + kChunk - 1) / kChunk;   // slice 0 is never shorter
    W += nch[i] * d.Hkv * d.P;
  }
  int64_t nch_max = 1;
  for (int i = 0; i < nb; ++i) nch_max = std::max(nch_max, nch[i]);
  auto split_size = [&](int tgt) {
    const int64_t c = std::max<int64_t>(minc, (W + tgt - 1) / tgt);
    return std::max<int64_t>(c, (nch_max + kMaxSplits - 1) / kMaxSplits);
  };
  int64_t cpw = split_size(target);
  // short contexts: slices of at most kShortSliceChunks tiles are not split
  // (one workgroup per slice, no fold launch; measured faster on the
  // 4,096-token single-request step, where fixed launch costs dominate).
  // The one-call forms fold every record in their second launch anyway, so
  // there short slices are split like long ones (HX_SHORT_ONE_CALL=1 keeps
  // them whole: tuning knob).
  const bool short_mode = nch_max <= kShortSliceChunks && (!final_out || env_int("HX_SHORT_ONE_CALL", 0, 0, 1));
  if (short_mode) cpw = std::max<int64_t>(cpw, nch_max);
  a.waves = geo.kind == 0 && short_mode ? kGqaShortWaves : kGqaWavesPerWg;
  const bool pairs = geo.kind == 1 || G > kGqaNarrowMaxHeads;   // MLA and wide-GQA tiles come in pairs
  // splits of every request for split size cpw: as even as its split count
  // allows (the last split of a slice is otherwise the remainder, up to
  // cpw - 1 tiles short), pairs kept whole; returns the workgroup count
  auto splits = [&](int64_t c) {
    if (pairs) c += c & 1;
    a.cpw = (int)std::min<int64_t>(c, 1 << 30);
    int64_t total = 0;
    for (int i = 0; i < nb; ++i) {
      const int64_t ns = (nch[i] + a.cpw - 1) / a.cpw;
      int64_t cb = (nch[i] + ns - 1) / ns;
      if (pairs) cb += cb & 1;
      a.cpw_b[i] = (int)cb;
      a.nsplit[i] = (int)((nch[i] + cb - 1) / cb);
      total += (int64_t)a.nsplit[i] * d.Hkv * d.P;
    }
    return total;
  };
  const int64_t total = splits(cpw);
  const int over = short_mode ? 0 : overflow_target_wgs(geo.kind, d.dtype, G);
  if (over > 0 && total > target) splits(split_size(over));
  int folds = 0;
  for (int i = 0; i < nb; ++i) {
    a.fold_begin[i] = folds;
    if (a.nsplit[i] > 1) folds += d.Hkv * d.P * G;
  }
  a.fold_begin[nb] = folds;
  // Workgroups of the requests with the longest splits first: the hardware
  // starts workgroups in index order as slots free up, so the shorter ones
  // fill the end of the launch.
  for (int i = 0; i < nb; ++i) a.order[i] = i;
  std::stable_sort(a.order, a.order + nb, [&](int x, int y) { return a.cpw_b[x] > a.cpw_b[y]; });
  int wgs = 0;
  for (int p = 0; p < nb; ++p) {
    const int i = a.order[p];
    a.pos_begin[p] = wgs;
    a.wg_begin[i] = wgs;
    wgs += a.nsplit[i] * d.Hkv * d.P;
  }
  a.pos_begin[nb] = wgs;
  a.wg_begin[nb] = wgs;
  return wgs;
}

// Bytes of the library's fixed scratch, the workspace of
// hx_decode_attn_noalloc (one array per device, held until the process
// ends): enough for the split records and slice partials of every workload
// here (the largest, 8 requests of 128 MLA heads at 2^20 tokens, uses about
// 80 MiB).
constexpr size_t kScratchBytes = (size_t)128 << 20;

// With `check_only`, every argument is checked and nothing is launched.
// With `tight`, the workspace holds just the split records this call uses
// (the fixed scratch of hx_decode_attn_noalloc) instead of the bound that
// hx_workspace_size reports.
static hx_status decode_step(const hx_kv_desc* desc, const hx_kv_cache* cache, PoolRef pool, const void* q,
                             int32_t Hq, const int64_t* ctx_len, float scale, float* o_part, float* lse_part,
                             void* ws, size_t ws_bytes, void* stream, float* o_final, float* lse_final,
                             const AppendArgs* fuse = nullptr, const int64_t* fuse_pos = nullptr,
                             bool check_only = false, bool tight = false) {
  const bool final_out = o_final != nullptr;
  // (the fixed scratch's address is taken after the checks: none yet then)
  if (!desc || !cache || !q || !ctx_len || (!ws && !(tight && check_only))) return fail(HX_EINVAL, "null argument");
  if (final_out ? !lse_final : (!o_part || !lse_part)) return fail(HX_EINVAL, "null argument");
  Geometry geo;
  hx_status s = geometry(*desc, &geo);
  if (s) return s;
  const hx_kv_desc& d = *desc;
  s = check_heads(d, geo, Hq);
  if (s) return s;
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(HX_EINVAL, "scale must be finite and > 0");
  PlaneRefs pr;
  s = plane_refs(d, geo, cache, &pr);
  if (s) return s;
  const void* ptrs[6] = {q, o_part, lse_part, ws, o_final, lse_final};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(HX_EINVAL, "device pointers must be 16-byte aligned");
  const int G = Hq / d.Hkv;
  const int64_t nmax = (int64_t)d.P * d.cap;
  for (int b = 0; b < d.B; ++b)
    if (ctx_len[b] < 1 || ctx_len[b] > nmax)
      return fail(HX_EINVAL, "ctx_len[%d]=%lld must be in [1, P*cap=%lld]", b, (long long)ctx_len[b], (long long)nmax);
  int64_t records = ws_records(d, geo.kind);
  if (tight) {
    records = 1;
    for (int b0 = 0; b0 < d.B; b0 += kMaxBatchPerLaunch) {
      PartialArgs t{};
      records = std::max<int64_t>(records, plan_launch(d, geo, ctx_len, b0, std::min(kMaxBatchPerLaunch, d.B - b0), G,
                                                        final_out, t));
    }
  }
  const WsLayout wl = ws_layout(d, G, records);
  if ((int64_t)ws_bytes < wl.total) {
    if (tight)
      return fail(HX_EINVAL, "this call needs %lld bytes of scratch, more than the %zu bytes of the library's fixed "
                  "scratch: call hx_decode_attn with a workspace instead", (long long)wl.total, ws_bytes);
    return fail(HX_EINVAL, "workspace of %zu bytes is smaller than the %lld needed", ws_bytes, (long long)wl.total);
  }
  if (final_out) {
    o_part = (float*)((uint8_t*)ws + wl.opart_off);
    lse_part = (float*)((uint8_t*)ws + wl.lpart_off);
  }
  if (check_only) return HX_OK;

  PartialArgs a{};
  a.k = pr.base[0];
  a.v = pr.base[1];
  a.ks = pr.base[2];
  a.vs = pr.base[3];
  a.q = (const uint16_t*)q;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.ws_o = (float*)((uint8_t*)ws + wl.o_off);
  a.ws_lse = (float*)((uint8_t*)ws + wl.lse_off);
  a.P = d.P;
  a.Btot = d.B;
  a.Hkv = d.Hkv;
  a.Hq = Hq;
  a.G = G;
  a.Dk = d.Dk;
  a.Dv = d.Dv;
  a.cap_chunks = d.cap / kChunk;
  a.table = pool.table;
  a.num_blocks = pool.num_blocks;
  a.k_tile = pr.stride[0];
  a.v_tile = pr.stride[1];
  a.ks_tile = pr.stride[2];
  a.vs_tile = pr.stride[3];
  a.c2 = scale * 1.44269504088896341f;
  a.split_p = (d.flags & HX_FLAG_P_BF16) == 0;
  for (int b0 = 0; b0 < d.B; b0 += kMaxBatchPerLaunch) {
    const int nb = std::min(kMaxBatchPerLaunch, d.B - b0);
    const int wgs = plan_launch(d, geo, ctx_len, b0, nb, G, final_out, a);
    if (wgs > records) return fail(HX_EINVAL, "internal: %d workgroups exceed the %lld workspace records", wgs, (long long)records);
    a.b0 = b0;
    a.nb = nb;
    a.fused_append = fuse ? (fuse->quant ? 2 : 1) : 0;
    if (fuse) a.app = append_batch(*fuse, fuse_pos, nullptr, b0, nb);
    hipError_t e = geo.kind == 1         ? launch_mla_partial(a, d.dtype, (hipStream_t)stream)
                   : G > kGqaNarrowMaxHeads ? launch_gqa_wide(a, d.dtype, (hipStream_t)stream)
                                            : launch_gqa_partial(a, d.dtype, (hipStream_t)stream);
    s = check_hip(e, "decode_attn_partial launch");
    if (s) return s;
    if (wgs > 0)
      trace_mark(geo.kind == 1 ? "mla_partial" : (G > kGqaNarrowMaxHeads ? "gqa_wide_partial" : "gqa_partial"),
                 (hipStream_t)stream);
    s = final_out ? check_hip(launch_fold_combine(a, o_final, lse_final, (hipStream_t)stream), "fold/combine launch")
                  : check_hip(launch_split_fold(a, (hipStream_t)stream), "split fold launch");
    if (s) return s;
    if (final_out)
      trace_mark("fold_combine", (hipStream_t)stream);
    else if (a.fold_begin[nb] > 0)
      trace_mark("split_fold", (hipStream_t)stream);
  }
  return HX_OK;
}

}  // namespace hx

extern "C" {

hx_status hx_decode_attn_partial(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* q, int32_t Hq,
                                 const int64_t* ctx_len, float scale, float* o_part, float* lse_part, void* ws,
                                 size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  return decode_step(desc, cache, PoolRef{nullptr, 0}, q, Hq, ctx_len, scale, o_part, lse_part, ws, ws_bytes, stream,
                     nullptr, nullptr);
}

hx_status hx_decode_attn(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* q, int32_t Hq,
                         const int64_t* ctx_len, float scale, float* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  g_err[0] = 0;
  if (!o) return fail(HX_EINVAL, "null argument");
  return decode_step(desc, cache, PoolRef{nullptr, 0}, q, Hq, ctx_len, scale, nullptr, nullptr, ws, ws_bytes, stream,
                     o, lse);
}

}  // extern "C"

namespace hx {

// The fixed scratch of hx_decode_attn_noalloc.  In host code `scratch` is a
// host-side stand-in, not a device address: its device address (one per
// GPU, each GPU holding its own copy) comes from hipGetSymbolAddress, taken
// once per device on the entry point's first call there, and only that
// address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static hx_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = -1;
  hx_status s = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (s) return s;
  if (dev < 0 || dev >= 64) return fail(HX_EUNSUPPORTED, "device %d: at most 64 devices are supported", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    s = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (s) return s;
    if (!p) return fail(HX_EHIP, "hipGetSymbolAddress(scratch) returned a null address");
    addr[dev] = p;
  }
  *out = addr[dev];
  return HX_OK;
}

}  // namespace hx

extern "C" {

hx_status hx_decode_attn_noalloc(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* q, int32_t Hq,
                                 const int64_t* ctx_len, float scale, float* o, float* lse, void* stream) {
  g_err[0] = 0;
  if (!o) return fail(HX_EINVAL, "null argument");
  // every argument (and the scratch size this call needs) first, then the
  // device's scratch address, then the launches
  hx_status s = decode_step(desc, cache, PoolRef{nullptr, 0}, q, Hq, ctx_len, scale, nullptr, nullptr, nullptr,
                            kScratchBytes, stream, o, lse, nullptr, nullptr, true, true);
  if (s) return s;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s) return s;
  return decode_step(desc, cache, PoolRef{nullptr, 0}, q, Hq, ctx_len, scale, nullptr, nullptr, ws, kScratchBytes,
                     stream, o, lse, nullptr, nullptr, false, true);
}

hx_status hx_decode_attn_partial_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* q, int32_t Hq,
                                       const int64_t* ctx_len, float scale, float* o_part, float* lse_part, void* ws,
                                       size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  PoolRef ref;
  hx_status s = check_pool(desc, pool, &ref);
  if (s) return s;
  return decode_step(desc, &pool->planes, ref, q, Hq, ctx_len, scale, o_part, lse_part, ws, ws_bytes, stream, nullptr,
                     nullptr);
}

hx_status hx_decode_attn_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* q, int32_t Hq,
                               const int64_t* ctx_len, float scale, float* o, float* lse, void* ws, size_t ws_bytes,
                               void* stream) {
  g_err[0] = 0;
  PoolRef ref;
  hx_status s = check_pool(desc, pool, &ref);
  if (s) return s;
  if (!o) return fail(HX_EINVAL, "null argument");
  return decode_step(desc, &pool->planes, ref, q, Hq, ctx_len, scale, nullptr, nullptr, ws, ws_bytes, stream, o, lse);
}

}  // extern "C"

namespace hx {

// hx_decode_step: rows [ctx_len[b] - n_new, ctx_len[b]) of every request are
// the step's new rows; append them inside the partial pass, then fold.
static hx_status fused_step(const hx_kv_desc* desc, const hx_kv_cache* cache, PoolRef pool, const void* k_new,
                            const void* v_new, const void* k_scale_new, const void* v_scale_new, int32_t n_new,
                            const void* q, int32_t Hq, const int64_t* ctx_len, float scale, float* o, float* lse,
                            void* ws, size_t ws_bytes, void* stream) {
  if (!desc || !ctx_len || !o || !lse) return fail(HX_EINVAL, "null argument");
  if (desc->B < 1) return fail(HX_EINVAL, "B=%d must be >= 1", desc->B);
  std::vector<int64_t> pos((size_t)desc->B);
  for (int b = 0; b < desc->B; ++b) {
    if (ctx_len[b] < n_new)
      return fail(HX_EINVAL, "ctx_len[%d]=%lld is shorter than the n_new=%d new rows", b, (long long)ctx_len[b], n_new);
    pos[(size_t)b] = ctx_len[b] - n_new;
  }
  AppendArgs base;
  hx_status s = append_setup(desc, cache, pool, k_new, v_new, k_scale_new, v_scale_new, pos.data(), nullptr, n_new,
                             &base);
  if (s) return s;
  // no fused append for MXFP4 codes (see decode_gqa.hip) nor quantised MLA
  // caches (their kernel converts tiles before reading them): append, then attend
  if (desc->dtype == HX_KV_MXFP4 || (desc->v_alias_k && desc->dtype != HX_KV_BF16)) {
    // every argument of the attention is checked before the append writes the
    // cache, so a call that fails leaves the cache unchanged
    s = decode_step(desc, cache, pool, q, Hq, ctx_len, scale, nullptr, nullptr, ws, ws_bytes, stream, o, lse, nullptr,
                    nullptr, true);
    if (s) return s;
    s = kv_append(desc, cache, pool, k_new, v_new, k_scale_new, v_scale_new, pos.data(), nullptr, n_new, stream);
    if (s) return s;
    return decode_step(desc, cache, pool, q, Hq, ctx_len, scale, nullptr, nullptr, ws, ws_bytes, stream, o, lse);
  }
  return decode_step(desc, cache, pool, q, Hq, ctx_len, scale, nullptr, nullptr, ws, ws_bytes, stream, o, lse, &base,
                     pos.data());
}

// hx_decode_step_bf16: the step's new rows as bf16 values, quantised inside
// the partial kernels by the workgroups that own their tiles (fp8, MXFP4);
// a bf16 cache takes them as storage-format rows.
static hx_status quant_step(const hx_kv_desc* desc, const hx_kv_cache* cache, PoolRef pool, const void* k_new,
                            const void* v_new, int32_t n_new, const void* q, int32_t Hq, const int64_t* ctx_len,
                            float scale, float* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!desc || !cache || !ctx_len || !o || !lse) return fail(HX_EINVAL, "null argument");
  if (desc->dtype == HX_KV_BF16)
    return fused_step(desc, cache, pool, k_new, v_new, nullptr, nullptr, n_new, q, Hq, ctx_len, scale, o, lse, ws,
                      ws_bytes, stream);
  if (desc->v_alias_k) {
    // quantised MLA caches: the quantising append kernel, then the attention
    // (every argument of the attention is checked before the cache is written)
    if (desc->B < 1) return fail(HX_EINVAL, "B=%d must be >= 1", desc->B);
    std::vector<int64_t> pos((size_t)desc->B);
    for (int b = 0; b < desc->B; ++b) {
      if (ctx_len[b] < n_new)
        return fail(HX_EINVAL, "ctx_len[%d]=%lld is shorter than the n_new=%d new rows", b, (long long)ctx_len[b],
                    n_new);
      pos[(size_t)b] = ctx_len[b] - n_new;
    }
    hx_status s = decode_step(desc, cache, pool, q, Hq, ctx_len, scale, nullptr, nullptr, ws, ws_bytes, stream, o,
                              lse, nullptr, nullptr, true);
    if (s) return s;
    s = kv_append_bf16(desc, cache, pool, k_new, v_new, pos.data(), nullptr, n_new, stream);
    if (s) return s;
    return decode_step(desc, cache, pool, q, Hq, ctx_len, scale, nullptr, nullptr, ws, ws_bytes, stream, o, lse);
  }
  Geometry g;
  hx_status s = geometry(*desc, &g);
  if (s) return s;
  const hx_kv_desc& d = *desc;
  if (n_new < 1) return fail(HX_EINVAL, "n_new=%d must be >= 1", n_new);
  PlaneRefs pr;
  s = plane_refs(d, g, cache, &pr);
  if (s) return s;
  // here quantised GQA caches (Dk = Dv = 128, separate V); MLA rows took the branch above
  if (!k_new || !v_new) return fail(HX_EINVAL, "null k_new or v_new");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(HX_EINVAL, "device pointers must be 16-byte aligned");
  std::vector<int64_t> pos((size_t)d.B);
  for (int b = 0; b < d.B; ++b) {
    if (ctx_len[b] < n_new)
      return fail(HX_EINVAL, "ctx_len[%d]=%lld is shorter than the n_new=%d new rows", b, (long long)ctx_len[b], n_new);
    pos[(size_t)b] = ctx_len[b] - n_new;
  }
  AppendArgs a{};
  a.src[0] = (const uint8_t*)k_new;
  a.src[1] = (const uint8_t*)v_new;
  for (int i = 0; i < 4; ++i) {
    a.dst[i] = pr.base[i];
    a.tile_stride[i] = pr.stride[i];
  }
  a.lay[0] = g.lay_k;
  a.lay[1] = g.lay_v;
  a.width[0] = a.width[1] = d.Dk;
  a.src_row_bytes[0] = a.src_row_bytes[1] = (int64_t)d.Dk * 2;   // bf16 rows
  a.nplanes = 2;
  a.P = d.P;
  a.B = d.B;
  a.Hkv = d.Hkv;
  a.cap_chunks = d.cap / kChunk;
  a.table = pool.table;
  a.num_blocks = pool.num_blocks;
  a.n_new = n_new;
  a.quant = d.dtype;
  return decode_step(desc, cache, pool, q, Hq, ctx_len, scale, nullptr, nullptr, ws, ws_bytes, stream, o, lse, &a,
                     pos.data());
}

}  // namespace hx

extern "C" {

hx_status hx_decode_step_bf16(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* k_new, const void* v_new,
                              int32_t n_new, const void* q, int32_t Hq, const int64_t* ctx_len, float scale, float* o,
                              float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  return quant_step(desc, cache, PoolRef{nullptr, 0}, k_new, v_new, n_new, q, Hq, ctx_len, scale, o, lse, ws, ws_bytes,
                    stream);
}

hx_status hx_decode_step_bf16_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* k_new,
                                    const void* v_new, int32_t n_new, const void* q, int32_t Hq,
                                    const int64_t* ctx_len, float scale, float* o, float* lse, void* ws,
                                    size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  PoolRef ref;
  hx_status s = check_pool(desc, pool, &ref);
  if (s) return s;
  return quant_step(desc, &pool->planes, ref, k_new, v_new, n_new, q, Hq, ctx_len, scale, o, lse, ws, ws_bytes,
                    stream);
}

hx_status hx_decode_step(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* k_new, const void* v_new,
                         const void* k_scale_new, const void* v_scale_new, int32_t n_new, const void* q, int32_t Hq,
                         const int64_t* ctx_len, float scale, float* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  g_err[0] = 0;
  return fused_step(desc, cache, PoolRef{nullptr, 0}, k_new, v_new, k_scale_new, v_scale_new, n_new, q, Hq, ctx_len,
                    scale, o, lse, ws, ws_bytes, stream);
}

hx_status hx_decode_step_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* k_new, const void* v_new,
                               const void* k_scale_new, const void* v_scale_new, int32_t n_new, const void* q,
                               int32_t Hq, const int64_t* ctx_len, float scale, float* o, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  PoolRef ref;
  hx_status s = check_pool(desc, pool, &ref);
  if (s) return s;
  return fused_step(desc, &pool->planes, ref, k_new, v_new, k_scale_new, v_scale_new, n_new, q, Hq, ctx_len, scale,
                    o, lse, ws, ws_bytes, stream);
}

hx_status hx_lse_combine(int32_t P, int32_t B, int32_t Hq, int32_t Dv, const float* o_part, const float* lse_part,
                         float* o, float* lse, void* stream) {
  g_err[0] = 0;
  if (!o_part || !lse_part || !o || !lse) return fail(HX_EINVAL, "null argument");
  if (P < 1 || P > 1024 || B < 1 || Hq < 1 || Dv < 1) return fail(HX_EINVAL, "need 1 <= P <= 1024 and B, Hq, Dv >= 1");
  const void* ptrs[4] = {o_part, lse_part, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(HX_EINVAL, "device pointers must be 16-byte aligned");
  hx_status s = check_hip(launch_lse_combine(P, B, Hq, Dv, o_part, lse_part, o, lse, (hipStream_t)stream),
                          "lse_combine launch");
  if (!s) trace_mark("lse_combine", (hipStream_t)stream);
  return s;
}

hx_status hx_trace_begin(int32_t capacity, void* stream) {
  g_err[0] = 0;
  if (capacity < 1 || capacity > (1 << 20)) return fail(HX_EINVAL, "capacity=%d must be in 1..2^20", capacity);
  std::lock_guard<std::mutex> lk(g_trace.mu);
  if (g_trace.open) return fail(HX_EINVAL, "a trace is already open");
  std::vector<hipEvent_t> ev;
  hipEvent_t start = nullptr;
  hx_status s = check_hip(hipEventCreate(&start), "hipEventCreate");
  for (int i = 0; !s && i < capacity; ++i) {
    hipEvent_t e = nullptr;
    s = check_hip(hipEventCreate(&e), "hipEventCreate");
    if (!s) ev.push_back(e);
  }
  if (!s) s = check_hip(hipEventRecord(start, (hipStream_t)stream), "hipEventRecord");
  if (s) {
    for (hipEvent_t e : ev) hipEventDestroy(e);
    if (start) hipEventDestroy(start);
    return s;
  }
  g_trace.ev.swap(ev);
  g_trace.start = start;
  g_trace.names.assign((size_t)capacity * kTraceName, 0);
  g_trace.cap = capacity;
  g_trace.n = 0;
  g_trace.overflow = false;
  g_trace.open = true;
  g_trace_open.store(true, std::memory_order_release);
  return HX_OK;
}

hx_status hx_trace_mark(const char* name, void* stream) {
  g_err[0] = 0;
  if (!name) return fail(HX_EINVAL, "null argument");
  if (!g_trace_open.load(std::memory_order_acquire)) return fail(HX_EINVAL, "no trace is open");
  trace_mark(name, (hipStream_t)stream);
  return HX_OK;
}

hx_status hx_trace_end(int32_t* n, float* ms, char* names) {
  g_err[0] = 0;
  if (!n || !ms || !names) return fail(HX_EINVAL, "null argument");
  std::lock_guard<std::mutex> lk(g_trace.mu);
  if (!g_trace.open) return fail(HX_EINVAL, "no trace is open");
  g_trace_open.store(false, std::memory_order_release);
  g_trace.open = false;
  hx_status s = HX_OK;
  if (g_trace.n > 0) s = check_hip(hipEventSynchronize(g_trace.ev[g_trace.n - 1]), "hipEventSynchronize");
  for (int i = 0; !s && i < g_trace.n; ++i)
    s = check_hip(hipEventElapsedTime(&ms[i], i ? g_trace.ev[i - 1] : g_trace.start, g_trace.ev[i]),
                  "hipEventElapsedTime");
  if (!s) {
    memcpy(names, g_trace.names.data(), (size_t)g_trace.n * kTraceName);
    *n = g_trace.n;
  }
  for (hipEvent_t e : g_trace.ev) hipEventDestroy(e);
  hipEventDestroy(g_trace.start);
  g_trace.ev.clear();
  g_trace.start = nullptr;
  if (!s && g_trace.overflow)
    return fail(HX_ENOSPC, "more launches than the trace's capacity of %d (the first %d are reported)", g_trace.cap,
                g_trace.n);
  return s;
}

hx_status hx_read_probe(const void* src, int64_t nbytes, uint32_t* out, void* stream) {
  g_err[0] = 0;
  if (!src || !out) return fail(HX_EINVAL, "null argument");
  if (!aligned16(src)) return fail(HX_EINVAL, "src must be 16-byte aligned");
  if (nbytes <= 0 || nbytes % 16 != 0) return fail(HX_EINVAL, "nbytes=%lld must be a positive multiple of 16",
                                                   (long long)nbytes);
  hx_status s = check_hip(launch_read_probe(src, nbytes, out, HX_READ_PROBE_BLOCKS, (hipStream_t)stream),
                          "read_probe launch");
  if (!s) trace_mark("read_probe", (hipStream_t)stream);
  return s;
}

}  // extern "C"
