// Internal declarations shared by the helixdecode HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "helixdecode.h"

#define HXHD __host__ __device__ __forceinline__

namespace hx {

constexpr int kChunk = HX_CHUNK;   // rows per chunk tile, the placement unit
constexpr int kMaxBatchPerLaunch = 64;

// ---------------------------------------------------------------- placement
// Token t of a request: group t/16 goes to slice (t/16) mod P as that
// slice's ((t/16)/P)-th group (Helix summary, paragraph on Helix's two
// layouts; NVIDIA blog, section on distributed KV placement).
HXHD int64_t slice_len(int64_t n, int P, int r) {
  const int64_t round = (int64_t)kChunk * P;
  const int64_t full = n / round;
  int64_t left = n - full * round - (int64_t)kChunk * r;
  left = left < 0 ? 0 : (left > kChunk ? kChunk : left);
  return full * kChunk + left;
}

// ---------------------------------------------------------------- tile layouts
// A cache plane is [P][B][Hkv][cap/16] tiles; a tile holds 16 rows.  The
// byte order inside a tile is chosen so that one 16-byte load per lane of a
// 64-lane wave fetches exactly the matrix-core operand fragment a lane
// needs, and every wave-wide load instruction reads 1 KiB contiguous:
//
//  * K tiles feed v_mfma_f32_16x16x32_bf16 as the A operand (rows = 16
//    tokens, k = 32 columns of d per step s): lane l = 16*h + m holds token m,
//    columns 32*s + 8*h .. +7.
//  * V tiles feed v_mfma_f32_16x16x16_bf16 as the A operand of O^T = V^T P^T
//    (rows = 16 columns of dv in block nb, k = 16 tokens): lane l = 16*hq + c
//    holds column 16*nb + c of tokens 4*hq .. 4*hq+3.
//
// Layout ids:
enum Layout : int {
  kLayGqaBf16K = 0, kLayGqaBf16V = 1,
  kLayGqaFp8K = 2, kLayGqaFp8V = 3,
  kLayGqaFp4K = 4, kLayGqaFp4V = 5,
  kLayMlaBf16 = 6,   // bf16 latent rows, 16-byte pieces XOR-swizzled inside each aligned group of 8
  kLayRowU8 = 7,     // plain row-major bytes (MXFP4 e8m0 scale rows, fp8 MLA latent rows)
  kLayRowU4 = 8,     // plain row-major 4-bit elements, the even one in the low nibble (MXFP4 MLA latent rows)
};

// MLA latent rows (1152 B = 72 pieces of 16 B): piece p of row m is stored at
// piece position p ^ mla_swz(m), a permutation inside each aligned group of 8
// pieces.  A row spans 72 16-byte LDS bank slots, so rows of equal parity
// start in the same slot.  The swizzle gives the 8 rows of each parity among
// 16 consecutive rows 8 different slots for one piece (the score operand: 32
// rows, one piece per half-wave), and maps rows m and m + 2 of an aligned
// group of 4 to opposite halves of the 8-piece group (the transposed value
// operand: 4 rows, 4 adjacent pieces).  Measured on gfx950 LDS for the score
// reads with eight waves per CU: about 200 B/clk/CU against 62 unswizzled.  Rows copied to LDS
// unchanged are then read efficiently in both views.
HXHD int mla_swz(int m) { return 4 * ((m >> 1) & 1) + ((m >> 2) & 3); }

// ---------------------------------------------------------------- lane exchanges
// x combined with lane l ^ 16 (resp. l ^ 32) of the wave through the gfx950
// row-swap permutes, VALU instructions without an LDS round trip: with x as
// both operands, v_permlane16_swap leaves lanes l and l ^ 16 each holding
// x[l] and x[l ^ 16] across its two results (v_permlane32_swap likewise for
// l ^ 32), in the same order on both lanes, so both get the same bits.
__device__ __forceinline__ uint2 swap_rows16(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_uint2(s[0], s[1]);
#else
  return make_uint2(__float_as_uint(x), __float_as_uint(x));   // host pass: never called
#endif
}
__device__ __forceinline__ uint2 swap_rows32(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_uint2(s[0], s[1]);
#else
  return make_uint2(__float_as_uint(x), __float_as_uint(x));   // host pass: never called
#endif
}
// max(a, b) as one v_med3_f32(a, b, +inf).  fmaxf under the IEEE mode that
// kernels run in makes the compiler quiet every operand it cannot prove
// canonical (matrix-core results, lane permutes) with an extra v_max_f32
// x, x first; the median against +inf needs none.  The +inf is opaque to
// the optimiser, which would otherwise fold the median back into fmaxf.
__device__ __forceinline__ float vmax(float a, float b) {
#if defined(__HIP_DEVICE_COMPILE__)
  float inf = INFINITY;
  asm("" : "+v"(inf));
  return __builtin_amdgcn_fmed3f(a, b, inf);
#else
  return a > b ? a : b;   // host pass: never called
#endif
}
__device__ __forceinline__ float max_xor16(float x) {
  const uint2 s = swap_rows16(x);
  return vmax(__uint_as_float(s.x), __uint_as_float(s.y));
}
__device__ __forceinline__ float max_xor32(float x) {
  const uint2 s = swap_rows32(x);
  return vmax(__uint_as_float(s.x), __uint_as_float(s.y));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const uint2 s = swap_rows16(x);
  return __uint_as_float(s.x) + __uint_as_float(s.y);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const uint2 s = swap_rows32(x);
  return __uint_as_float(s.x) + __uint_as_float(s.y);
}

// Element (row m, column d) -> 2 * byte offset + nibble (nibble is 1 for the
// high half of an FP4 byte).  `width` is the row width for row layouts.
HXHD int64_t tile_off2(int lay, int width, int m, int d) {
  switch (lay) {
    case kLayGqaBf16K: {
      const int s = d >> 5, h = (d >> 3) & 3, e = d & 7;
      return 2 * (int64_t)(s * 1024 + (h * 16 + m) * 16 + e * 2);
    }
    case kLayGqaBf16V: {
      const int nb = d >> 4, c = d & 15, hq = m >> 2, j = m & 3;
      return 2 * (int64_t)((nb >> 1) * 1024 + (hq * 16 + c) * 16 + (nb & 1) * 8 + j * 2);
    }
    case kLayGqaFp8K: {
      const int s = d >> 5, h = (d >> 3) & 3, e = d & 7;
      return 2 * (int64_t)((s >> 1) * 1024 + (h * 16 + m) * 16 + (s & 1) * 8 + e);
    }
    case kLayGqaFp8V: {
      const int nb = d >> 4, c = d & 15, hq = m >> 2, j = m & 3;
      return 2 * (int64_t)((nb >> 2) * 1024 + (hq * 16 + c) * 16 + (nb & 3) * 4 + j);
    }
    case kLayGqaFp4K: {
      const int s = d >> 5, h = (d >> 3) & 3, e = d & 7;
      const int ni = s * 8 + e;
      return 2 * (int64_t)((h * 16 + m) * 16 + (ni >> 1)) + (ni & 1);
    }
    case kLayGqaFp4V: {
      const int nb = d >> 4, c = d & 15, hq = m >> 2, j = m & 3;
      const int ni = nb * 4 + j;
      return 2 * (int64_t)((hq * 16 + c) * 16 + (ni >> 1)) + (ni & 1);
    }
    case kLayMlaBf16: {
      const int p = (d >> 3) ^ mla_swz(m);
      return 2 * ((int64_t)m * width * 2 + p * 16 + (d & 7) * 2);
    }
    case kLayRowU4:
      return (int64_t)m * width + d;
    case kLayRowU8:
    default:
      return 2 * ((int64_t)m * width + d);
  }
}

// Inverse: (2 * byte offset + nibble) of an element -> (m, d).  Used by the
// append kernel, which owns destination bytes.  `ebits` is the element size.
HXHD void tile_inv(int lay, int width, int64_t off2, int* m, int* d) {
  const int b = (int)(off2 >> 1);
  const int nib = (int)(off2 & 1);
  switch (lay) {
    case kLayGqaBf16K: {
      const int s = b >> 10, lane = (b >> 4) & 63, e = (b >> 1) & 7;
      *m = lane & 15;
      *d = s * 32 + (lane >> 4) * 8 + e;
      return;
    }
    case kLayGqaBf16V: {
      const int p = b >> 10, lane = (b >> 4) & 63, w = (b >> 1) & 7;
      *m = (lane >> 4) * 4 + (w & 3);
      *d = (2 * p + (w >> 2)) * 16 + (lane & 15);
      return;
    }
    case kLayGqaFp8K: {
      const int i = b >> 10, lane = (b >> 4) & 63, w = b & 15;
      const int s = 2 * i + (w >> 3);
      *m = lane & 15;
      *d = s * 32 + (lane >> 4) * 8 + (w & 7);
      return;
    }
    case kLayGqaFp8V: {
      const int i = b >> 10, lane = (b >> 4) & 63, w = b & 15;
      *m = (lane >> 4) * 4 + (w & 3);
      *d = (4 * i + (w >> 2)) * 16 + (lane & 15);
      return;
    }
    case kLayGqaFp4K: {
      const int lane = b >> 4, ni = (b & 15) * 2 + nib;
      *m = lane & 15;
      *d = (ni >> 3) * 32 + (lane >> 4) * 8 + (ni & 7);
      return;
    }
    case kLayGqaFp4V: {
      const int lane = b >> 4, ni = (b & 15) * 2 + nib;
      *m = (lane >> 4) * 4 + (ni & 3);
      *d = (ni >> 2) * 16 + (lane & 15);
      return;
    }
    case kLayMlaBf16: {
      const int row = b / (width * 2);
      const int p = ((b % (width * 2)) >> 4) ^ mla_swz(row);
      *m = row;
      *d = p * 8 + ((b & 15) >> 1);
      return;
    }
    case kLayRowU4: {
      const int64_t e = off2;   // element index: two per byte
      *m = (int)(e / width);
      *d = (int)(e % width);
      return;
    }
    case kLayRowU8:
    default:
      *m = b / width;
      *d = b % width;
      return;
  }
}

// Rows [*mlo, *mhi] that the 16-byte piece at byte0 of a tile can hold
// (a superset: the exact test follows).
HXHD void piece_rows(int lay, int width, int64_t byte0, int nbytes, int* mlo, int* mhi) {
  const int b = (int)byte0;
  switch (lay) {
    case kLayGqaBf16K:
    case kLayGqaFp8K:
    case kLayGqaFp4K:   // lane l = 16 h + m holds one token m
      *mlo = *mhi = (b >> 4) & 15;
      return;
    case kLayGqaBf16V:
    case kLayGqaFp8V:
    case kLayGqaFp4V: {   // lane l = 16 hq + c holds tokens 4 hq .. 4 hq + 3
      const int hq = ((b >> 4) & 63) >> 4;
      *mlo = 4 * hq;
      *mhi = 4 * hq + 3;
      return;
    }
    case kLayMlaBf16:     // pieces never straddle a 1,152-byte row
      *mlo = *mhi = b / (width * 2);
      return;
    case kLayRowU4:       // row-major nibbles
      *mlo = 2 * b / width;
      *mhi = (2 * (b + nbytes) - 1) / width;
      return;
    default:              // row-major bytes
      *mlo = b / width;
      *mhi = (b + nbytes - 1) / width;
      return;
  }
}

// ---------------------------------------------------------------- tile addressing
// Dense cache: tile (slice r, request b, KV head g, local 16-row group c) is
// tile ((r * B + b) * Hkv + g) * cap_chunks + c of every plane.  Block pool:
// group c of slice r of request b is block table[(b * P + r) * cap_chunks +
// c]; a block holds the tiles of all Hkv heads, so the tile is
// block * Hkv + g.  Block ids outside [0, num_blocks) are clamped into it:
// a bad table reads wrong rows but never leaves the planes.
struct TileMap {
  const int32_t* table;   // device [B][P][cap_chunks]; null for a dense cache
  int32_t num_blocks;
  int P, B, Hkv;
  int64_t cap_chunks;
};

HXHD int64_t clamp_block(int32_t blk, int32_t num_blocks) {
  return blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
}

HXHD int64_t tile_of(const TileMap& m, int r, int b, int g, int64_t c) {
  if (!m.table) return ((int64_t)(r * m.B + b) * m.Hkv + g) * m.cap_chunks + c;
  return clamp_block(m.table[((int64_t)b * m.P + r) * m.cap_chunks + c], m.num_blocks) * m.Hkv + g;
}

// ---------------------------------------------------------------- cache geometry
struct Geometry {
  int kind;            // 0 GQA (Dk = Dv = 128), 1 MLA (576 / 512, aliased)
  int lay_k, lay_v;    // tile layouts of the K and V code planes
  int ebits;           // bits per code element: 16, 8 or 4
  int64_t k_tile, v_tile;          // code bytes per chunk tile
  int64_t ks_tile, vs_tile;        // scale bytes per chunk tile (0 = none)
  int64_t tiles;                   // P * B * Hkv * cap / 16
  // MXFP4: the four parts of a chunk tile (K codes, V codes, K scales, V
  // scales) are stored together, `packed_tile` bytes per tile in one plane,
  // so a workgroup streams one contiguous run instead of four
  bool packed;
  int64_t packed_tile;
};

// Fills `g` from a validated descriptor; returns HX_EUNSUPPORTED for a
// combination with no kernel.
hx_status geometry(const hx_kv_desc& d, Geometry* g);

// Error reporting (thread-local message; entry points clear it first).
hx_status fail(hx_status s, const char* fmt, ...);
void clear_error();
hx_status check_hip(hipError_t e, const char* what);

// ---------------------------------------------------------------- launchers
// Append of storage-format rows (hx_kv_append; also fused into a decode
// step's partial kernels).
struct AppendArgs {
  const uint8_t* src[4];   // k codes, v codes, k scales, v scales (token-major)
  uint8_t* dst[4];         // planes
  int lay[4];              // tile layout per plane
  int width[4];            // row width (row layouts)
  int ebits[4];            // element bits per plane (16, 8, 4; 32 = fp8 group scale)
  int64_t src_row_bytes[4];
  int64_t tile_bytes[4];   // bytes of a chunk tile's part in this plane
  int64_t tile_stride[4];  // bytes between consecutive chunk tiles of this plane
  int nplanes;
  int P, B, Hkv;
  int64_t cap_chunks;
  const int32_t* table;    // pool cache block table (null: dense)
  int32_t num_blocks;
  int n_new;
  int max_chunks;          // largest number of chunks one request touches
  int64_t pos[kMaxBatchPerLaunch];
  int32_t count[kMaxBatchPerLaunch];
  int b0;                  // first request of this launch
  // 0: src holds storage-format rows, copied.  HX_KV_FP8_E4M3 / HX_KV_MXFP4:
  // src[0], src[1] hold bf16 K and V rows (width[0] = D), quantised into the
  // code planes dst[0], dst[1] and the scale planes dst[2], dst[3]
  // (quant_tile in hx_quant.h)
  int quant;
};

struct PartialArgs {
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* ks;
  const uint8_t* vs;
  const uint16_t* q;       // bf16 bits [Btot][Hq][Dk]
  float* o_part;           // [P][Btot][Hq][Dv]
  float* lse_part;         // [P][Btot][Hq]
  float* ws_o;             // [records][G][Dv]
  float* ws_lse;           // [records][G]
  int P, Btot, b0, nb, Hkv, Hq, G, Dk, Dv;
  int64_t cap_chunks;
  const int32_t* table;    // block table of a pool cache (tile addressing above); null: dense
  int32_t num_blocks;
  int64_t k_tile, v_tile, ks_tile, vs_tile;   // bytes between consecutive tiles of each plane
  float c2;                // softmax scale * log2(e)
  int split_p;             // MLA: P as bf16 high part + residual (else rounded once)
  int fused_append;        // the workgroups first append app's rows into the tiles they own:
                           // 0 no, 1 storage-format rows, 2 bf16 rows quantised (app.quant)
  AppendArgs app;          // (same requests as this launch: app.b0 = b0)
  int cpw;                 // chunks per workgroup (split size), the largest over the requests
  int waves;               // GQA: waves per workgroup (kGqaWavesPerWg, or kGqaShortWaves for unsplit slices)
  int64_t n[kMaxBatchPerLaunch];
  int nsplit[kMaxBatchPerLaunch];
  int cpw_b[kMaxBatchPerLaunch];            // split size of each request: its slices' tiles spread evenly
  int wg_begin[kMaxBatchPerLaunch + 1];     // first workgroup (= split record) of each request; [nb]: the total
  int fold_begin[kMaxBatchPerLaunch + 1];   // first fold workgroup of each request
  // dispatch order: the requests' workgroup ranges follow one another in the
  // order order[0], order[1], ... (longest splits first), the range of
  // order[i] starting at workgroup pos_begin[i] (= wg_begin[order[i]])
  int order[kMaxBatchPerLaunch];
  int pos_begin[kMaxBatchPerLaunch + 1];
};
HXHD TileMap tile_map(const PartialArgs& a) { return TileMap{a.table, a.num_blocks, a.P, a.Btot, a.Hkv, a.cap_chunks}; }

// The request (index in the launch) that workgroup wg belongs to, and wg's
// index among that request's workgroups.
__device__ __forceinline__ int request_of(const PartialArgs& a, int wg, int* rem) {
  int i = 0;
  while (i + 1 < a.nb && a.pos_begin[i + 1] <= wg) ++i;
  *rem = wg - a.pos_begin[i];
  return a.order[i];
}

hipError_t launch_gqa_partial(const PartialArgs& a, int dtype, hipStream_t st);
// GQA groups of more than 16 query heads (decode_gqa_wide.hip): tiles in
// pairs, so split sizes (cpw) are even.
constexpr int kGqaNarrowMaxHeads = 16;
constexpr int kGqaWideMaxHeads = 128;
hipError_t launch_gqa_wide(const PartialArgs& a, int dtype, hipStream_t st);
// dtype: the latent rows' format (bf16 tiles are read as stored; fp8 and
// MXFP4 tiles are converted to bf16 in LDS first)
hipError_t launch_mla_partial(const PartialArgs& a, int dtype, hipStream_t st);
// Folds the split records of every slice with more than one split into the
// slice outputs (o_part, lse_part); no-op when every slice has one split.
hipError_t launch_split_fold(const PartialArgs& a, hipStream_t st);

// hx_decode_attn's completion: folds every (slice, split) partial of each
// (request, query head) - the slice outputs of one-split slices, the split
// records of the others - into the final O and LSE in one pass.
hipError_t launch_fold_combine(const PartialArgs& a, float* o, float* lse, hipStream_t st);

hipError_t launch_lse_combine(int P, int B, int Hq, int Dv, const float* o_part, const float* lse_part, float* o,
                              float* lse, hipStream_t st);

// Plain streaming read of nbytes (a multiple of 16) by nblocks workgroups;
// out[i] receives the XOR of what workgroup i read (read_probe.hip).
hipError_t launch_read_probe(const void* src, int64_t nbytes, uint32_t* out, int nblocks, hipStream_t st);

// Split policy shared by hx_workspace_size and hx_decode_attn_partial.
constexpr int kGqaWavesPerWg = 4;
// Short slices (not split) are latency-bound: their one workgroup per slice
// gets more waves, each with fewer tiles in its chain.
#ifndef HX_GQA_SHORT_WAVES
#define HX_GQA_SHORT_WAVES 8
#endif
constexpr int kGqaShortWaves = HX_GQA_SHORT_WAVES;
constexpr int kGqaTargetWgs = 2048;   // upper bound on the split target
constexpr int kMlaTargetWgs = 1024;
constexpr int kMaxSplits = 256;       // splits per slice (the fold keeps their weights in LDS)
int target_wgs(int kind, int dtype, int G);  // device-dependent, <= the bounds above
int min_chunks_per_wg(int kind);

}  // namespace hx
