// Arguments and launchers of the cache kernels (append, quantising append,
// row dequantisation).  Kept apart from hx_common.h so that the attention
// kernels do not depend on them.
#pragma once

#include "hx_common.h"

namespace hx {

hipError_t launch_append(const AppendArgs& a, int nb, hipStream_t st);

// Quantising append of bf16 rows into fp8 or MXFP4 planes (D = 128).
struct QAppendArgs {
  const uint16_t* src[2];  // bf16 rows of K and V, token-major [nb][Hkv][n_new][D] for this launch
  uint8_t* dst[2];         // code planes
  uint8_t* sc[2];          // scale planes
  int lay[2];              // tile layouts
  int nplanes;             // 2 (K, V), or 1 when V aliases K
  int dtype;               // HX_KV_FP8_E4M3 or HX_KV_MXFP4
  int D;
  int P, B, Hkv;
  int64_t cap_chunks;
  const int32_t* table;    // pool cache block table (null: dense)
  int32_t num_blocks;
  int64_t tile_stride;     // bytes between consecutive chunk tiles of a code plane
  int64_t sc_tile_stride;  // bytes between consecutive chunk tiles of a scale plane
  int n_new;
  int max_chunks;
  int b0;
  int64_t pos[kMaxBatchPerLaunch];
  int32_t count[kMaxBatchPerLaunch];
};
hipError_t launch_quant_append(const QAppendArgs& a, int nb, hipStream_t st);

struct DequantArgs {
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* ks;
  const uint8_t* vs;
  float* k_out;
  float* v_out;
  int dtype, lay_k, lay_v, Dk, Dv, v_alias;
  int64_t k_tile, v_tile, ks_tile, vs_tile;   // bytes between consecutive tiles of each plane
  TileMap map;             // tile addressing of the cache
  int r, b, g;             // the slice rows read: slice r of request b, KV head g
  int64_t j0, n;
};
hipError_t launch_dequant(const DequantArgs& a, hipStream_t st);

}  // namespace hx
