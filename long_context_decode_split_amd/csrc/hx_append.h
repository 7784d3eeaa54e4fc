// The append of a decode step's new rows into the chunk tiles it owns, as
// device functions the partial kernels run before streaming those tiles
// (hx_decode_step, hx_decode_step_bf16): the storage-format copy through
// the forward tile map (append_rows) and the quantising form (fused_quant,
// with quant_tile of hx_quant.h, the append kernel's own encoder).  The
// standalone append kernel (kv_cache.hip) owns destination bytes instead.
//
// Placement (Helix summary, paragraph on Helix's two layouts; NVIDIA blog,
// section on distributed KV placement): token t of a request belongs to the
// 16-token group c = t / 16, which lives in slice c mod P as that slice's
// (c / P)-th chunk tile.
#pragma once

#include "hx_common.h"
#include "hx_quant.h"

namespace hx {

// The new rows of request-level group c (request bl of the launch, KV head
// g), written element by element through the forward tile map: the threads
// tid, tid + nthr, ... of a workgroup take the new (row, column) elements of
// every plane; 4-bit planes go by destination byte (a byte of a K tile holds
// two columns of one row, a byte of a V tile the same column of two rows,
// rewritten together).  Cheap when few rows are new (a decode step).
__device__ __forceinline__ void append_rows(const AppendArgs& a, int bl, int g, int64_t c, int tid, int nthr) {
  const int64_t pos = a.pos[bl], end = pos + a.count[bl];
  const int64_t row0 = c * kChunk;
  const int mlo = (int)((pos > row0 ? pos : row0) - row0);
  const int mhi = (int)((end < row0 + kChunk ? end : row0 + kChunk) - row0);   // exclusive
  if (mhi <= mlo) return;
  const int r = (int)(c % a.P);
  const int64_t tile = tile_of(TileMap{a.table, a.num_blocks, a.P, a.B, a.Hkv, a.cap_chunks}, r, a.b0 + bl, g, c / a.P);
  const int64_t src_tok0 = ((int64_t)bl * a.Hkv + g) * a.n_new - pos;   // + token = source row
  for (int p = 0; p < a.nplanes; ++p) {
    const uint8_t* src = a.src[p];
    uint8_t* dst = a.dst[p] + tile * a.tile_stride[p];
    const int64_t srow = a.src_row_bytes[p];
    const int eb = a.ebits[p], lay = a.lay[p], width = a.width[p];
    if (eb == 32) {   // the group's fp8 scale: set when its first row is new, else kept
      if (tid == 0 && mlo == 0) *reinterpret_cast<float*>(dst) = reinterpret_cast<const float*>(src)[src_tok0 + row0];
      continue;
    }
    if (eb == 16 || eb == 8) {
      const int items = (mhi - mlo) * width;
      for (int it = tid; it < items; it += nthr) {
        const int m = mlo + it / width, d = it % width;
        const uint8_t* s = src + (src_tok0 + row0 + m) * srow;
        const int64_t off = tile_off2(lay, width, m, d) >> 1;
        if (eb == 16)
          *reinterpret_cast<uint16_t*>(dst + off) = *reinterpret_cast<const uint16_t*>(s + 2 * d);
        else
          dst[off] = s[d];
      }
      continue;
    }
    if (lay == kLayGqaFp4K) {   // a byte = columns d, d + 1 (d even) of one row, as in the source
      const int items = (mhi - mlo) * (width / 2);
      for (int it = tid; it < items; it += nthr) {
        const int m = mlo + it / (width / 2), d = 2 * (it % (width / 2));
        dst[tile_off2(lay, width, m, d) >> 1] = src[(src_tok0 + row0 + m) * srow + (d >> 1)];
      }
      continue;
    }
    // kLayGqaFp4V: a byte = one column of rows 2k, 2k + 1
    const int klo = mlo >> 1, khi = (mhi + 1) >> 1;
    const int items = (khi - klo) * width;
    for (int it = tid; it < items; it += nthr) {
      const int k = klo + it / width, d = it % width;
      const int64_t o2 = tile_off2(lay, width, 2 * k, d);   // even row: low nibble
      uint8_t byte = dst[o2 >> 1];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int m = 2 * k + q;
        if (m < mlo || m >= mhi) continue;
        const uint8_t sb = src[(src_tok0 + row0 + m) * srow + (d >> 1)];
        const uint8_t code = (d & 1) ? (sb >> 4) : (sb & 0xf);
        byte = q ? (uint8_t)((byte & 0x0f) | (code << 4)) : (uint8_t)((byte & 0xf0) | code);
      }
      dst[o2 >> 1] = byte;
    }
  }
}

// Fused decode step: the partial-kernel workgroup of (request bl, KV head g,
// slice r) that owns the slice's local chunk tiles [c0, c1) first appends the
// step's new rows that fall in them, then holds every wave at a workgroup
// barrier before any tile is read.  The barrier is a workgroup-scope
// release/acquire, so the workgroup's later reads of the tiles (vector loads
// or direct global-to-LDS copies, issued from the same CU) see these stores;
// no other workgroup reads these tiles during the launch.  The new rows are
// the newest of the context, so each lies in some workgroup's range.
// Uniform over the workgroup.
__device__ __forceinline__ void fused_append(const AppendArgs& a, int bl, int g, int r, int64_t c0, int64_t c1) {
  const int64_t pos = a.pos[bl], end = pos + a.count[bl];
  if (end <= pos || c1 <= c0) return;
  const int64_t cf = pos / kChunk, cl = (end - 1) / kChunk;
  const int64_t first = cf + ((r - cf % a.P) % a.P + a.P) % a.P;   // first group of slice r at or after cf
  bool mine = false;
  for (int64_t c = first; c <= cl; c += a.P) mine |= c / a.P >= c0 && c / a.P < c1;
  if (!mine) return;
  for (int64_t c = first; c <= cl; c += a.P) {
    if (c / a.P < c0 || c / a.P >= c1) continue;
    append_rows(a, bl, g, c, threadIdx.x, blockDim.x);
  }
  __syncthreads();
}

// Fused quantising decode step: as fused_append, with the step's new rows
// given as bf16 values (a.quant set) and quantised by the owning workgroup
// into its tiles (quant_tile: the fp8 group's scale grows and its stored
// codes are re-encoded when the new rows need it), K tile then V tile of
// each touched group; then a workgroup barrier before any tile is read.
// Uniform over the workgroup.
__device__ __forceinline__ void fused_quant(const AppendArgs& a, int bl, int g, int r, int64_t c0, int64_t c1) {
  const int64_t pos = a.pos[bl], end = pos + a.count[bl];
  if (end <= pos || c1 <= c0) return;
  const int64_t cf = pos / kChunk, cl = (end - 1) / kChunk;
  const int64_t first = cf + ((r - cf % a.P) % a.P + a.P) % a.P;   // first group of slice r at or after cf
  bool mine = false;
  for (int64_t c = first; c <= cl; c += a.P) mine |= c / a.P >= c0 && c / a.P < c1;
  if (!mine) return;
  __shared__ float s_red[16];
  __shared__ uint8_t s_e[kChunk * (128 / 32)];   // GQA rows: 4 exponent blocks each
  const int D = a.width[0];
  for (int64_t c = first; c <= cl; c += a.P) {
    if (c / a.P < c0 || c / a.P >= c1) continue;
    const int64_t row0 = c * kChunk;
    const int64_t tile = tile_of(TileMap{a.table, a.num_blocks, a.P, a.B, a.Hkv, a.cap_chunks}, r, a.b0 + bl, g, c / a.P);
    for (int p = 0; p < 2; ++p) {
      QuantJob j;
      j.src = reinterpret_cast<const uint16_t*>(a.src[p]) + (((int64_t)bl * a.Hkv + g) * a.n_new + (row0 - pos)) * D;
      j.tile = a.dst[p] + tile * a.tile_stride[p];
      j.sc = a.dst[2 + p] + tile * a.tile_stride[2 + p];
      j.lay = a.lay[p];
      j.D = D;
      j.dtype = a.quant;
      j.m_lo = (int)(pos > row0 ? pos - row0 : 0);
      j.m_hi = (int)(end - row0 < kChunk ? end - row0 : kChunk);
      quant_tile(j, threadIdx.x, blockDim.x, s_red, s_e);
    }
  }
  __syncthreads();
}

}  // namespace hx
