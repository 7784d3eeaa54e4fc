// The append of new rows into chunk tiles, as a device function shared by
// the append kernel and the fused decode step (the partial kernels append a
// step's rows into the tiles they own before streaming them).
//
// Placement (Helix summary, paragraph on Helix's two layouts; NVIDIA blog,
// section on distributed KV placement): token t of a request belongs to the
// 16-token group c = t / 16, which lives in slice c mod P as that slice's
// (c / P)-th chunk tile.  One call owns destination bytes, not source
// tokens: a 16-byte piece of one chunk tile of one plane, built from the new
// rows that fall in it and the stored bytes of the others.  No two pieces
// share bytes, so concurrent calls on different pieces do not depend on
// their order, and bytes move unconverted (bit-exact).
#pragma once

#include "hx_common.h"
#include "hx_quant.h"

namespace hx {

// 16-byte pieces of all planes of one chunk tile (a fp8 group scale counts
// as one piece).
__device__ __forceinline__ int64_t append_pieces(const AppendArgs& a, int64_t* pieces) {
  int64_t sum = 0;
  for (int p = 0; p < a.nplanes; ++p) {
    pieces[p] = a.ebits[p] == 32 ? 1 : (a.tile_bytes[p] + 15) / 16;
    sum += pieces[p];
  }
  return sum;
}

// Piece `piece` (over all planes, in plane order) of the chunk tile holding
// request-level group pos / 16 + ci of request bl of the launch, KV head g.
__device__ __forceinline__ void append_piece(const AppendArgs& a, int bl, int g, int ci, int64_t piece) {
  int64_t pieces[4];
  append_pieces(a, pieces);
  int plane = 0;
  while (piece >= pieces[plane]) piece -= pieces[plane++];

  const int b = a.b0 + bl;
  const int64_t pos = a.pos[bl];
  const int64_t end = pos + a.count[bl];
  const int64_t c = pos / kChunk + ci;           // request-level chunk (group) index
  const int64_t row0 = c * kChunk;
  if (end == pos || row0 >= end) return;   // nothing of this request lands in this chunk
  int r;
  int64_t lc;
  if (c <= 0xffffffffll) {
    r = (int)((uint32_t)c % (uint32_t)a.P);
    lc = (uint32_t)c / (uint32_t)a.P;
  } else {
    r = (int)(c % a.P);
    lc = c / a.P;
  }
  const int64_t tile = tile_of(TileMap{a.table, a.num_blocks, a.P, a.B, a.Hkv, a.cap_chunks}, r, b, g, lc);
  const int64_t src_tok0 = ((int64_t)bl * a.Hkv + g) * a.n_new;   // token-major source, this launch's rows
  const uint8_t* src = a.src[plane];
  uint8_t* dst = a.dst[plane] + tile * a.tile_stride[plane];

  if (a.ebits[plane] == 32) {
    // one fp32 scale per chunk: a chunk whose first row is new takes the scale
    // of that row; a chunk that already holds rows keeps its stored scale
    if (row0 < pos) return;
    const float v = reinterpret_cast<const float*>(src)[src_tok0 + (row0 - pos)];
    *reinterpret_cast<float*>(dst) = v;
    return;
  }

  const int64_t byte0 = piece * 16;
  const int nbytes = (int)((a.tile_bytes[plane] - byte0) < 16 ? (a.tile_bytes[plane] - byte0) : 16);
  const int eb = a.ebits[plane];
  const int lay = a.lay[plane], width = a.width[plane];
  const int64_t srow = a.src_row_bytes[plane];
  const int nelem = eb == 16 ? nbytes / 2 : (eb == 8 ? nbytes : 2 * nbytes);
  auto elem_off2 = [&](int e) -> int64_t {
    return eb == 16 ? 2 * (byte0 + 2 * e) : (eb == 8 ? 2 * (byte0 + e) : 2 * byte0 + e);
  };
  // a piece holding none of the new rows stays as it is: first a cheap test
  // on the piece's row range, then the exact one
  {
    int mlo, mhi;
    piece_rows(lay, width, byte0, nbytes, &mlo, &mhi);
    if (row0 + mhi < pos || row0 + mlo >= end) return;
  }
  bool any = false;
  for (int e = 0; e < nelem; ++e) {
    int mm, d;
    tile_inv(lay, width, elem_off2(e), &mm, &d);
    any |= row0 + mm >= pos && row0 + mm < end;
  }
  if (!any) return;
  const bool whole = row0 >= pos && row0 + kChunk <= end;
  if (!whole && nbytes == 16 && eb != 4) {
    // part of the piece is new (a decode step's row): store just the new 1- or
    // 2-byte elements, so the stored bytes of other rows are not read; every
    // source element is loaded before the first store (the source and the
    // planes might alias as far as the compiler knows, so interleaved loads
    // and stores would serialise on memory latency)
    if (eb == 16) {
      uint16_t v[8];
      bool nw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int mm, d;
        tile_inv(lay, width, elem_off2(e), &mm, &d);
        const int64_t tok = row0 + mm;
        nw[e] = tok >= pos && tok < end;
        v[e] = nw[e] ? *reinterpret_cast<const uint16_t*>(src + (src_tok0 + (tok - pos)) * srow + 2 * d) : 0;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (nw[e]) *reinterpret_cast<uint16_t*>(dst + byte0 + 2 * e) = v[e];
    } else {
      uint8_t v[16];
      bool nw[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int mm, d;
        tile_inv(lay, width, elem_off2(e), &mm, &d);
        const int64_t tok = row0 + mm;
        nw[e] = tok >= pos && tok < end;
        v[e] = nw[e] ? src[(src_tok0 + (tok - pos)) * srow + d] : 0;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (nw[e]) dst[byte0 + e] = v[e];
    }
    return;
  }
  uint8_t buf[16];
  if (nbytes == 16) {
    const uint4 v = whole ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4*>(dst + byte0);
    __builtin_memcpy(buf, &v, 16);
  } else {
    for (int i = 0; i < nbytes; ++i) buf[i] = dst[byte0 + i];
  }
  for (int e = 0; e < nelem; ++e) {
    int mm, d;
    tile_inv(lay, width, elem_off2(e), &mm, &d);
    const int64_t tok = row0 + mm;
    if (tok < pos || tok >= end) continue;
    const uint8_t* srcrow = src + (src_tok0 + (tok - pos)) * srow;
    if (eb == 16) {
      buf[2 * e] = srcrow[2 * d];
      buf[2 * e + 1] = srcrow[2 * d + 1];
    } else if (eb == 8) {
      buf[e] = srcrow[d];
    } else {   // 4-bit codes, even element in the low nibble of the source
      const uint8_t sb = srcrow[d >> 1];
      const uint8_t code = (d & 1) ? (sb >> 4) : (sb & 0xf);
      uint8_t& o = buf[e >> 1];
      o = (e & 1) ? (uint8_t)((o & 0x0f) | (code << 4)) : (uint8_t)((o & 0xf0) | code);
    }
  }
  if (nbytes == 16) {
    uint4 v;
    __builtin_memcpy(&v, buf, 16);
    *reinterpret_cast<uint4*>(dst + byte0) = v;
  } else {
    for (int i = 0; i < nbytes; ++i) dst[byte0 + i] = buf[i];
  }
}

}  // namespace hx

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
