// Quantising append: new bf16 K/V rows (the output of the QKV projection,
// written round-robin as produced: Helix summary, paragraph on Helix's two
// layouts) encoded on the device into fp8 e4m3 or MXFP4 chunk tiles.
//
// One workgroup owns one (request, KV head, chunk, K or V) tile (K only when
// V aliases K, as in MLA latent rows), so the
// per-chunk fp8 scale, the re-encoding of stored codes when it grows, and
// the bytes of rows that share a 16-byte piece with new rows are all handled
// inside one workgroup (quant_tile in hx_quant.h, which states the rules).

#include "hx_cache.h"
#include "hx_quant.h"

namespace hx {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void quant_append_kernel(const QAppendArgs a) {
  __shared__ float s_red[kThreads / 64];
  __shared__ uint8_t s_e[kChunk * kQuantMaxBlocks];   // MXFP4 exponents of the new rows
  int t = blockIdx.x;
  const int plane = t % a.nplanes;   // K, then V (none when V aliases K)
  t /= a.nplanes;
  const int ci = t % a.max_chunks;
  t /= a.max_chunks;
  const int g = t % a.Hkv;
  const int bl = t / a.Hkv;
  const int b = a.b0 + bl;
  const int64_t pos = a.pos[bl];
  const int64_t end = pos + a.count[bl];
  const int64_t c = pos / kChunk + ci;
  const int64_t row0 = c * kChunk;
  if (end == pos || row0 >= end) return;   // whole workgroup: nothing of this request lands here
  const int r = (int)(c % a.P);
  const int64_t tile = tile_of(TileMap{a.table, a.num_blocks, a.P, a.B, a.Hkv, a.cap_chunks}, r, b, g, c / a.P);
  QuantJob j;
  j.D = a.D;
  j.lay = a.lay[plane];
  j.dtype = a.dtype;
  j.m_lo = (int)(pos > row0 ? pos - row0 : 0);
  j.m_hi = (int)(end - row0 < kChunk ? end - row0 : kChunk);
  // new row m of this tile is source token (row0 + m - pos) of this (request, head)
  j.src = a.src[plane] + (((int64_t)bl * a.Hkv + g) * a.n_new + (row0 - pos)) * a.D;
  j.tile = a.dst[plane] + tile * a.tile_stride;
  j.sc = a.sc[plane] + tile * a.sc_tile_stride;
  quant_tile(j, threadIdx.x, kThreads, s_red, s_e);
}

}  // namespace

hipError_t launch_quant_append(const QAppendArgs& a, int nb, hipStream_t st) {
  const int64_t wgs = (int64_t)nb * a.Hkv * a.max_chunks * a.nplanes;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_append_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace hx
