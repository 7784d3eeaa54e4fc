// KV cache writes and reads: append with the 16-token round-robin placement,
// and row dequantisation for inspection.
//
// Placement (Helix summary, paragraph on Helix's two layouts; NVIDIA blog,
// section on distributed KV placement): token t of a request belongs to the
// 16-token group c = t / 16, which lives in slice c mod P as that slice's
// (c / P)-th chunk tile.
//
// The append kernel owns destination bytes, not source tokens: one thread
// builds one 16-byte piece of a chunk tile, fetching each element of the
// piece from the new tokens when its row is being appended and keeping the
// stored bytes otherwise.  No two threads touch the same bytes, so the result
// does not depend on scheduling, and bytes move unconverted (bit-exact).

#include "hx_cache.h"

namespace hx {
namespace {

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void append_kernel(const AppendArgs a, int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  if (gid >= total) return;

  // pieces of every plane for one (request, head, chunk)
  int64_t pieces[4], piece_sum = 0;
  for (int p = 0; p < a.nplanes; ++p) {
    pieces[p] = a.ebits[p] == 32 ? 1 : (a.tile_bytes[p] + 15) / 16;
    piece_sum += pieces[p];
  }
  // thread -> (request, head, chunk, piece); 32-bit division when the grid
  // allows it (64-bit division is a long software sequence on the GPU)
  int64_t piece;
  int ci, g, bl;
  if (total <= 0xffffffffll) {
    uint32_t t = (uint32_t)gid;
    const uint32_t ps = (uint32_t)piece_sum, mc = (uint32_t)a.max_chunks, hk = (uint32_t)a.Hkv;
    piece = t % ps;
    t /= ps;
    ci = (int)(t % mc);
    t /= mc;
    g = (int)(t % hk);
    bl = (int)(t / hk);
  } else {
    int64_t t = gid;
    piece = t % piece_sum;
    t /= piece_sum;
    ci = (int)(t % a.max_chunks);
    t /= a.max_chunks;
    g = (int)(t % a.Hkv);
    bl = (int)(t / a.Hkv);
  }
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
  uint8_t* dst = a.dst[plane] + tile * a.tile_bytes[plane];

  if (a.ebits[plane] == 32) {
    // one fp32 scale per chunk: taken from the first new token of the chunk
    const int64_t tf = row0 > pos ? row0 : pos;
    const float v = reinterpret_cast<const float*>(src)[src_tok0 + (tf - pos)];
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
  if (!whole && eb != 4) {
    // part of the piece is new (a decode step's row): store just the new
    // 1- or 2-byte elements, so the stored bytes of other rows are not read
    for (int e = 0; e < nelem; ++e) {
      int mm, d;
      tile_inv(lay, width, elem_off2(e), &mm, &d);
      const int64_t tok = row0 + mm;
      if (tok < pos || tok >= end) continue;
      const uint8_t* srcrow = src + (src_tok0 + (tok - pos)) * srow;
      if (eb == 16)
        *reinterpret_cast<uint16_t*>(dst + byte0 + 2 * e) = *reinterpret_cast<const uint16_t*>(srcrow + 2 * d);
      else
        dst[byte0 + e] = srcrow[d];
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

// fp8 e4m3 code -> fp32 (hardware conversion, OCP e4m3 on gfx950).
__device__ __forceinline__ float fp8_to_f32(uint32_t code) { return __builtin_amdgcn_cvt_f32_fp8(code, 0); }

// e2m1 code (low nibble) -> fp32 (hardware conversion, scale 1).
__device__ __forceinline__ float fp4_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code & 0xf, 1.0f, 0)[0];
}

__global__ __launch_bounds__(256) void dequant_kernel(const DequantArgs a, int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int width = a.Dk + a.Dv;
  const int64_t i = gid / width;
  int d = (int)(gid % width);
  const bool is_v = d >= a.Dk;
  if (is_v) {
    d -= a.Dk;
    if (!a.v_out) return;
  }
  const int64_t j = a.j0 + i;
  const int64_t tile = tile_of(a.map, a.r, a.b, a.g, j / kChunk);
  const int mm = (int)(j % kChunk);
  const bool from_k = !is_v || a.v_alias;
  const uint8_t* plane = from_k ? a.k : a.v;
  const int lay = from_k ? a.lay_k : a.lay_v;
  const int64_t tb = from_k ? a.k_tile : a.v_tile;
  const int rw = from_k ? a.Dk : a.Dv;
  const int64_t off2 = tile_off2(lay, rw, mm, d);
  const uint8_t* tp = plane + tile * tb;
  float val;
  if (a.dtype == HX_KV_BF16) {
    const uint16_t bits = *reinterpret_cast<const uint16_t*>(tp + (off2 >> 1));
    val = __uint_as_float((uint32_t)bits << 16);
  } else if (a.dtype == HX_KV_FP8_E4M3) {
    const float s = reinterpret_cast<const float*>(from_k ? a.ks : a.vs)[tile];
    val = fp8_to_f32(tp[off2 >> 1]) * s;   // one fp32 rounding
  } else {
    const uint8_t byte = tp[off2 >> 1];
    const uint32_t code = (off2 & 1) ? (byte >> 4) : (byte & 0xf);
    const uint8_t* sp = (from_k ? a.ks : a.vs) + tile * (from_k ? a.ks_tile : a.vs_tile);
    const int e = sp[mm * (rw / 32) + d / 32];
    val = e == 255 ? __uint_as_float(0x7fc00000u) : ldexpf(fp4_to_f32(code), e - 127);
  }
  float* out = is_v ? a.v_out : a.k_out;
  out[i * (is_v ? a.Dv : a.Dk) + d] = val;
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int nb, hipStream_t st) {
  int64_t piece_sum = 0;
  for (int p = 0; p < a.nplanes; ++p) piece_sum += a.ebits[p] == 32 ? 1 : (a.tile_bytes[p] + 15) / 16;
  const int64_t total = (int64_t)nb * a.Hkv * a.max_chunks * piece_sum;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + kAppendThreads - 1) / kAppendThreads;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(kAppendThreads), 0, st, a, total);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t st) {
  const int64_t total = a.n * (a.Dk + a.Dv);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a, total);
  return hipGetLastError();
}

}  // namespace hx
