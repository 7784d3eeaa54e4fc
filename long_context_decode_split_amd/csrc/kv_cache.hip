// KV cache writes and reads: append with the 16-token round-robin placement
// (one thread per 16-byte destination piece, append_piece in hx_append.h),
// and row dequantisation for inspection.

#include "hx_append.h"
#include "hx_cache.h"

namespace hx {
namespace {

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void append_kernel(const AppendArgs a, int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  if (gid >= total) return;

  // pieces of every plane for one (request, head, chunk)
  int64_t pieces[4];
  const int64_t piece_sum = append_pieces(a, pieces);
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
  append_piece(a, bl, g, ci, piece);
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
    const float s = *reinterpret_cast<const float*>((from_k ? a.ks : a.vs) + tile * (from_k ? a.ks_tile : a.vs_tile));
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
