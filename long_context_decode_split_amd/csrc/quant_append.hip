// Quantising append: new bf16 K/V rows (the output of the QKV projection,
// written round-robin as produced: Helix summary, paragraph on Helix's two
// layouts) encoded on the device into fp8 e4m3 or MXFP4 chunk tiles.
//
// One workgroup owns one (request, KV head, chunk, K or V) tile, so the
// per-chunk fp8 scale, the re-encoding of stored codes when it grows, and
// the bytes of rows that share a 16-byte piece with new rows are all handled
// inside one workgroup: each thread owns whole bytes of the tile and writes
// them once.  Encoding is done with integer and exact power-of-two
// arithmetic (no hardware conversion), rounding to nearest with ties to the
// even code.
//
// fp8 e4m3: scale = amax / 448 of the group (1 when zero); a group filled
// over several calls keeps a scale that only grows, re-encoding its stored
// codes from their values times old / new scale when it does.
// MXFP4: per 32 elements of a row, E = clamp(floor(log2 amax) - 2, -127,
// 127) + 127, code = e2m1 of x / 2^(E-127), saturating at 6.

#include "hx_cache.h"

namespace hx {
namespace {

constexpr int kThreads = 256;
constexpr float kFp8Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// e4m3 code of q, |q| <= 448: nearest, ties to the even code; the sign bit
// is q's sign bit (negative zero included).
__device__ __forceinline__ uint32_t encode_e4m3(float q) {
  const uint32_t bits = __float_as_uint(q);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(q);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal steps of 2^-9
    code = (uint32_t)rintf(a * 512.0f);      // exact scaling, rint = nearest-even; 8 is the smallest normal
  } else {
    const uint32_t ab = __float_as_uint(a);
    int e = (int)(ab >> 23) - 127;           // -6 .. 8
    uint32_t keep = (ab >> 20) & 7u;         // top 3 mantissa bits
    const uint32_t rem = ab & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) {
      if (++keep == 8u) {
        keep = 0;
        ++e;
      }
    }
    code = ((uint32_t)(e + 7) << 3) | keep;  // at most 0x7E since a <= 448
  }
  return sign | code;
}

__device__ __forceinline__ float decode_e4m3(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? (float)m * 0.001953125f                       // m * 2^-9
                           : __uint_as_float(((e + 120u) << 23) | (m << 20));   // (1 + m/8) * 2^(e-7)
  return (c & 0x80u) ? -mag : mag;
}

// e2m1 code of y: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even
// code, saturating at 6; a value that rounds to zero gets code 0.
__device__ __forceinline__ uint32_t encode_e2m1(float y) {
  const float a = fabsf(y);
  const uint32_t idx = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return idx | ((y < 0.f && idx != 0) ? 8u : 0u);
}

// floor(log2 a) of a finite a > 0, from the fp32 bits (exact, subnormals too)
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t b = __float_as_uint(a) & 0x7FFFFFFFu;
  const int ex = (int)(b >> 23);
  if (ex != 0) return ex - 127;
  return 31 - __clz((int)(b & 0x7FFFFFu)) - 149;
}

__device__ __forceinline__ float block_max(float v, float* s_red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = s_red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, s_red[w]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void quant_append_kernel(const QAppendArgs a) {
  __shared__ float s_red[kThreads / 64];
  __shared__ uint8_t s_e[kChunk][4];   // MXFP4 exponents of the new rows (D / 32 = 4 blocks)
  int t = blockIdx.x;
  const int plane = t & 1;
  t >>= 1;
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
  const int m_lo = (int)(pos > row0 ? pos - row0 : 0);   // rows below m_lo were stored earlier
  const int m_hi = (int)(end - row0 < kChunk ? end - row0 : kChunk);
  const int r = (int)(c % a.P);
  const int64_t tile = tile_of(TileMap{a.table, a.num_blocks, a.P, a.B, a.Hkv, a.cap_chunks}, r, b, g, c / a.P);
  const int D = a.D;
  const int lay = a.lay[plane];
  // new row m of this tile is source token (row0 + m - pos) of this (request, head)
  const uint16_t* src = a.src[plane] + (((int64_t)bl * a.Hkv + g) * a.n_new + (row0 - pos)) * D;
  uint8_t* tp = a.dst[plane] + tile * a.tile_stride;
  const int tid = threadIdx.x;

  if (a.dtype == HX_KV_FP8_E4M3) {
    float* scp = reinterpret_cast<float*>(a.sc[plane] + tile * a.sc_tile_stride);
    // amax of the new rows, and whether a stored code of the group is non-zero
    float amax = 0.f, nz = 0.f;
    for (int i = tid; i < (m_hi - m_lo) * D; i += kThreads)
      amax = fmaxf(amax, fabsf(bf16_to_f32(src[(int64_t)(m_lo + i / D) * D + i % D])));
    for (int i = tid; i < m_lo * D; i += kThreads)
      if (tp[tile_off2(lay, D, i / D, i % D) >> 1] & 0x7Fu) nz = 1.f;
    amax = block_max(amax, s_red);
    nz = block_max(nz, s_red);
    const float s_old = m_lo > 0 ? *scp : 1.f;
    const float m_old = nz > 0.f ? s_old * kFp8Max : 0.f;
    float scale = s_old;
    bool reencode = false;
    if (m_lo == 0) {
      scale = amax > 0.f ? amax / kFp8Max : 1.f;
    } else if (amax > m_old) {
      scale = amax / kFp8Max;     // amax > 0 here
      reencode = m_old > 0.f;
    }
    const float ratio = s_old / scale;
    // each thread owns 8 bytes of the 2 KiB tile
    const int64_t byte0 = (int64_t)tid * 8;
    uint2 w = *reinterpret_cast<const uint2*>(tp + byte0);
    uint8_t* wb = reinterpret_cast<uint8_t*>(&w);
    bool touched = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int m, d;
      tile_inv(lay, D, 2 * (byte0 + e), &m, &d);
      if (m >= m_lo && m < m_hi) {
        const float q = fminf(fmaxf(bf16_to_f32(src[(int64_t)m * D + d]) / scale, -kFp8Max), kFp8Max);
        wb[e] = (uint8_t)encode_e4m3(q);
        touched = true;
      } else if (m < m_lo && reencode) {
        const float q = fminf(fmaxf(decode_e4m3(wb[e]) * ratio, -kFp8Max), kFp8Max);
        wb[e] = (uint8_t)encode_e4m3(q);
        touched = true;
      }
    }
    if (touched) *reinterpret_cast<uint2*>(tp + byte0) = w;
    if (tid == 0) *scp = scale;
  } else {   // MXFP4: exponents per (new row, block), then codes
    uint8_t* sp = a.sc[plane] + tile * a.sc_tile_stride;
    if (tid < kChunk * 4) {
      const int m = tid >> 2, j = tid & 3;
      if (m >= m_lo && m < m_hi) {
        float amax = 0.f;
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(bf16_to_f32(src[(int64_t)m * D + 32 * j + i])));
        int e = amax > 0.f ? floor_log2(amax) - 2 : -127;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        s_e[m][j] = (uint8_t)(e + 127);
        sp[m * 4 + j] = (uint8_t)(e + 127);
      }
    }
    __syncthreads();
    // each thread owns 4 bytes of the 1 KiB tile
    const int64_t byte0 = (int64_t)tid * 4;
    uint32_t w = *reinterpret_cast<const uint32_t*>(tp + byte0);
    bool touched = false;
#pragma unroll
    for (int n = 0; n < 8; ++n) {   // nibble n of the 4 bytes
      int m, d;
      tile_inv(lay, D, 2 * byte0 + n, &m, &d);
      if (m >= m_lo && m < m_hi) {
        const float y = ldexpf(bf16_to_f32(src[(int64_t)m * D + d]), 127 - (int)s_e[m][d >> 5]);
        const uint32_t code = encode_e2m1(y);
        w = (w & ~(0xFu << (4 * n))) | (code << (4 * n));
        touched = true;
      }
    }
    if (touched) *reinterpret_cast<uint32_t*>(tp + byte0) = w;
  }
}

}  // namespace

hipError_t launch_quant_append(const QAppendArgs& a, int nb, hipStream_t st) {
  const int64_t wgs = (int64_t)nb * a.Hkv * a.max_chunks * 2;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_append_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace hx
