// Quantisation of new bf16 K/V rows into one fp8 e4m3 or MXFP4 chunk tile,
// as a device function any workgroup can run: the quantising append kernel
// (one workgroup per tile) and the decode step's partial kernels (the
// workgroup that owns a tile, before it streams it) share it, so both write
// the same bytes.  New rows come out of the QKV projection and are written
// round-robin as produced (Helix summary, paragraph on Helix's two layouts);
// the pages do not fix how they are quantised, so these are the readings:
//
// fp8 e4m3: scale = amax / 448 of the 16-row group (1 when zero), code =
// nearest e4m3 (ties to even) of x / scale clamped to +-448; a group filled
// over several calls keeps a scale that only grows, re-encoding its stored
// codes from their values times old / new scale when it does (so a group
// written at once gets exactly the per-group rule).
// MXFP4: per 32 elements of a row, E = clamp(floor(log2 amax) - 2, -127, 127)
// + 127, code = nearest e2m1 (ties to even) of x / 2^(E-127), saturating at 6.
//
// Encoding uses integer and exact power-of-two arithmetic only (no hardware
// conversion).  Each thread owns whole bytes of the tile and writes them
// once, so rows that share bytes with the new rows are handled in place.
#pragma once

#include "hx_common.h"

namespace hx {

struct QuantJob {
  const uint16_t* src;   // bf16 row m of the tile at src + m * D, for m in [m_lo, m_hi)
  uint8_t* tile;         // the tile's codes
  uint8_t* sc;           // fp8: the tile's float scale; MXFP4: its 16 x D/32 e8m0 bytes
  int lay, D, dtype;
  int m_lo, m_hi;        // the new rows; rows below m_lo were stored earlier
};

namespace quant {

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
  const float mag = e == 0 ? (float)m * 0.001953125f                            // m * 2^-9
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

// Max of v over the nthr threads of the workgroup (a multiple of 64, all
// calling); s_red holds nthr / 64 floats.
__device__ __forceinline__ float block_max(float v, float* s_red, int tid, int nthr) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = v;
  __syncthreads();
  float r = s_red[0];
  for (int w = 1; w < nthr / 64; ++w) r = fmaxf(r, s_red[w]);
  __syncthreads();
  return r;
}

}  // namespace quant

// 32-element blocks per row of the widest quantised row (576-wide MLA latent rows).
constexpr int kQuantMaxBlocks = 576 / 32;

// Quantises the new rows of one tile (fp8: one K or V tile and its scale;
// MXFP4: one K or V code tile and its row exponents; quant_tile below picks
// the layout's instantiation).  Called by all nthr
// threads of a workgroup (nthr a multiple of 64, at most 1024), uniformly;
// s_red: nthr / 64 floats of LDS, s_e: 16 x kQuantMaxBlocks bytes of LDS.
// LAY is the tile layout as a compile-time constant, so the layout switches
// of the element maps fold away (quant_tile below dispatches on j.lay).
template <int LAY>
__device__ __forceinline__ void quant_tile_lay(const QuantJob& j, int tid, int nthr, float* s_red, uint8_t* s_e) {
  using namespace quant;
  const int D = j.D;
  constexpr int lay = LAY;
  // the layout fixes the format: fp8 codes (GQA tiles, MLA row-major bytes)
  // or MXFP4 codes (GQA tiles, MLA row-major nibbles)
  constexpr bool kFp8 = LAY == kLayGqaFp8K || LAY == kLayGqaFp8V || LAY == kLayRowU8;
  if constexpr (kFp8) {
    float* scp = reinterpret_cast<float*>(j.sc);
    // amax of the new rows, and whether a stored code of the group is non-zero
    float amax = 0.f, nz = 0.f;
    for (int i = tid; i < (j.m_hi - j.m_lo) * D; i += nthr)
      amax = fmaxf(amax, fabsf(bf16_to_f32(j.src[(int64_t)(j.m_lo + i / D) * D + i % D])));
    for (int i = tid; i < j.m_lo * D; i += nthr)
      if (j.tile[tile_off2(lay, D, i / D, i % D) >> 1] & 0x7Fu) nz = 1.f;
    amax = block_max(amax, s_red, tid, nthr);
    nz = block_max(nz, s_red, tid, nthr);
    const float s_old = j.m_lo > 0 ? *scp : 1.f;
    const float m_old = nz > 0.f ? s_old * kFp8Max : 0.f;
    float scale = s_old;
    bool reencode = false;
    if (j.m_lo == 0) {
      scale = amax > 0.f ? amax / kFp8Max : 1.f;
    } else if (amax > m_old) {
      scale = amax / kFp8Max;   // amax > 0 here
      reencode = m_old > 0.f;
    }
    const float ratio = s_old / scale;
    // each thread owns 8-byte pieces of the code tile (16 x D bytes)
    for (int64_t byte0 = (int64_t)tid * 8; byte0 < kChunk * D; byte0 += (int64_t)nthr * 8) {
      uint2 w = *reinterpret_cast<const uint2*>(j.tile + byte0);
      uint8_t* wb = reinterpret_cast<uint8_t*>(&w);
      bool touched = false;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int m, d;
        tile_inv(lay, D, 2 * (byte0 + e), &m, &d);
        if (m >= j.m_lo && m < j.m_hi) {
          const float q = fminf(fmaxf(bf16_to_f32(j.src[(int64_t)m * D + d]) / scale, -kFp8Max), kFp8Max);
          wb[e] = (uint8_t)encode_e4m3(q);
          touched = true;
        } else if (m < j.m_lo && reencode) {
          const float q = fminf(fmaxf(decode_e4m3(wb[e]) * ratio, -kFp8Max), kFp8Max);
          wb[e] = (uint8_t)encode_e4m3(q);
          touched = true;
        }
      }
      if (touched) *reinterpret_cast<uint2*>(j.tile + byte0) = w;
    }
    // every thread has read the stored scale (s_old) before the barriers of
    // block_max, so the new one can be written now
    if (tid == 0) *scp = scale;
  } else {   // MXFP4: exponents per (new row, 32-element block), then codes
    const int nblk = D / 32;
    for (int i = tid; i < kChunk * nblk; i += nthr) {
      const int m = i / nblk, jb = i % nblk;
      if (m >= j.m_lo && m < j.m_hi) {
        float amax = 0.f;
        for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(bf16_to_f32(j.src[(int64_t)m * D + 32 * jb + k])));
        int e = amax > 0.f ? floor_log2(amax) - 2 : -127;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        s_e[m * nblk + jb] = (uint8_t)(e + 127);
        j.sc[m * nblk + jb] = (uint8_t)(e + 127);
      }
    }
    __syncthreads();
    // each thread owns 4-byte pieces of the code tile (16 x D / 2 bytes)
    for (int64_t byte0 = (int64_t)tid * 4; byte0 < kChunk * D / 2; byte0 += (int64_t)nthr * 4) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(j.tile + byte0);
      bool touched = false;
#pragma unroll
      for (int n = 0; n < 8; ++n) {   // nibble n of the 4 bytes
        int m, d;
        tile_inv(lay, D, 2 * byte0 + n, &m, &d);
        if (m >= j.m_lo && m < j.m_hi) {
          const float y = ldexpf(bf16_to_f32(j.src[(int64_t)m * D + d]), 127 - (int)s_e[m * nblk + (d >> 5)]);
          const uint32_t code = encode_e2m1(y);
          w = (w & ~(0xFu << (4 * n))) | (code << (4 * n));
          touched = true;
        }
      }
      if (touched) *reinterpret_cast<uint32_t*>(j.tile + byte0) = w;
    }
    __syncthreads();   // s_e is free again
  }
}

__device__ __forceinline__ void quant_tile(const QuantJob& j, int tid, int nthr, float* s_red, uint8_t* s_e) {
  switch (j.lay) {   // uniform over the workgroup
    case kLayGqaFp8K: quant_tile_lay<kLayGqaFp8K>(j, tid, nthr, s_red, s_e); break;
    case kLayGqaFp8V: quant_tile_lay<kLayGqaFp8V>(j, tid, nthr, s_red, s_e); break;
    case kLayGqaFp4K: quant_tile_lay<kLayGqaFp4K>(j, tid, nthr, s_red, s_e); break;
    case kLayGqaFp4V: quant_tile_lay<kLayGqaFp4V>(j, tid, nthr, s_red, s_e); break;
    case kLayRowU4: quant_tile_lay<kLayRowU4>(j, tid, nthr, s_red, s_e); break;
    default: quant_tile_lay<kLayRowU8>(j, tid, nthr, s_red, s_e); break;
  }
}

}  // namespace hx
