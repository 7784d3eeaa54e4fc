// Split-KV decode attention for GQA caches with wide query groups: 17 to 128
// query heads per KV head (Dk = Dv = 128), on gfx950.
//
// What one launch computes is what the narrow kernel (decode_gqa.hip)
// computes (Helix summary, paragraph on KV parallelism: each slice attends
// over its part of the history and returns a partial output and a
// log-sum-exp), for groups of more than 16 query heads: GQA with few KV heads
// per GPU shares every K/V row among many query heads (Helix summary,
// paragraph on tensor parallelism), which makes both products dense enough
// for the matrix cores to matter.
//
// Each K/V chunk tile is read from HBM once.  A workgroup of W waves streams
// one split of a slice as pairs of chunk tiles: the pair is copied unchanged
// into a ring of LDS buffers by direct global-to-LDS loads (each wave copies
// its share; one barrier per pair publishes it and frees the buffer of the
// pair before), and every wave reads the whole pair from LDS for its own
// query heads: wave w owns 16-head blocks w, w + W, ... (NHW of them), so the
// waves never exchange partial results.
//
// Per pair and 16-head block, on the tile byte orders of the cache:
//   * S^T = K Q^T: four v_mfma_f32_16x16x32_bf16 per tile (rows = the tile's
//     16 tokens, columns = the block's heads), the K fragments read once per
//     pair and reused by the wave's head blocks;
//   * online softmax in base 2 over the pair's 32 tokens (lane l holds head
//     l % 16, tokens 4 (l / 16) .. + 3 of both tiles);
//   * O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with k = the pair's 32
//     tokens: the k index of a lane group is tokens 4h .. 4h + 3 of the
//     first tile then of the second, which is exactly where the two score
//     fragments leave P and where the V tiles keep those tokens' values, so
//     P moves nowhere and each value block takes one full-rate product (bf16
//     caches: two, P as a bf16 high part plus its residual).
// fp8 and MXFP4 pairs are converted to bf16 fragments as in the narrow
// kernel (scales folded into the scores and into P).

#include "hx_append.h"
#include "hx_gqa_frag.h"

#include <type_traits>

namespace hx {
namespace {

using namespace frag;

constexpr int kD = 128;
constexpr float kLn2 = 0.693147180559945309f;
// log2 of the largest unnormalised probability: bf16 caches keep the
// reference at the running max, the quantised formats let it lag by 2^8
// (the narrow kernel's policy).
template <int FMT>
constexpr float kHeadroomW = FMT == 0 ? 0.0f : 8.0f;

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint4 lds_u4;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) float lds_f32;

// LDS bytes of one buffered tile pair, and where its parts sit:
//   bf16 : K0, K1, V0, V1 codes (4 KiB each);
//   fp8  : K0, K1, V0, V1 codes (2 KiB each), then the floats ks0 ks1 vs0 vs1;
//   MXFP4: K0, V0, K1, V1 codes (1 KiB each), then the e8m0 bytes of tile 0
//          (K then V, 64 B each) and of tile 1.
template <int FMT>
struct PairLay;
template <>
struct PairLay<0> {
  static constexpr int kBytes = 16384, kJobs = 16;   // 1 KiB copies per pair
};
template <>
struct PairLay<1> {
  static constexpr int kBytes = 8208, kJobs = 8, kSc = 8192;
};
template <>
struct PairLay<2> {
  static constexpr int kBytes = 4352, kJobs = 4, kSc = 4096;
};
// Buffers in the ring (pairs in flight + the one in use).  Each wave's work
// on a pair is a chain of LDS reads, score products, softmax and value
// products behind a barrier, so throughput comes from several workgroups per
// CU rather than from a deep ring: measured at 2^20 tokens, 64 heads, bf16,
// 4 workgroups per CU with two buffers (32 KiB) beat 2 with four (829 vs
// 902 us on one box) and one workgroup with six (1,055 us); fp8 and MXFP4
// pairs likewise run best with two buffers and eight workgroups per CU.
#ifndef HX_WIDE_RING_BF16
#define HX_WIDE_RING_BF16 2
#endif
#ifndef HX_WIDE_RING_FP8
#define HX_WIDE_RING_FP8 2
#endif
#ifndef HX_WIDE_RING_FP4
#define HX_WIDE_RING_FP4 2
#endif
template <int FMT>
constexpr int kRing = FMT == 0 ? HX_WIDE_RING_BF16 : (FMT == 1 ? HX_WIDE_RING_FP8 : HX_WIDE_RING_FP4);
// Copy instructions each wave issues per pair: its code blocks plus (fp8,
// MXFP4) its lanes of the scale copy.
template <int FMT, int W>
constexpr int kWaveJobs = PairLay<FMT>::kJobs / W + (FMT == 0 ? 0 : 1);

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Direct global-to-LDS copies: every active lane copies 16 (dma16) or 4
// (dma4) bytes from its own 64-bit address to LDS byte lds + 16 l (4 l),
// l its lane.  M0 (the wave-uniform LDS base) is an asm input, so the
// compiler sets it; the asm carries the wait states the compiler cannot see
// it needs (five after a VALU write of an SGPR, one after the M0 write).
// Completion is awaited with explicit vmcnt waits before the barrier that
// publishes a pair.  KV rows are read once: non-temporal.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Barrier once this wave's copies down to N still in flight have landed and
// its LDS accesses are done (also a compiler memory barrier).
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same with N = J * q for a runtime q in [0, Q].
template <int J, int Q>
__device__ __forceinline__ void wait_pairs(int q) {
  if constexpr (Q == 0) {
    wait_barrier<0>();
  } else {
    if (q >= Q)
      wait_barrier<J * Q>();
    else
      wait_pairs<J, Q - 1>(q);
  }
}

template <int FMT, bool PAGED, int W, int NHW, int FUSE>
__global__ __launch_bounds__(64 * W, NHW > 1 ? 2 : 1) void gqa_wide_kernel(const PartialArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // device-only builtins (LDS address space) below
  using Lay = PairLay<FMT>;
  constexpr int kNBuf = kRing<FMT>;
  constexpr int kJ = kWaveJobs<FMT, W>;
  __shared__ __attribute__((aligned(1024))) uint8_t s_buf[kNBuf][Lay::kBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;   // head column / token row inside a fragment
  const int h = lane >> 4;   // lane group

  // ---- which (request, KV head, slice, split) this workgroup owns
  const int wg = blockIdx.x;
  int rem;
  const int bl = request_of(a, wg, &rem);
  const int nsplit = a.nsplit[bl];
  const int split = rem % nsplit;
  rem /= nsplit;
  const int r = rem % a.P;
  const int g = rem / a.P;
  const int b = a.b0 + bl;

  const int64_t L = slice_len(a.n[bl], a.P, r);
  const int nch = (int)((L + kChunk - 1) / kChunk);
  const int c0 = split * a.cpw_b[bl];
  const int c1 = min(c0 + a.cpw_b[bl], nch);
  // the step's new rows of these tiles first: copied (storage format) or quantised from bf16
  if constexpr (FUSE == 1) fused_append(a.app, bl, g, r, c0, c1);
  if constexpr (FUSE == 2) fused_quant(a.app, bl, g, r, c0, c1);
  const int tail_valid = (int)(L - (int64_t)(nch - 1) * kChunk);   // rows in the slice's last chunk
  const int npairs = c1 > c0 ? (c1 - c0 + 1) >> 1 : 0;
  const int G = a.G;

  // Tile index (the same in every plane) of the slice's local chunk c:
  // consecutive from tile0 in a dense cache, through the block table in a
  // pool (tile_of in hx_common.h).
  const int64_t tile0 = PAGED ? 0 : ((int64_t)(r * a.Btot + b) * a.Hkv + g) * a.cap_chunks;
  // (read through the constant address space: the table does not change
  // during the kernel, and only so are the lookups scalar loads; the copies'
  // memory clobbers keep the compiler from proving it otherwise)
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* trow = PAGED ? (const_i32*)(a.table + ((int64_t)b * a.P + r) * a.cap_chunks) : nullptr;
  // the tiles of the pair to copy next; pool lookups are made before the
  // barrier that precedes the copy, so their latency hides in its wait.  A
  // pair of one tile copies its first tile twice (the second is masked), so
  // every pair is the same number of copies and the waits stay exact.
  int64_t nt0 = 0, nt1 = 0;
  auto prep = [&](int k) {
    // uniform indices, so the lookups are scalar loads (a vector load here
    // would make the compiler wait for every copy in flight)
    const int c = __builtin_amdgcn_readfirstlane(c0 + 2 * k);
    const int cb = __builtin_amdgcn_readfirstlane(c + 1 < c1 ? c + 1 : c);
    if constexpr (PAGED) {
      nt0 = clamp_block(trow[c], a.num_blocks) * a.Hkv + g;
      nt1 = cb == c ? nt0 : clamp_block(trow[cb], a.num_blocks) * a.Hkv + g;
    } else {
      nt0 = tile0 + c;
      nt1 = tile0 + cb;
    }
  };
  // This wave's copies of pair k (tiles nt0, nt1) into buffer k % kNBuf:
  // code blocks wave, wave + W, ... of the pair, then its lanes of the scales.
  auto issue = [&](int k) {
    uint8_t* buf = &s_buf[k % kNBuf][0];
#pragma unroll
    for (int i = 0; i < Lay::kJobs / W; ++i) {
      const int j = wave + W * i;
      const uint8_t* src;
      int dst;
      if constexpr (FMT == 0) {   // j: part j / 4 (K0 K1 V0 V1), 1 KiB block j % 4
        const int part = j >> 2;
        src = (part < 2 ? a.k + ((part & 1) ? nt1 : nt0) * a.k_tile : a.v + ((part & 1) ? nt1 : nt0) * a.v_tile) +
              (j & 3) * 1024;
        dst = j * 1024;
      } else if constexpr (FMT == 1) {   // j: part j / 2 (K0 K1 V0 V1), block j % 2
        const int part = j >> 1;
        src = (part < 2 ? a.k + ((part & 1) ? nt1 : nt0) * a.k_tile : a.v + ((part & 1) ? nt1 : nt0) * a.v_tile) +
              (j & 1) * 1024;
        dst = j * 1024;
      } else {   // j: tile j / 2, K codes (j even) or V codes of the packed tile
        src = a.k + ((j >> 1) ? nt1 : nt0) * a.k_tile + (j & 1) * 1024;
        dst = j * 1024;
      }
      dma16(src + lane * 16, lds_addr(buf + dst));
    }
    if constexpr (FMT == 1) {   // lane q < 4 of the pair: ks0 ks1 vs0 vs1, split over the waves
      constexpr int kPer = 4 / W;
      if (lane >= kPer * wave && lane < kPer * (wave + 1)) {
        const int64_t t = (lane & 1) ? nt1 : nt0;
        const uint8_t* src = (lane < 2 ? a.ks + t * a.ks_tile : a.vs + t * a.vs_tile);
        dma4(src, lds_addr(buf + Lay::kSc));
      }
    } else if constexpr (FMT == 2) {   // lane q < 16: e8m0 bytes 16 (q % 8) .. of tile q / 8
      constexpr int kPer = 16 / W;
      if (lane >= kPer * wave && lane < kPer * (wave + 1)) {
        const int64_t t = lane >= 8 ? nt1 : nt0;
        dma16(a.ks + t * a.ks_tile + (lane & 7) * 16, lds_addr(buf + Lay::kSc));
      }
    }
  };

  // ---- Q^T fragments of this wave's head blocks (B operand of S^T = K Q^T:
  //      head m of the block, columns 32 s + 8 h .. + 7); dead heads are 0
  //      (every load issued before any is used: a dead head reads head 0
  //      and is masked afterwards, without a branch)
  bf16x8 qf[NHW][4];
  {
    uint4 qr[NHW][4];
#pragma unroll
    for (int i = 0; i < NHW; ++i) {
      const int head = 16 * (wave + W * i) + m;
      const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + g * G + (head < G ? head : 0)) * a.Dk;
#pragma unroll
      for (int s = 0; s < 4; ++s) qr[i][s] = *reinterpret_cast<const uint4*>(qrow + s * 32 + h * 8);
    }
#pragma unroll
    for (int i = 0; i < NHW; ++i) {
      const uint32_t keep = 16 * (wave + W * i) + m < G ? 0xffffffffu : 0u;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        qf[i][s] = as_bf16x8(make_uint4(qr[i][s].x & keep, qr[i][s].y & keep, qr[i][s].z & keep, qr[i][s].w & keep));
    }
  }
  // Q is in place before the first copy, so no wait the compiler derives for
  // Q can later count the copies.
  __builtin_amdgcn_s_waitcnt(0);

  f32x4 acc[NHW][8];
  float mrun[NHW], lsum[NHW], lsm[NHW];
#pragma unroll
  for (int i = 0; i < NHW; ++i) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[i][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    mrun[i] = -INFINITY;
    lsum[i] = 0.f;
    lsm[i] = 0.f;
  }
  // head blocks of this wave with at least one live head (uniform)
  const int nlive = (G + 15) / 16;
  const float c2 = a.c2;

  // ---- one pair from LDS: scores, softmax, value product
  // FULL: both tiles hold 16 valid rows, so no row is masked (MXFP4 only,
  // where the masking is a measurable share of the issue slots)
  auto compute = [&](auto full_t, const lds_u8* pb, int v0, int v1) {
    constexpr bool FULL = decltype(full_t)::value;
    // K fragments of both tiles as bf16, and the per-tile scales
    bf16x8 kf[2][4];
    float ks[2] = {1.f, 1.f}, vs[2] = {1.f, 1.f};
    uint32_t ksc[2] = {0u, 0u};
    uint4 vsc[2];
    if constexpr (FMT == 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[t][s] = as_bf16x8(*(const lds_u4*)(pb + t * 4096 + s * 1024 + lane * 16));
    } else if constexpr (FMT == 1) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        ks[t] = *(const lds_f32*)(pb + Lay::kSc + 4 * t);
        vs[t] = *(const lds_f32*)(pb + Lay::kSc + 8 + 4 * t);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 raw = *(const lds_u4*)(pb + t * 2048 + i * 1024 + lane * 16);
          const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {   // bytes 0-7 -> step 2i, 8-15 -> step 2i+1
            uint4 u;
            u.x = fp8x2_to_bf16x2<false>(w[2 * hs]);
            u.y = fp8x2_to_bf16x2<true>(w[2 * hs]);
            u.z = fp8x2_to_bf16x2<false>(w[2 * hs + 1]);
            u.w = fp8x2_to_bf16x2<true>(w[2 * hs + 1]);
            kf[t][2 * i + hs] = as_bf16x8(u);
          }
        }
      }
      if (v1 == 0) {   // a pair of one tile: its second slot holds no scale of its own
        ks[1] = 1.f;
        vs[1] = 1.f;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint4 raw = *(const lds_u4*)(pb + t * 2048 + lane * 16);
        ksc[t] = *(const lds_u32*)(pb + Lay::kSc + t * 128 + m * 4);          // 4 e8m0 of token m
        vsc[t] = *(const lds_u4*)(pb + Lay::kSc + t * 128 + 64 + h * 16);     // tokens 4h..4h+3, 4 blocks each
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float sc = e8m0_sel(ksc[t], s);
          uint4 u;
          u.x = fp4x2_to_bf16x2<0>(w[s], sc);
          u.y = fp4x2_to_bf16x2<1>(w[s], sc);
          u.z = fp4x2_to_bf16x2<2>(w[s], sc);
          u.w = fp4x2_to_bf16x2<3>(w[s], sc);
          kf[t][s] = as_bf16x8(u);
        }
      }
    }
    // V fragments (raw codes) of both tiles
    constexpr int kVW = FMT == 0 ? 4 : (FMT == 1 ? 2 : 1);
    uint4 vr[2][kVW];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int p = 0; p < kVW; ++p) {
        const int off = FMT == 0 ? 8192 + t * 4096 + p * 1024 : (FMT == 1 ? 4096 + t * 2048 + p * 1024 : t * 2048 + 1024);
        vr[t][p] = *(const lds_u4*)(pb + off + lane * 16);
      }
    // rows of each tile this lane's V halves may use (tokens 4h+{0,1}, 4h+{2,3});
    // bf16 and fp8 pairs need no mask here: the V values of rows past the
    // slice end were zeroed in LDS (zero_tail_v), so their weight 0 adds 0
    uint32_t keep01[2], keep23[2];
    {
      const int vv[2] = {v0, v1};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bool all = FULL || FMT != 2;
        keep01[t] = all ? ~0u : (4 * h + 0 < vv[t] ? 0x0000ffffu : 0u) | (4 * h + 1 < vv[t] ? 0xffff0000u : 0u);
        keep23[t] = all ? ~0u : (4 * h + 2 < vv[t] ? 0x0000ffffu : 0u) | (4 * h + 3 < vv[t] ? 0xffff0000u : 0u);
      }
    }

#pragma unroll
    for (int i = 0; i < NHW; ++i) {
      if (wave + W * i >= nlive) continue;   // no live head in this block (uniform)
      // ---- scores of the block's heads over the pair's 32 tokens
      float s8[8];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][s], qf[i][s], sc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) s8[4 * t + j] = FMT == 1 ? sc[j] * (c2 * ks[t]) : sc[j];
      }
      // masked scores: selects, taken only on pairs with rows past the slice
      // end (a uniform branch: no per-pair cost on full pairs)
      if (!FULL && (v0 < kChunk || v1 < kChunk)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (4 * h + j >= v0) s8[j] = -INFINITY;
          if (4 * h + j >= v1) s8[4 + j] = -INFINITY;
        }
      }
      // ---- online softmax (base 2): the reference moves only when some
      //      head's scores exceed it by more than the headroom
      float cm = fmaxf(fmaxf(vmax(s8[0], s8[1]), vmax(s8[2], s8[3])), fmaxf(vmax(s8[4], s8[5]), vmax(s8[6], s8[7])));
      cm = max_xor32(max_xor16(cm));
      const float cms = FMT == 1 ? cm : cm * c2;
      if (__any(cms > mrun[i] + kHeadroomW<FMT>)) {   // wave-uniform
        const float mnew = fmaxf(mrun[i], cms);
        const float alpha = __builtin_amdgcn_exp2f(mrun[i] - mnew);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[i][nb] *= alpha;
        lsm[i] *= alpha;
        lsum[i] *= alpha;
        mrun[i] = mnew;
      }
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        p[j] = __builtin_amdgcn_exp2f(FMT == 1 ? s8[j] - mrun[i] : fmaf(s8[j], c2, -mrun[i]));
      lsum[i] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));

      // ---- O^T += V^T P^T, k = the pair's 32 tokens
      if constexpr (FMT == 0) {
        // P as a bf16 high part plus the bf16 of its residual (about 16
        // significant bits; the narrow kernel's reasoning)
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ph[q] = pack_bf16(p[2 * q], p[2 * q + 1]);
          pl[q] = pack_bf16(p[2 * q] - bf16lo(ph[q]), p[2 * q + 1] - bf16hi(ph[q]));
        }
        float sm = lsm[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) sm = add_bf16x2(pl[q], add_bf16x2(ph[q], sm));
        lsm[i] = sm;
        const bf16x8 PH = as_bf16x8(make_uint4(ph[0], ph[1], ph[2], ph[3]));
        const bf16x8 PL = as_bf16x8(make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int q = nb >> 1;   // 16-byte chunk; value block nb is its half nb & 1
          const uint4 u0 = vr[0][q], u1 = vr[1][q];
          const uint4 va = (nb & 1) ? make_uint4(u0.z & keep01[0], u0.w & keep23[0], u1.z & keep01[1], u1.w & keep23[1])
                                    : make_uint4(u0.x & keep01[0], u0.y & keep23[0], u1.x & keep01[1], u1.y & keep23[1]);
          acc[i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), PH, acc[i][nb], 0, 0, 0);
          acc[i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), PL, acc[i][nb], 0, 0, 0);
        }
      } else if constexpr (FMT == 1) {
        // each tile's V scale folded into its half of P; the rounded
        // products divided by the scale normalise O (a zero scale: the
        // weights unrounded, the values being 0)
        uint32_t pk[4];
        float sm = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          pk[2 * t] = pack_bf16(p[4 * t] * vs[t], p[4 * t + 1] * vs[t]);
          pk[2 * t + 1] = pack_bf16(p[4 * t + 2] * vs[t], p[4 * t + 3] * vs[t]);
          const float rounded = add_bf16x2(pk[2 * t + 1], add_bf16x2(pk[2 * t], 0.f));
          sm += vs[t] != 0.f ? rounded * __builtin_amdgcn_rcpf(vs[t])
                             : (p[4 * t] + p[4 * t + 1]) + (p[4 * t + 2] + p[4 * t + 3]);
        }
        lsm[i] += sm;
        const bf16x8 PB = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int q = nb >> 2, wd = nb & 3;   // chunk q, word wd: 4 codes (tokens 4h..4h+3)
          uint32_t lo[2], hi[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const uint4 u = vr[t][q];
            const uint32_t w = wd == 0 ? u.x : (wd == 1 ? u.y : (wd == 2 ? u.z : u.w));
            lo[t] = fp8x2_to_bf16x2<false>(w) & keep01[t];
            hi[t] = fp8x2_to_bf16x2<true>(w) & keep23[t];
          }
          const bf16x8 va = as_bf16x8(make_uint4(lo[0], hi[0], lo[1], hi[1]));
          acc[i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, PB, acc[i][nb], 0, 0, 0);
        }
      } else {
        // per (token, 32-column block) power-of-two scales added into the
        // exponents of P's bf16 pairs (scale_bf16x2_e8m0: the rounded
        // product), one P fragment per block; the sum of the rounded,
        // unscaled P normalises O.  P is clamped at 2^-126 below (an exact
        // 0 would not stay 0 through the exponent arithmetic).
        const float kMinP = 1.17549435e-38f;   // 2^-126
        uint32_t p2[2][2];   // [tile][tokens 4h+0,1 | 4h+2,3]
        {
          float sm = lsm[i];
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              p2[t][q] = pack_bf16(fmaxf(p[4 * t + 2 * q], kMinP), fmaxf(p[4 * t + 2 * q + 1], kMinP));
              sm = add_bf16x2(p2[t][q], sm);
            }
          lsm[i] = sm;
        }
        const uint32_t vw[2][4] = {{vsc[0].x, vsc[0].y, vsc[0].z, vsc[0].w}, {vsc[1].x, vsc[1].y, vsc[1].z, vsc[1].w}};
        auto block = [&](auto blk_t) {
          constexpr int blk = decltype(blk_t)::value;
          uint32_t sp[2][2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            sp[t][0] = scale_bf16x2_e8m0(p2[t][0], e8m0_pair<blk>(vw[t][0], vw[t][1]));
            sp[t][1] = scale_bf16x2_e8m0(p2[t][1], e8m0_pair<blk>(vw[t][2], vw[t][3]));
            if constexpr (!FULL) {   // rows past the slice: any scale byte
              sp[t][0] &= keep01[t];
              sp[t][1] &= keep23[t];
            }
          }
          const bf16x8 PB = as_bf16x8(make_uint4(sp[0][0], sp[0][1], sp[1][0], sp[1][1]));
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const int nb = 2 * blk + hb;   // bytes 2nb, 2nb+1 of the lane's 16 B
            uint32_t lo[2], hi[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const uint4 u = vr[t][0];
              const uint32_t word = (nb >> 1) == 0 ? u.x : ((nb >> 1) == 1 ? u.y : ((nb >> 1) == 2 ? u.z : u.w));
              if ((nb & 1) == 0) {
                lo[t] = fp4x2_to_bf16x2<0>(word, 1.0f) & keep01[t];
                hi[t] = fp4x2_to_bf16x2<1>(word, 1.0f) & keep23[t];
              } else {
                lo[t] = fp4x2_to_bf16x2<2>(word, 1.0f) & keep01[t];
                hi[t] = fp4x2_to_bf16x2<3>(word, 1.0f) & keep23[t];
              }
            }
            const bf16x8 va = as_bf16x8(make_uint4(lo[0], hi[0], lo[1], hi[1]));
            acc[i][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, PB, acc[i][nb], 0, 0, 0);
          }
        };
        block(std::integral_constant<int, 0>{});
        block(std::integral_constant<int, 1>{});
        block(std::integral_constant<int, 2>{});
        block(std::integral_constant<int, 3>{});
      }
    }
  };

  // ---- bf16 and fp8 pairs with rows past the slice end (a slice's last
  //      tile, or the empty second slot of a one-tile pair): the V values of
  //      those rows, whose bytes may be anything (NaN included), are set to
  //      zero in the LDS copy once, so the value products need no per-pair
  //      mask (their weights are 0; 0 times a NaN would not be).  Each 16-byte
  //      piece of a V tile holds tokens 4h .. 4h + 3 (h = bits 4-5 of the
  //      piece's lane index) of two value columns (bf16: 2 bytes per token in
  //      each 8-byte half) or four (fp8: one byte per token in each word).
  //      Every wave's stores are done before the barrier that follows.
  auto zero_tail_v = [&](uint8_t* pbw, int v0, int v1) {
    if constexpr (FMT != 2) {
      constexpr int kPieces = FMT == 0 ? 256 : 128;   // 16-byte pieces per V tile
      constexpr int kVOff = FMT == 0 ? 8192 : 4096, kVTile = FMT == 0 ? 4096 : 2048;
      for (int pi = threadIdx.x; pi < 2 * kPieces; pi += 64 * W) {
        const int t = pi / kPieces, q = pi % kPieces;
        const int v = t ? v1 : v0;
        const int hh = (q & 63) >> 4;
        if (4 * hh + 3 < v) continue;   // every token of the piece is a row of the slice
        uint32_t m01, m23;
        if constexpr (FMT == 0) {
          m01 = (4 * hh + 0 < v ? 0x0000ffffu : 0u) | (4 * hh + 1 < v ? 0xffff0000u : 0u);
          m23 = (4 * hh + 2 < v ? 0x0000ffffu : 0u) | (4 * hh + 3 < v ? 0xffff0000u : 0u);
        } else {
          m01 = (4 * hh + 0 < v ? 0x000000ffu : 0u) | (4 * hh + 1 < v ? 0x0000ff00u : 0u) |
                (4 * hh + 2 < v ? 0x00ff0000u : 0u) | (4 * hh + 3 < v ? 0xff000000u : 0u);
          m23 = m01;
        }
        lds_u4* ptr = (lds_u4*)(pbw + kVOff + t * kVTile + 16 * q);
        uint4 u = *ptr;
        if constexpr (FMT == 0) u = make_uint4(u.x & m01, u.y & m23, u.z & m01, u.w & m23);
        else u = make_uint4(u.x & m01, u.y & m01, u.z & m01, u.w & m01);
        *ptr = u;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };

  // ---- the pairs, kNBuf - 1 in flight: pair k lands in buffer k % kNBuf;
  //      iteration k waits for its own copies of pair k, then the barrier
  //      publishes every wave's part and certifies that all waves are done
  //      with pair k - 1, whose buffer takes pair k + kNBuf - 1.
  for (int k = 0; k < kNBuf - 1 && k < npairs; ++k) {
    prep(k);
    issue(k);
  }
  for (int k = 0; k < npairs; ++k) {
    const int ahead = min(npairs - 1, k + kNBuf - 2) - k;   // pairs copied after k
    const bool more = k + kNBuf - 1 < npairs;
    if (more) prep(k + kNBuf - 1);
    wait_pairs<kJ, kNBuf - 2>(ahead);
    if (more) issue(k + kNBuf - 1);
    const int ct = c0 + 2 * k;
    const int v0 = ct == nch - 1 ? tail_valid : kChunk;
    const int v1 = ct + 1 < c1 ? (ct + 1 == nch - 1 ? tail_valid : kChunk) : 0;
    const lds_u8* pb = (const lds_u8*)&s_buf[k % kNBuf][0];
    if constexpr (FMT == 2) {
      if (v0 == kChunk && v1 == kChunk)
        compute(std::true_type{}, pb, v0, v1);
      else
        compute(std::false_type{}, pb, v0, v1);
    } else {
      if (v0 < kChunk || v1 < kChunk) zero_tail_v((uint8_t*)&s_buf[k % kNBuf][0], v0, v1);   // uniform
      compute(std::false_type{}, pb, v0, v1);
    }
  }

  // ---- finalize this wave's heads (no exchange between waves)
  const bool direct = nsplit == 1;
#pragma unroll
  for (int i = 0; i < NHW; ++i) {
    const int head = 16 * (wave + W * i) + m;
    const float ls = sum_xor32(sum_xor16(lsum[i]));
    const float lm = sum_xor32(sum_xor16(lsm[i]));
    if (head >= G) continue;
    float* out_o;
    float* out_l;
    if (direct) {
      out_o = a.o_part + (((int64_t)r * a.Btot + b) * a.Hq + g * G + head) * a.Dv;
      out_l = a.lse_part + ((int64_t)r * a.Btot + b) * a.Hq + g * G + head;
    } else {
      out_o = a.ws_o + ((int64_t)wg * G + head) * a.Dv;
      out_l = a.ws_lse + (int64_t)wg * G + head;
    }
    const float inv = lm > 0.f ? 1.0f / lm : 0.f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const f32x4 v = acc[i][nb];
      *reinterpret_cast<float4*>(out_o + 16 * nb + 4 * h) = make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    }
    if (h == 0) *out_l = ls > 0.f ? (mrun[i] + __log2f(ls)) * kLn2 : -INFINITY;
  }
#endif
}

template <int FMT, bool PAGED, int FUSE>
void launch_heads(const PartialArgs& a, int nwg, hipStream_t st) {
  const int nh = (a.G + 15) / 16;
  if (nh <= 2)
    hipLaunchKernelGGL((gqa_wide_kernel<FMT, PAGED, 2, 1, FUSE>), dim3(nwg), dim3(128), 0, st, a);
  else if (nh <= 4)
    hipLaunchKernelGGL((gqa_wide_kernel<FMT, PAGED, 4, 1, FUSE>), dim3(nwg), dim3(256), 0, st, a);
  else if constexpr (FMT == 0)
    // bf16, five to eight head blocks: eight waves of one block each (125
    // registers) measured 2-4% faster than four waves of two (230): G = 96
    // 1,072 -> 1,028 us, G = 128 1,179 -> 1,148 us.  The quantised pairs'
    // copies do not divide over eight waves.
    hipLaunchKernelGGL((gqa_wide_kernel<FMT, PAGED, 8, 1, FUSE>), dim3(nwg), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((gqa_wide_kernel<FMT, PAGED, 4, 2, FUSE>), dim3(nwg), dim3(256), 0, st, a);
}

// Fused append modes per format as in the narrow kernel: bf16 1; fp8 1 or 2;
// MXFP4 only 2 (stored MXFP4 codes take the append kernel first).
template <int FMT, bool PAGED>
void launch_fmt_wide(const PartialArgs& a, int nwg, hipStream_t st) {
  if constexpr (FMT == 1) {
    if (a.fused_append == 1) return launch_heads<FMT, PAGED, 1>(a, nwg, st);
  }
  if constexpr (FMT == 0) {
    if (a.fused_append) return launch_heads<FMT, PAGED, 1>(a, nwg, st);
  } else {
    if (a.fused_append == 2) return launch_heads<FMT, PAGED, 2>(a, nwg, st);
  }
  launch_heads<FMT, PAGED, 0>(a, nwg, st);
}

}  // namespace

hipError_t launch_gqa_wide(const PartialArgs& a, int dtype, hipStream_t st) {
  const int nwg = a.wg_begin[a.nb];
  if (nwg == 0) return hipSuccess;
  if (a.G < 1 || a.G > kGqaWideMaxHeads || a.Dk != kD || a.Dv != kD) return hipErrorInvalidValue;
  const bool paged = a.table != nullptr;
  switch (dtype) {
    case HX_KV_BF16:
      paged ? launch_fmt_wide<0, true>(a, nwg, st) : launch_fmt_wide<0, false>(a, nwg, st);
      break;
    case HX_KV_FP8_E4M3:
      paged ? launch_fmt_wide<1, true>(a, nwg, st) : launch_fmt_wide<1, false>(a, nwg, st);
      break;
    default:
      paged ? launch_fmt_wide<2, true>(a, nwg, st) : launch_fmt_wide<2, false>(a, nwg, st);
      break;
  }
  return hipGetLastError();
}

}  // namespace hx
