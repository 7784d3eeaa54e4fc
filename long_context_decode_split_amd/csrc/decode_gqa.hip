// Split-KV decode attention for GQA caches (Dk = Dv = 128, up to 16 query
// heads per KV head) on gfx950.
//
// What one launch computes (Helix summary, paragraph on KV parallelism): for
// every request b, KV head g and slice r, the partial attention of the G
// query heads of g over the rows of slice r, as a normalised output and a
// natural-log LSE.  The rows of a slice are cut into splits of `cpw` 16-row
// chunk tiles so the launch fills the GPU; each workgroup streams one split
// and writes its partial (straight into the slice's output when the slice has
// a single split).  A second, small kernel folds the splits of each slice with
// the LSE combine (jaehun.me review, Prompt 1.3.2): the kernel boundary makes
// the records visible, where an in-kernel last-workgroup fold would need a
// device-scope release and acquire per workgroup (an L2 write-back and
// invalidate each), which measured at about 15% of the kernel time.
//
// Work per wave, per 16-row chunk tile (no LDS on the streaming path):
//   * 4 x 16 B loads of K and 4 x 16 B loads of V (bf16; fewer for fp8 and
//     MXFP4), each wave-wide load reading 1 KiB contiguous;
//   * S^T = K Q^T with four v_mfma_f32_16x16x32_bf16 (rows = tokens,
//     columns = query heads);
//   * online softmax in base 2 on the accumulator layout: lane l holds the
//     scores of head l % 16 for tokens 4*(l/16)..+3, so the row max needs two
//     lane exchanges and the running sum stays per lane;
//   * O^T += V^T P^T with eight v_mfma_f32_16x16x16_bf16, whose B operand is
//     the probability fragment exactly as the first product left it (bf16
//     tiles: sixteen, P as a bf16 high part plus its residual).
// The rescale of the accumulator runs only on tiles that move a head's
// reference max (bf16: any growth; fp8 / MXFP4: growth by more than 2^8).
// Template parameters: storage format, dense or block-pool addressing, waves
// per workgroup (8 for short unsplit slices), and whether the workgroup first
// appends a decode step's new rows into its tiles (hx_decode_step).

#include <type_traits>

#include "hx_append.h"
#include "hx_gqa_frag.h"

namespace hx {
namespace {

using namespace frag;

// Chunk tiles a wave keeps in flight (register budget: 32 VGPRs per bf16
// tile).  fp8 measured 4-5% faster with two than with three or four (same
// box); MXFP4 runs the same with two to four.
#ifndef HX_GQA_TILES_BF16
#define HX_GQA_TILES_BF16 2
#endif
#ifndef HX_GQA_TILES_FP8
#define HX_GQA_TILES_FP8 2
#endif
#ifndef HX_GQA_TILES_FP4
#define HX_GQA_TILES_FP4 3
#endif
template <int FMT>
constexpr int kTilesInFlight = FMT == 0 ? HX_GQA_TILES_BF16 : (FMT == 1 ? HX_GQA_TILES_FP8 : HX_GQA_TILES_FP4);
constexpr int kD = 128;
constexpr float kLn2 = 0.693147180559945309f;
// log2 of the largest unnormalised probability (see chunk_step).  bf16
// caches keep the reference at the running max (P <= 1, and the rows at the
// max get the exact weight 1); the quantised formats, whose dequantisation
// leaves less VALU time per tile, let it lag by up to 2^8.
#ifndef HX_GQA_HEADROOM_Q
#define HX_GQA_HEADROOM_Q 8.0f
#endif
template <int FMT>
constexpr float kHeadroom = FMT == 0 ? 0.0f : HX_GQA_HEADROOM_Q;

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// KV bytes are read exactly once: streaming (non-temporal) 16-byte loads, so
// they do not evict what is reused (Q, partials) from the caches.
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}


// Raw bytes of one chunk tile that a lane needs; FMT 0 bf16, 1 fp8, 2 MXFP4.
template <int FMT>
struct Frag;

template <>
struct Frag<0> {
  uint4 k[4], v[4];
  __device__ __forceinline__ void load(const uint8_t* kt, const uint8_t* vt, const uint8_t*, const uint8_t*, int lane,
                                       int) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = ld16(kt + i * 1024 + lane * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld16(vt + i * 1024 + lane * 16);
  }
};

template <>
struct Frag<1> {
  uint4 k[2], v[2];
  float ks, vs;
  __device__ __forceinline__ void load(const uint8_t* kt, const uint8_t* vt, const uint8_t* kst, const uint8_t* vst,
                                       int lane, int) {
#pragma unroll
    for (int i = 0; i < 2; ++i) k[i] = ld16(kt + i * 1024 + lane * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) v[i] = ld16(vt + i * 1024 + lane * 16);
    ks = *reinterpret_cast<const float*>(kst);
    vs = *reinterpret_cast<const float*>(vst);
  }
};

template <>
struct Frag<2> {
  uint4 k, v, vsc;
  uint32_t ksc;
  __device__ __forceinline__ void load(const uint8_t* kt, const uint8_t* vt, const uint8_t* kst, const uint8_t* vst,
                                       int lane, int) {
    k = ld16(kt + lane * 16);
    v = ld16(vt + lane * 16);
    ksc = *reinterpret_cast<const uint32_t*>(kst + (lane & 15) * 4);    // 4 e8m0 of token m
    vsc = ld16(vst + (lane >> 4) * 16);                               // tokens 4h..4h+3, 4 blocks each
  }
};

// Running state of one wave: O^T accumulator (lane l: heads l%16, value
// columns 16*nb + 4*(l/16) + i), the running max of head l%16 in base-2
// units (equal on the four lanes of a head), and this lane's shares of two
// running sums: of the probabilities as rounded for the matrix cores (it
// normalises O, keeping O a convex combination of V rows) and of the exact
// probabilities (it gives the LSE).
struct WaveState {
  f32x4 acc[8];
  float mrun;
  float lsum_mfma;
  float lsum;
};

// One 16-row chunk tile: scores, online softmax, O^T += V^T P^T.  TAIL marks
// the last tile of a slice, whose rows at or past `valid` are masked (their
// bytes may be anything, NaN included).
template <int FMT, bool TAIL>
__device__ __forceinline__ void chunk_step(const Frag<FMT>& cur, WaveState& st, const bf16x8 (&qf)[4], float c2,
                                           int h, int valid) {
  // ---- K fragments as bf16
  bf16x8 kf[4];
  float cscale = c2;
  if constexpr (FMT == 0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) kf[s] = as_bf16x8(cur.k[s]);
  } else if constexpr (FMT == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t w[4] = {cur.k[i].x, cur.k[i].y, cur.k[i].z, cur.k[i].w};
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {   // bytes 0-7 -> step 2i, 8-15 -> step 2i+1
        uint4 t;
        t.x = fp8x2_to_bf16x2<false>(w[2 * hs]);
        t.y = fp8x2_to_bf16x2<true>(w[2 * hs]);
        t.z = fp8x2_to_bf16x2<false>(w[2 * hs + 1]);
        t.w = fp8x2_to_bf16x2<true>(w[2 * hs + 1]);
        kf[2 * i + hs] = as_bf16x8(t);
      }
    }
    cscale = c2 * cur.ks;
  } else {
    const uint32_t w[4] = {cur.k.x, cur.k.y, cur.k.z, cur.k.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float sc = e8m0_sel(cur.ksc, s);
      uint4 t;
      t.x = fp4x2_to_bf16x2<0>(w[s], sc);
      t.y = fp4x2_to_bf16x2<1>(w[s], sc);
      t.z = fp4x2_to_bf16x2<2>(w[s], sc);
      t.w = fp4x2_to_bf16x2<3>(w[s], sc);
      kf[s] = as_bf16x8(t);
    }
  }

  // ---- scores: S^T[token 4h+i][head m]
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], sc, 0, 0, 0);

  // fp8: the tile's K scale is applied to the scores before the max and the
  // masking, so a zero scale (scores 0) or a negative one (order reversed)
  // still gives the right max, and masked rows stay at exactly -inf (a
  // masked -inf times a zero scale would be NaN).  The other formats scale
  // by c2 > 0 inside the exponent.
  if constexpr (FMT == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] *= cscale;
  }
  uint32_t keep01 = 0xffffffffu, keep23 = 0xffffffffu;   // V halves of tokens 4h+{0,1} / 4h+{2,3}
  if constexpr (TAIL) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * h + i >= valid) sc[i] = -INFINITY;
    keep01 = (4 * h + 0 < valid ? 0x0000ffffu : 0u) | (4 * h + 1 < valid ? 0xffff0000u : 0u);
    keep23 = (4 * h + 2 < valid ? 0x0000ffffu : 0u) | (4 * h + 3 < valid ? 0xffff0000u : 0u);
  }

  // ---- online softmax (base 2)
  float cm = fmaxf(vmax(sc[0], sc[1]), vmax(sc[2], sc[3]));
  cm = max_xor32(max_xor16(cm));
  // The reference max mrun moves only when some head's scores exceed it by
  // more than kHeadroom: P = 2^(s - mrun) is bounded by 2^kHeadroom, and the
  // rescale of the accumulator (32 multiplies; a factor of exactly 1 for the
  // heads whose max did not move) runs only on the tiles that raise it.
  const float cms = FMT == 1 ? cm : cm * cscale;
  if (__any(cms > st.mrun + kHeadroom<FMT>)) {   // wave-uniform
    const float mnew = fmaxf(st.mrun, cms);
    const float alpha = __builtin_amdgcn_exp2f(st.mrun - mnew);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[i] *= alpha;
    st.lsum_mfma *= alpha;
    st.lsum *= alpha;
    st.mrun = mnew;
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    p[i] = __builtin_amdgcn_exp2f(FMT == 1 ? sc[i] - st.mrun : fmaf(sc[i], cscale, -st.mrun));
  st.lsum += (p[0] + p[1]) + (p[2] + p[3]);

  // ---- P^T fragments (bf16) and V^T fragments, then O^T += V^T P^T
  if constexpr (FMT == 0) {
    // P enters the matrix cores as two bf16 fragments, its rounding and the
    // bf16 of the residual, so the products carry about 16 significant bits
    // of P: with one bf16 fragment the output error can reach 2^-8 times half
    // the range of V (a few weights dominate in short slices), above the
    // 2e-3 bound for bf16 caches.  The second set of products is cheap here:
    // bf16 tiles leave the matrix cores mostly idle.
    const uint32_t p01 = pack_bf16(p[0], p[1]), p23 = pack_bf16(p[2], p[3]);
    const uint32_t r01 = pack_bf16(p[0] - bf16lo(p01), p[1] - bf16hi(p01));
    const uint32_t r23 = pack_bf16(p[2] - bf16lo(p23), p[3] - bf16hi(p23));
    st.lsum_mfma = add_bf16x2(r23, add_bf16x2(r01, add_bf16x2(p23, add_bf16x2(p01, st.lsum_mfma))));
    const s16x4 ph = as_s16x4(p01, p23), pl = as_s16x4(r01, r23);
    s16x4 va[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 vv = cur.v[i];
      va[2 * i] = as_s16x4(vv.x & keep01, vv.y & keep23);
      va[2 * i + 1] = as_s16x4(vv.z & keep01, vv.w & keep23);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[i], ph, st.acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[i], pl, st.acc[i], 0, 0, 0);
  } else if constexpr (FMT == 1) {
    // The tile's V scale is folded into P; the rounded products, divided by
    // the scale, are what normalises O.  A zero V scale makes the tile's
    // values exactly 0: its weights then enter the normalisation unrounded.
    const float vsc = cur.vs;
    const uint32_t p01 = pack_bf16(p[0] * vsc, p[1] * vsc), p23 = pack_bf16(p[2] * vsc, p[3] * vsc);
    const float rounded = add_bf16x2(p23, add_bf16x2(p01, 0.f));
    st.lsum_mfma += vsc != 0.f ? rounded * __builtin_amdgcn_rcpf(vsc) : (p[0] + p[1]) + (p[2] + p[3]);
    const s16x4 pb = as_s16x4(p01, p23);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t w[4] = {cur.v[i].x, cur.v[i].y, cur.v[i].z, cur.v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {   // value block nb = 4i + q: 4 codes (tokens 4h..4h+3)
        const uint32_t lo = fp8x2_to_bf16x2<false>(w[q]) & keep01;
        const uint32_t hi = fp8x2_to_bf16x2<true>(w[q]) & keep23;
        st.acc[4 * i + q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_s16x4(lo, hi), pb, st.acc[4 * i + q], 0, 0, 0);
      }
    }
  } else {
    // Per (token, 32-column block) scales are powers of two: fold them into
    // P, one P fragment per block, by adding them into the exponents of P's
    // bf16 pairs (scale_bf16x2_e8m0), which gives the rounded product.  So
    // the sum of the rounded, unscaled P is what normalises O.  P enters
    // clamped at 2^-126 below (a weight that small relative to the reference
    // adds at most 2^-126 |V| per row; an exact 0 would not stay 0 through
    // the exponent arithmetic).
    const float kMinP = 1.17549435e-38f;   // 2^-126
    const uint32_t p01 = pack_bf16(fmaxf(p[0], kMinP), fmaxf(p[1], kMinP));
    const uint32_t p23 = pack_bf16(fmaxf(p[2], kMinP), fmaxf(p[3], kMinP));
    st.lsum_mfma = add_bf16x2(p23, add_bf16x2(p01, st.lsum_mfma));
    const uint32_t vs[4] = {cur.vsc.x, cur.vsc.y, cur.vsc.z, cur.vsc.w};   // token 4h+j: 4 block scales
    const uint32_t w[4] = {cur.v.x, cur.v.y, cur.v.z, cur.v.w};
    auto block = [&](auto blk_t) {
      constexpr int blk = decltype(blk_t)::value;
      uint32_t s01 = scale_bf16x2_e8m0(p01, e8m0_pair<blk>(vs[0], vs[1]));
      uint32_t s23 = scale_bf16x2_e8m0(p23, e8m0_pair<blk>(vs[2], vs[3]));
      if constexpr (TAIL) {   // rows past the slice end may hold any scale byte
        s01 &= keep01;
        s23 &= keep23;
      }
      const s16x4 pb = as_s16x4(s01, s23);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int nb = 2 * blk + hb;   // bytes 2nb, 2nb+1 of the lane's 16 B
        const uint32_t word = w[nb >> 1];
        uint32_t lo, hi;
        if ((nb & 1) == 0) {
          lo = fp4x2_to_bf16x2<0>(word, 1.0f);
          hi = fp4x2_to_bf16x2<1>(word, 1.0f);
        } else {
          lo = fp4x2_to_bf16x2<2>(word, 1.0f);
          hi = fp4x2_to_bf16x2<3>(word, 1.0f);
        }
        st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_s16x4(lo & keep01, hi & keep23), pb, st.acc[nb], 0, 0, 0);
      }
    };
    block(std::integral_constant<int, 0>{});
    block(std::integral_constant<int, 1>{});
    block(std::integral_constant<int, 2>{});
    block(std::integral_constant<int, 3>{});
  }
}

template <int FMT, bool PAGED, int WAVES, int FUSE>
__global__ __launch_bounds__(64 * WAVES) void gqa_partial_kernel(const PartialArgs a) {
  constexpr int kWaves = WAVES;
  constexpr int kThreads = 64 * kWaves;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
  const int tail_valid = (int)(L - (int64_t)(nch - 1) * kChunk);   // rows in the last chunk

  // Dense cache: the slice's tiles are consecutive from tile0.  Block pool:
  // chunk c is the tile of head g in block trow[c] (tile_of in hx_common.h).
  const int64_t tile0 = PAGED ? 0 : ((int64_t)(r * a.Btot + b) * a.Hkv + g) * a.cap_chunks;
  const int32_t* trow = PAGED ? a.table + ((int64_t)b * a.P + r) * a.cap_chunks : nullptr;
  auto pool_tile = [&](int c) -> int64_t { return clamp_block(trow[c], a.num_blocks) * a.Hkv + g; };
  const uint8_t* kp = a.k + tile0 * a.k_tile;
  const uint8_t* vp = a.v + tile0 * a.v_tile;
  const uint8_t* ksp = a.ks ? a.ks + tile0 * a.ks_tile : nullptr;
  const uint8_t* vsp = a.vs ? a.vs + tile0 * a.vs_tile : nullptr;

  // ---- query fragment: B operand of S^T = K Q^T, head m, columns 32s+8h..+7
  bf16x8 qf[4];
  {
    const bool live = m < a.G;
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + g * a.G + (live ? m : 0)) * a.Dk;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 t = *reinterpret_cast<const uint4*>(qrow + s * 32 + h * 8);
      if (!live) t = make_uint4(0, 0, 0, 0);
      qf[s] = as_bf16x8(t);
    }
  }

  WaveState st;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.mrun = -INFINITY;
  st.lsum_mfma = 0.f;
  st.lsum = 0.f;

  const float c2 = a.c2;
  // Tile c of a dense slice lies at kp + c * k_tile (and likewise for V and
  // the scales).  Loads go through byte cursors that hold wave-uniform
  // offsets, so addresses are a scalar base plus the lane's 16-byte offset.
  auto load_at = [&](Frag<FMT>& f, int64_t ok, int64_t ov, int64_t oks, int64_t ovs) {
    if constexpr (FMT == 0)
      f.load(kp + ok, vp + ov, nullptr, nullptr, lane, 0);
    else
      f.load(kp + ok, vp + ov, ksp + oks, vsp + ovs, lane, 0);
  };
  // The slice's partial last tile (if this split holds it) is taken out of
  // the streaming loop and done once at the end, so the loop has no branch.
  const bool has_tail = c1 == nch && c1 > c0 && tail_valid < kChunk;
  const int c1f = has_tail ? c1 - 1 : c1;

  // NBUF tiles in flight per wave: each reload goes straight into the
  // registers of the tile just consumed.  The steady-state loop issues its
  // loads unconditionally so the wait counts stay exact (the wave keeps the
  // other tiles' loads in flight while it computes); the last tiles are
  // drained after it.  A wave takes chunks c0 + wave, + kWaves, ... in order,
  // so one cursor advanced by kWaves tiles per load covers all its loads.
  constexpr int NBUF = kTilesInFlight<FMT>;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int first = c0 + wv;
  const int nmine = __builtin_amdgcn_readfirstlane(first < c1f ? (c1f - first + kWaves - 1) / kWaves : 0);
  if (nmine > 0) {
    int64_t ok = (int64_t)first * a.k_tile, ov = (int64_t)first * a.v_tile;
    int64_t oks = (int64_t)first * a.ks_tile, ovs = (int64_t)first * a.vs_tile;
    const int64_t dk = (int64_t)kWaves * a.k_tile, dv = (int64_t)kWaves * a.v_tile;
    const int64_t dks = (int64_t)kWaves * a.ks_tile, dvs = (int64_t)kWaves * a.vs_tile;
    // pool: the tile of the next load, looked up one load ahead (a scalar
    // load whose latency the tile in between covers); lookups stop at the
    // wave's last chunk, so only entries of the slice's rows are read
    int cn = first;
    const int clast = c1f - 1;
    int64_t tn = PAGED ? pool_tile(first) : 0;
    auto load_next = [&](Frag<FMT>& f, bool advance) {
      if constexpr (PAGED) {
        load_at(f, tn * a.k_tile, tn * a.v_tile, tn * a.ks_tile, tn * a.vs_tile);
        if (advance) {
          cn += kWaves;
          tn = pool_tile(min(cn, clast));
        }
      } else {
        load_at(f, ok, ov, oks, ovs);
        if (advance) {
          ok += dk;
          ov += dv;
          oks += dks;
          ovs += dvs;
        }
      }
    };
    Frag<FMT> f[NBUF];
    // with fewer than NBUF tiles the cursor stays on the last one
#pragma unroll
    for (int k = 0; k < NBUF; ++k) load_next(f[k], k + 1 < nmine);
    int i = 0;
    for (; i + 2 * NBUF - 1 < nmine; i += NBUF) {
#pragma unroll
      for (int k = 0; k < NBUF; ++k) {
        chunk_step<FMT, false>(f[k], st, qf, c2, h, kChunk);
        load_next(f[k], true);
#if HX_GQA_SCHED_BARRIER
        __builtin_amdgcn_sched_barrier(0);   // keep the next tile's math below this reload
#endif
      }
    }
#pragma unroll
    for (int k = 0; k < NBUF; ++k) {
      if (i + k < nmine) {
        chunk_step<FMT, false>(f[k], st, qf, c2, h, kChunk);
        if (i + k + NBUF < nmine) load_next(f[k], true);
      }
    }
#pragma unroll
    for (int k = 0; k < NBUF; ++k)
      if (i + NBUF + k < nmine) chunk_step<FMT, false>(f[k], st, qf, c2, h, kChunk);
  }
  if (has_tail && wave == (c1 - 1 - c0) % kWaves) {
    const int64_t c = PAGED ? pool_tile(c1 - 1) : c1 - 1;
    Frag<FMT> t;
    load_at(t, c * a.k_tile, c * a.v_tile, c * a.ks_tile, c * a.vs_tile);
    chunk_step<FMT, true>(t, st, qf, c2, h, tail_valid);
  }
  float mrun = st.mrun, lsum = st.lsum, lsum_mfma = st.lsum_mfma;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = st.acc[i];

  // ---- fold the lanes' running sums of each head
  lsum = sum_xor32(sum_xor16(lsum));
  lsum_mfma = sum_xor32(sum_xor16(lsum_mfma));

  // ---- combine the waves of this workgroup (LSE rule, base 2)
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_lm[kWaves][16];
  __shared__ float s_acc[kWaves][16][kD + 4];
  if (h == 0) {
    s_m[wave][m] = mrun;
    s_l[wave][m] = lsum;
    s_lm[wave][m] = lsum_mfma;
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
    *reinterpret_cast<f32x4*>(&s_acc[wave][m][16 * nb + 4 * h]) = acc[nb];
  __syncthreads();

  const int G = a.G;
  const bool direct = nsplit == 1;
  float* out_o;
  float* out_l;
  int64_t ostride_head;   // floats between heads in the output
  if (direct) {
    out_o = a.o_part + (((int64_t)r * a.Btot + b) * a.Hq + g * G) * a.Dv;
    out_l = a.lse_part + ((int64_t)r * a.Btot + b) * a.Hq + g * G;
  } else {
    out_o = a.ws_o + (int64_t)wg * G * a.Dv;
    out_l = a.ws_lse + (int64_t)wg * G;
  }
  ostride_head = a.Dv;
  for (int idx = threadIdx.x; idx < G * kD; idx += kThreads) {
    const int hd = idx / kD, dv = idx % kD;
    float M = s_m[0][hd];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][hd]);
    float num = 0.f, den = 0.f, den_mfma = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(s_m[w][hd] - M);
        num += f * s_acc[w][hd][dv];
        den += f * s_l[w][hd];
        den_mfma += f * s_lm[w][hd];
      }
    }
    out_o[hd * ostride_head + dv] = den_mfma > 0.f ? num / den_mfma : 0.f;
    if (dv == 0) out_l[hd] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
  }

}

template <int FMT, bool PAGED, int FUSE>
void launch_waves(const PartialArgs& a, int nwg, hipStream_t st) {
  if (a.waves == kGqaShortWaves)
    hipLaunchKernelGGL((gqa_partial_kernel<FMT, PAGED, kGqaShortWaves, FUSE>), dim3(nwg), dim3(64 * kGqaShortWaves), 0,
                       st, a);
  else
    hipLaunchKernelGGL((gqa_partial_kernel<FMT, PAGED, kGqaWavesPerWg, FUSE>), dim3(nwg), dim3(64 * kGqaWavesPerWg), 0,
                       st, a);
}

// Fused append modes per format: bf16 rows are the storage format (mode 1);
// fp8 caches take stored codes (1) or bf16 rows to quantise (2); MXFP4
// caches only the quantising mode (2): a step with stored MXFP4 codes runs
// the append kernel first (the copy's registers slowed the kernel's loop by
// 5% (dense) to 19% (block pool), more than the launch it saves).
template <int FMT, bool PAGED>
void launch_fmt(const PartialArgs& a, int nwg, hipStream_t st) {
  if constexpr (FMT == 1) {
    if (a.fused_append == 1) return launch_waves<FMT, PAGED, 1>(a, nwg, st);
  }
  if constexpr (FMT == 0) {
    if (a.fused_append) return launch_waves<FMT, PAGED, 1>(a, nwg, st);
  } else {
    if (a.fused_append == 2) return launch_waves<FMT, PAGED, 2>(a, nwg, st);
  }
  launch_waves<FMT, PAGED, 0>(a, nwg, st);
}

}  // namespace

hipError_t launch_gqa_partial(const PartialArgs& a, int dtype, hipStream_t st) {
  const int nwg = a.wg_begin[a.nb];
  if (nwg == 0) return hipSuccess;
  const bool paged = a.table != nullptr;
  switch (dtype) {
    case HX_KV_BF16:
      paged ? launch_fmt<0, true>(a, nwg, st) : launch_fmt<0, false>(a, nwg, st);
      break;
    case HX_KV_FP8_E4M3:
      paged ? launch_fmt<1, true>(a, nwg, st) : launch_fmt<1, false>(a, nwg, st);
      break;
    default:
      paged ? launch_fmt<2, true>(a, nwg, st) : launch_fmt<2, false>(a, nwg, st);
      break;
  }
  return hipGetLastError();
}

}  // namespace hx
