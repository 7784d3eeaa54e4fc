// Split-KV decode attention for MLA caches on gfx950: one latent KV head of
// 576 columns whose first 512 columns are also the value row, 128 query heads
// per latent head (the DeepSeek-R1 shape of the Helix review, Prompt 1.4.1;
// the Helix summary notes MLA effectively has one KV head).
//
// The query-group contraction is dense here (128 heads share every latent
// row), so both products run on v_mfma_f32_32x32x16_bf16:
//   S^T[32 tokens][32 heads] = K[32 tokens][576] . Q^T[576][32 heads]
//   O^T[512][32 heads]      += V^T[512][32 tokens] . P^T[32 tokens][32 heads]
//
// A workgroup of eight waves streams a run of 32-token tiles of one slice.
// Wave w works on head group hg = w % 4 (heads 32 hg .. +31) and half
// dh = w / 4 of both contractions: k-steps 18 dh .. +17 of the score product
// (its Q^T fragments: 12 in VGPRs, 6 parked in LDS) and value blocks
// 8 dh .. +7 of the output (its accumulator, 128 VGPRs).  The two waves of a
// head group add their partial scores through LDS, so both hold the same
// scores and run the same softmax.  With everything in VGPRs the softmax
// rescale is a plain multiply and two waves fit on each SIMD.
//
// A tile (two chunk tiles, 36 KiB) is copied from HBM into LDS unchanged with
// direct global-to-LDS loads (no VGPRs), the next tile loading while one is
// used.  The cache
// stores each latent row with its 16-byte pieces XOR-swizzled inside aligned
// groups of 8, so the unchanged copy is already bank-conflict free for both
// views: every wave reads the K view with 16-byte LDS loads and the
// transposed V view with ds_read_b64_tr_b16, and one stored copy of the latent
// row serves both products.
//
// Lane layouts used below (64-lane wave, l = lane, half = l / 32):
//   32x32x16 A operand: row l % 32, k = 8 * half + j (j = 0..7);
//   B operand: column l % 32, same k; C/D: register r holds row
//   8 * (r / 4) + 4 * half + r % 4, column l % 32.
//   ds_read_b64_tr_b16, per group of 16 lanes: lane i receives element i % 4
//   of the 4-element reads of lanes i / 4 + 4 k, k = 0..3.

#include "hx_common.h"

namespace hx {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerGroup = 32;
constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kTileTok = 32;                       // tokens per LDS tile (two chunk tiles)
constexpr int kRowBytes = kDk * 2;                 // 1152
constexpr int kTileBytes = kTileTok * kRowBytes;   // 36 KiB
constexpr int kTileBlocks = kTileBytes / 1024;     // 1 KiB direct loads per tile (36)
constexpr int kNBuf = 2;                           // tiles in flight
constexpr int kSteps = kDk / 16;                   // k-steps of the score product (36)
constexpr int kHalfSteps = kSteps / 2;             // per wave (18)
constexpr int kVBlocks = kDv / 32;                 // 32-column value blocks (16)
constexpr int kHalfVBlocks = kVBlocks / 2;         // per wave (8)
constexpr int kQLds = 6;                           // of a wave's 18 Q^T fragments, the first 6 live in LDS
constexpr float kLn2 = 0.693147180559945309f;

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint4 lds_u4;
typedef __attribute__((address_space(3))) f32x4 lds_f4;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// One direct global-to-LDS load of 16 bytes per lane: lane l's bytes from
// sbase + voff land at LDS byte lds + 16 l (M0 holds the wave-uniform LDS
// base).  Issued from inline assembly so the compiler does not treat the
// address registers as pending load results (it would otherwise wait for the
// next tile's loads before every reuse of those registers).  Completion is
// awaited with explicit vmcnt waits before the barrier that publishes a tile;
// no other M0 user is live in the kernel.
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  const uint64_t sb = (uint64_t)sbase;
  const uint64_t sbu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbu),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Workgroup barrier after this wave's outstanding loads have landed: global
// (and direct-to-LDS) loads down to VMCNT still in flight, all LDS accesses
// done.  The asm is also a compiler memory barrier, so no LDS access moves
// across it.
template <int VMCNT>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VMCNT) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

__global__ __launch_bounds__(kThreads) void mla_partial_kernel(const PartialArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // device-only builtins (LDS address space) below
  __shared__ __attribute__((aligned(1024))) uint8_t s_tile[kNBuf][kTileBytes];
  __shared__ __attribute__((aligned(1024))) float s_part[kWaves][16][64];   // partial scores per wave
  // Q^T fragments that do not fit in registers next to the accumulator:
  // [wave][step][lane] x 16 B; each lane reads back only what it wrote.
  __shared__ __attribute__((aligned(1024))) uint8_t s_q[kWaves][kQLds][1024];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int hg = wave & 3;     // head group
  const int dh = wave >> 2;    // contraction half

  // ---- which (request, latent head, slice, split) this workgroup owns
  const int wg = blockIdx.x;
  int bl = 0;
  while (bl + 1 < a.nb && a.wg_begin[bl + 1] <= wg) ++bl;
  const int nsplit = a.nsplit[bl];
  int rem = wg - a.wg_begin[bl];
  const int split = rem % nsplit;
  rem /= nsplit;
  const int r = rem % a.P;
  const int g = rem / a.P;
  const int b = a.b0 + bl;

  const int64_t L = slice_len(a.n[bl], a.P, r);
  const int64_t t_begin = (int64_t)split * a.cpw * kChunk;   // cpw is even: tiles start on 32 rows
  const int64_t t_end = min((int64_t)(split + 1) * a.cpw * kChunk, L);
  const int ntok = t_end > t_begin ? (int)(t_end - t_begin) : 0;
  const int ntiles = (ntok + kTileTok - 1) / kTileTok;

  const int64_t tile0 = ((int64_t)(r * a.Btot + b) * a.Hkv + g) * a.cap_chunks;
  const uint8_t* base = a.k + tile0 * a.k_tile + t_begin * kRowBytes;   // latent rows, 1152 B each

  // ---- Q^T fragments of head 32 hg + col for k-steps 18 dh .. +17 (B
  //      operand: step s covers columns 16 s + 8 half .. +7)
  bf16x8 qf[kHalfSteps - kQLds];
  {
    const int head = g * a.G + kHeadsPerGroup * hg + col;
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + head) * kDk + 16 * kHalfSteps * dh + 8 * half;
#pragma unroll
    for (int s = 0; s < kQLds; ++s)
      *(lds_u4*)((lds_u8*)&s_q[wave][s][0] + 16 * lane) = *reinterpret_cast<const uint4*>(qrow + 16 * s);
#pragma unroll
    for (int s = kQLds; s < kHalfSteps; ++s)
      qf[s - kQLds] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 16 * s));
  }
  const lds_u8* q_lds = (const lds_u8*)&s_q[wave][0][0] + 16 * lane;
  // Q is in place before any tile load is issued, so no wait the compiler
  // derives for Q can later count the tile loads.
  __builtin_amdgcn_s_waitcnt(0);

  // ---- direct global -> LDS copy of tile k into buffer buf: 1 KiB blocks
  //      w, w + 8, ... (waves 0-3 move five, 4-7 four); lane l moves bytes
  //      16 l .. +15 of each.  Rows past the slice end (last tile only) are
  //      fetched from row 0 of the tile instead: finite values that the
  //      masked scores give weight 0.
  const int nload = wave < 4 ? 5 : 4;
  const uint32_t lane_off = 16u * lane;
  auto load_tile = [&](int k, int buf) {
    const int valid = min(kTileTok, ntok - k * kTileTok);
    const uint8_t* src = base + (int64_t)k * kTileBytes;
    uint8_t* dst = &s_tile[buf][0];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int blk = wave + kWaves * j;
      uint32_t off = blk * 1024u + lane_off;   // byte of the tile this lane moves
      if (valid < kTileTok && off / kRowBytes >= (uint32_t)valid) off %= kRowBytes;
      if (j < 4 || wave < 4) dma16(off, src, lds_addr(dst + blk * 1024));
    }
  };

  f32x16 acc[kHalfVBlocks];
#pragma unroll
  for (int i = 0; i < kHalfVBlocks; ++i) acc[i] = f32x16{};
  float mrun = -INFINITY;   // running max of head 32 hg + col (base 2)
  float lsum = 0.f, lsum_mfma = 0.f;
  const float c2 = a.c2;

  // per-lane LDS byte offsets inside a tile.  K view: row col, piece
  // 2 s + half + 36 dh, swizzled by row; 4 consecutive k-steps move 8 pieces
  // (128 B), so offsets repeat with period 4 plus an immediate.
  const int swk = mla_swz(col);
  int k_off[4];   // steps s and s + 4 differ by 8 pieces (128 B): four bases, immediate offsets
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int pc = 2 * s + half + 2 * kHalfSteps * dh;
    k_off[s] = kRowBytes * col + 16 * ((pc & ~7) | ((pc & 7) ^ swk));
  }
  // V view for ds_read_b64_tr_b16: lane i16 of its 16-lane group reads row
  // 16 u + 4 half + i16 / 4 (+ 8 for the second half of the k-step), columns
  // 32 nb + 16 cb + 4 (i16 % 4) .. +3, i.e. piece 4 nb + 2 cb + (i16 % 4) / 2;
  // value blocks 8 dh + nb.  nb and nb + 2 differ by 8 pieces: two bases.
  const int i16 = lane & 15;
  const int cb = (lane >> 4) & 1;
  const int vrow = 4 * half + (i16 >> 2);
  const int swv = mla_swz(vrow);   // rows + 8 and + 16 share the swizzle
  int v_off[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int pc = 4 * (kHalfVBlocks * dh + e) + 2 * cb + ((i16 & 3) >> 1);
    v_off[e] = kRowBytes * vrow + 16 * ((pc & ~7) | ((pc & 7) ^ swv)) + 8 * (i16 & 1);
  }
  lds_f4* my_part = (lds_f4*)&s_part[wave][0][0] + lane;
  const lds_f4* other_part = (const lds_f4*)&s_part[wave ^ 4][0][0] + lane;

  // tile k + 1 loads while tile k is used
  if (ntiles > 0) load_tile(0, 0);
  for (int k = 0; k < ntiles; ++k) {
    const int buf = k % kNBuf;
    if (k + 1 < ntiles) {
      load_tile(k + 1, (k + 1) % kNBuf);
      // wait for tile k's blocks: the newer loads are tile k + 1's
      if (wave < 4) wait_barrier<5>();
      else wait_barrier<4>();
    } else {
      wait_barrier<0>();
    }
    const lds_u8* tb = (const lds_u8*)&s_tile[buf][0];

    // ---- partial scores over this wave's 18 k-steps
    f32x16 sc = {};
    uint4 kv[kHalfSteps];
    uint4 qv[kQLds];
#pragma unroll
    for (int s = 0; s < 2; ++s) kv[s] = *(const lds_u4*)(tb + k_off[s & 3] + 128 * (s >> 2));
#pragma unroll
    for (int s = 0; s < 2; ++s) qv[s] = *(const lds_u4*)(q_lds + 1024 * s);
#pragma unroll
    for (int s = 0; s < kHalfSteps; ++s) {
      if (s + 2 < kHalfSteps) kv[s + 2] = *(const lds_u4*)(tb + k_off[(s + 2) & 3] + 128 * ((s + 2) >> 2));
      if (s + 2 < kQLds) qv[s + 2] = *(const lds_u4*)(q_lds + 1024 * (s + 2));
      const bf16x8 qb = s < kQLds ? __builtin_bit_cast(bf16x8, qv[s < kQLds ? s : 0]) : qf[s < kQLds ? 0 : s - kQLds];
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv[s]), qb, sc, 0, 0, 0);
    }
    // ---- add the other half's partial scores (same lanes, same registers)
#pragma unroll
    for (int i = 0; i < 4; ++i) my_part[64 * i] = f32x4{sc[4 * i], sc[4 * i + 1], sc[4 * i + 2], sc[4 * i + 3]};
    wait_barrier<63>();   // the partial scores are in LDS (tile loads may still fly)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 o = other_part[64 * i];
      // fixed order (half 0's partial first) so both waves of the pair get identical sums
      if (dh == 0) {
        sc[4 * i] += o.x; sc[4 * i + 1] += o.y; sc[4 * i + 2] += o.z; sc[4 * i + 3] += o.w;
      } else {
        sc[4 * i] = o.x + sc[4 * i]; sc[4 * i + 1] = o.y + sc[4 * i + 1];
        sc[4 * i + 2] = o.z + sc[4 * i + 2]; sc[4 * i + 3] = o.w + sc[4 * i + 3];
      }
    }
    const int valid = min(kTileTok, ntok - k * kTileTok);
    if (valid < kTileTok) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * half + (i & 3) >= valid) sc[i] = -INFINITY;
    }

    // ---- online softmax (base 2)
    float cm = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) cm = fmaxf(cm, sc[i]);
    cm = fmaxf(cm, __shfl_xor(cm, 32)) * c2;
    const float mnew = fmaxf(mrun, cm);
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
#pragma unroll
    for (int i = 0; i < kHalfVBlocks; ++i) acc[i] *= alpha;
    lsum *= alpha;
    lsum_mfma *= alpha;
    mrun = mnew;
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[2 * i], c2, -mrun));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[2 * i + 1], c2, -mrun));
      lsum += p0 + p1;
      pk[i] = pack_bf16(p0, p1);
      lsum_mfma += bf16lo(pk[i]) + bf16hi(pk[i]);
    }

    // ---- O^T += V^T P^T over this wave's 8 value blocks.  k-step u takes P
    //      registers 8u..8u+7 = tokens 16u + 4 half + (0..3) and
    //      16u + 8 + 4 half + (0..3); the V^T operand is two transposed reads.
    auto vread = [&](int i) {   // i = 8u + nb
      const int nb = i & 7;
      const lds_u8* vp = tb + v_off[nb & 1] + 128 * (nb >> 1) + kRowBytes * 16 * (i >> 3);
      const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp));
      const uint2 hi =
          __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + kRowBytes * 8)));
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
    uint4 vv[2 * kHalfVBlocks];
    vv[0] = vread(0);
#pragma unroll
    for (int i = 0; i < 2 * kHalfVBlocks; ++i) {
      if (i + 1 < 2 * kHalfVBlocks) vv[i + 1] = vread(i + 1);
      const int u = i >> 3, nb = i & 7;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]));
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv[i]), pb, acc[nb], 0, 0, 0);
    }
    wait_barrier<63>();   // every wave is done with this buffer and the partial scores
  }

  // ---- finalize: this wave's heads, its half of the value columns
  lsum += __shfl_xor(lsum, 32);
  lsum_mfma += __shfl_xor(lsum_mfma, 32);
  const int G = a.G;
  const int hd = kHeadsPerGroup * hg + col;   // head inside the group
  float* out_o;
  float* out_l;
  if (nsplit == 1) {
    out_o = a.o_part + (((int64_t)r * a.Btot + b) * a.Hq + g * G + hd) * kDv;
    out_l = a.lse_part + ((int64_t)r * a.Btot + b) * a.Hq + g * G + hd;
  } else {
    out_o = a.ws_o + ((int64_t)wg * G + hd) * kDv;
    out_l = a.ws_lse + (int64_t)wg * G + hd;
  }
  const float inv = lsum_mfma > 0.f ? 1.0f / lsum_mfma : 0.f;
#pragma unroll
  for (int nb = 0; nb < kHalfVBlocks; ++nb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v = make_float4(acc[nb][4 * q4] * inv, acc[nb][4 * q4 + 1] * inv, acc[nb][4 * q4 + 2] * inv,
                                   acc[nb][4 * q4 + 3] * inv);
      *reinterpret_cast<float4*>(out_o + 32 * (kHalfVBlocks * dh + nb) + 8 * q4 + 4 * half) = v;
    }
  }
  if (half == 0 && dh == 0) *out_l = lsum > 0.f ? (mrun + __log2f(lsum)) * kLn2 : -INFINITY;
#endif
}

}  // namespace

hipError_t launch_mla_partial(const PartialArgs& a, hipStream_t st) {
  const int nwg = a.wg_begin[a.nb];
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_partial_kernel, dim3(nwg), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace hx
