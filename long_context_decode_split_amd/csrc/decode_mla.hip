// Split-KV decode attention for MLA caches on gfx950: one latent KV head of
// 576 columns whose first 512 columns are also the value row, 128 query heads
// per latent head (the DeepSeek-R1 shape of the Helix review, Prompt 1.4.1;
// the Helix summary notes MLA effectively has one KV head).
//
// Both products are dense (128 heads share every latent row) and run on
// v_mfma_f32_32x32x16_bf16:
//   S^T[32 tokens][32 heads] = K[32 tokens][576] . Q^T[576][32 heads]
//   O^T[512][32 heads]      += V^T[512][32 tokens] . P^T[32 tokens][32 heads]
//
// A workgroup of four waves (one per SIMD, 512 registers each) streams a run
// of 32-token tiles of one slice.  Wave w owns heads 32 w .. 32 w + 31: their
// Q^T fragments for all 576 columns stay in VGPRs (144 registers), their
// O^T accumulator for all 512 value columns in AGPRs (256 registers), so a
// wave needs nothing from the other waves but the shared tile: no partial
// sums are exchanged and every score is computed once.  The softmax keeps
// the first tile's max as its reference, so the accumulator never needs
// rescaling (a score more than 2^kHeadroom above it restarts the run).
// P enters the value product as a bf16 high part plus the bf16 of its
// rounding residual (SPLITP, the default): rounded once, P's 8 significant
// bits put the output's error at up to 2^-8 times half the range of V, which
// for short slices reaches the 2e-3 bound of bf16 caches; the residual's
// products double the value product's matrix-core work.  They are what
// keeps heavy weights exact, so a wave skips them on a tile where every
// weight of its heads is at most 2^-HX_MLA_RES_LOG2 of that head's running
// sum (each weight then is at most that fraction of the final sum, and the
// rounding errors of many such small weights average out instead of adding
// up); the first tiles of a run, tiles with needles and short slices keep
// them.  Measured at 2^20 tokens: 2^-12 / 2^-10 / 2^-8 / always skipping
// took 2,845 / 2,635 / 2,585 / 2,600 us, every output within 4e-6 of the
// oracle (the residual everywhere: 3,112 us).
//
// A tile (two chunk tiles, 36 KiB) is copied from HBM into LDS unchanged with
// direct global-to-LDS loads (no VGPRs), into one of four buffers: three
// tiles are in flight while one is used, and one barrier per tile both
// publishes a tile and frees the buffer for the copy three tiles ahead.  The
// cache stores each latent row with its 16-byte pieces XOR-swizzled inside
// aligned groups of 8, so the unchanged copy is read efficiently both as
// 16-byte rows (score operand) and through ds_read_b64_tr_b16 (transposed
// value operand), and one stored copy of the latent row serves both.
//
// fp8 and MXFP4 latent rows (one plane of packed chunk tiles: 16 rows of
// codes, row-major, then the group's fp32 scale resp. the rows' e8m0 bytes)
// are copied unchanged into a two-buffer LDS staging ring and converted by
// all threads into the bf16 tile layout above (rows past the slice end as
// zeros), so the products below run as for bf16 rows; three bf16 tile
// buffers then fit next to the staging ring.  One copy is in flight while
// the workgroup converts the tile after next and computes the current one.
// Their P is rounded once (as for the quantised GQA caches).
//
// Lane layouts used below (64-lane wave, l = lane, half = l / 32):
//   32x32x16 A operand: row l % 32, k = 8 * half + j (j = 0..7);
//   B operand: column l % 32, same k; C/D: register r holds row
//   8 * (r / 4) + 4 * half + r % 4, column l % 32.
//   ds_read_b64_tr_b16, per group of 16 lanes: lane i receives element i % 4
//   of the 4-element reads of lanes i / 4 + 4 k, k = 0..3.

#include <type_traits>

#include "hx_append.h"
#include "hx_gqa_frag.h"

namespace hx {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerWave = 32;
constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kTileTok = 32;                       // tokens per LDS tile (two chunk tiles)
constexpr int kRowBytes = kDk * 2;                 // 1152
constexpr int kTileBytes = kTileTok * kRowBytes;   // 36 KiB
constexpr int kBlocksPerWave = kTileBytes / 1024 / kWaves;   // 1 KiB copies per wave per tile (9)
constexpr int kNBuf = 4;                           // tile buffers (bf16 rows)
// Quantised latent rows: packed chunk tiles of kQChunk bytes (codes, then
// scales), staged two 32-row tiles at a time, copied in 16-byte pieces of
// which each wave takes a quarter (kQCopies copy instructions per wave).
template <int FMT>
constexpr int kQChunk = FMT == 1 ? 16 * 576 + 16 : 16 * 288 + 16 * 18;   // 9,232 / 4,896 bytes
template <int FMT>
constexpr int kQCodes = FMT == 1 ? 16 * 576 : 16 * 288;                  // code bytes of a chunk tile
template <int FMT>
constexpr int kQPieces = kQChunk<FMT> / 16;                              // 577 / 306
template <int FMT>
constexpr int kQCopies = ((2 * kQPieces<FMT> + 3) / 4 + 63) / 64;        // 5 / 3
constexpr int kQBuf = 3;                                                 // bf16 tile buffers next to the staging
constexpr int kSteps = kDk / 16;                   // k-steps of the score product (36)
constexpr int kVBlocks = kDv / 32;                 // 32-column value blocks (16)
constexpr int kKPre = 4;                           // score operands read ahead
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kHeadroom = 64.0f;                 // log2 of the largest unnormalised P
#ifndef HX_MLA_RES_LOG2
#define HX_MLA_RES_LOG2 10
#endif
// a tile's residual products are skipped when each weight is at most
// 2^-HX_MLA_RES_LOG2 of its head's running sum
constexpr float pow2i(int e) { return e == 0 ? 1.0f : (e > 0 ? 2.0f * pow2i(e - 1) : 0.5f * pow2i(e + 1)); }
constexpr float kResFrac = pow2i(-HX_MLA_RES_LOG2);

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint4 lds_u4;

constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// One direct global-to-LDS load of 16 bytes per lane: lane l's bytes from
// sbase + voff land at LDS byte lds + 16 l (M0 holds the wave-uniform LDS
// base), with the non-temporal policy since every row is read once
// (measured 1.2% faster than the default).  Issued from inline assembly so
// the compiler does not treat the address registers as pending load results
// (it would otherwise wait for the tile loads before every reuse of those
// registers).  Completion is awaited with explicit vmcnt waits before the
// barrier that publishes a tile.  M0 is an input operand of the asm (the
// "{m0}" constraint), so the compiler itself sets it and knows it is used.
// The compiler cannot see the load inside the asm, so the asm carries the
// wait states it needs: five after a VALU write of an SGPR the load reads
// (the readfirstlanes of the base address; the compiler pads the same
// sequence with s_nop 4 when it emits the load itself), which also covers
// the one wait state after the M0 write.
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  const uint64_t sb = (uint64_t)sbase;
  const uint64_t sbu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbu),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// The same copy from a per-lane 64-bit address (lanes may read from two
// different chunk tiles); inactive lanes copy nothing.
__device__ __forceinline__ void dma16a(const void* g, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Workgroup barrier after this wave's loads down to VMCNT still in flight
// have landed and all its LDS accesses are done.  The asm is also a compiler
// memory barrier, so no LDS access moves across it.
template <int VMCNT>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VMCNT) : "memory");
}

// Score-product step with the accumulator in VGPRs (the AGPRs hold the value
// accumulator).  Back-to-back steps on the same accumulator need no wait
// states; the first VALU read of the result needs more than 18, which the
// caller provides.
__device__ __forceinline__ f32x16 mfma_s(bf16x8 a, bf16x8 b, f32x16 c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  return c;
}
__device__ __forceinline__ f32x16 mfma_s0(bf16x8 a, bf16x8 b) {
  f32x16 c;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  return c;
}

// The lane index, opaque to the optimiser: addresses derived from it inside
// the tile loop are recomputed there (a few integer ops) instead of being
// hoisted out and kept live in VGPRs across the loop.
__device__ __forceinline__ int opaque_lane() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

// The same for the thread index.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

template <bool PAGED, bool SPLITP, bool FUSED, int FMT>
__global__ __launch_bounds__(kThreads, 1) void mla_partial_kernel(const PartialArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // device-only builtins (LDS address space) below
  constexpr int kNB = FMT == 0 ? kNBuf : kQBuf;
  __shared__ __attribute__((aligned(1024))) uint8_t s_tile[kNB][kTileBytes];
  // quantised rows: the staging ring (two 32-row tiles as stored); fp8: the
  // group scales of the tile in each bf16 buffer (rows 0-15, 16-31)
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[FMT == 0 ? 1 : 2][FMT == 0 ? 16 : 2 * kQChunk<FMT>];
  __shared__ float s_qscale[kNB][2];
  // 1 when a wave saw a score beyond its headroom; two sets, by the parity of
  // the iteration, so that a wave writing the next flag cannot overtake a
  // slower wave still reading the current ones
  __shared__ uint32_t s_over[2][kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = PAGED ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- which (request, latent head, slice, split) this workgroup owns
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
  const int64_t t_begin = (int64_t)split * a.cpw_b[bl] * kChunk;   // cpw_b is even: tiles start on 32 rows
  const int64_t t_end = min((int64_t)(split + 1) * a.cpw_b[bl] * kChunk, L);
  const int ntok = t_end > t_begin ? (int)(t_end - t_begin) : 0;
  const int ntiles = (ntok + kTileTok - 1) / kTileTok;

  // Dense cache: the slice's rows are consecutive (latent rows, 1152 B
  // each).  Block pool: 16-row group c of the slice is the tile of head g in
  // block trow[c] (tile_of in hx_common.h), so a 32-row tile is two tiles.
  const int64_t tile0 = PAGED ? 0 : ((int64_t)(r * a.Btot + b) * a.Hkv + g) * a.cap_chunks;
  const uint8_t* base = a.k + tile0 * a.k_tile + t_begin * kRowBytes;
  const int32_t* trow = PAGED ? a.table + ((int64_t)b * a.P + r) * a.cap_chunks : nullptr;
  const int64_t cbeg = t_begin / kChunk;   // first 16-row group of the split
  if constexpr (FUSED) fused_append(a.app, bl, g, r, cbeg, cbeg + (ntok + kChunk - 1) / kChunk);

  // ---- Q^T fragments of head 32 wave + col (B operand: step s covers
  //      columns 16 s + 8 half .. +7)
  bf16x8 qf[kSteps];
  {
    const int head = g * a.G + kHeadsPerWave * wave + col;
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + head) * kDk + 8 * half;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 16 * s));
  }
  // Q is in place before any tile load is issued, so no wait the compiler
  // derives for Q can later count the tile loads.
  __builtin_amdgcn_s_waitcnt(0);

  // ---- direct global -> LDS copy of tile k into buffer k % 4: 1 KiB blocks
  //      w, w + 4, ..., w + 32; lane l moves bytes 16 l .. +15 of each.  Rows
  //      past the slice end (last tile only) are fetched from row 0 of the
  //      tile instead: finite values that the masked scores give weight 0.
  //      Block pool: the two 16-row halves come from their own blocks
  //      (src0, src1, looked up by prep(k) before the copy); a row past the
  //      slice end is fetched from row 0 of its half, or of the first half
  //      when the second holds no row of the slice (then src1 = src0).
  const uint8_t* src0 = nullptr;   // the two halves of the next tile to copy
  const uint8_t* src1 = nullptr;
  auto prep = [&](int k) {
    if constexpr (PAGED) {
      const int valid = min(kTileTok, ntok - k * kTileTok);
      const int64_t c = cbeg + 2 * k;
      src0 = a.k + (clamp_block(trow[c], a.num_blocks) * a.Hkv + g) * a.k_tile;
      src1 = valid > kChunk ? a.k + (clamp_block(trow[c + 1], a.num_blocks) * a.Hkv + g) * a.k_tile : src0;
    }
  };
  auto load_tile = [&](int k) {
    const int valid = min(kTileTok, ntok - k * kTileTok);
    uint8_t* dst = &s_tile[k % kNBuf][0];
    if constexpr (PAGED) {
      constexpr int kHalfBlocks = kChunk * kRowBytes / 1024;   // 1 KiB blocks per 16-row half
#pragma unroll
      for (int j = 0; j < kBlocksPerWave; ++j) {
        const int blk = wave + kWaves * j;
        const bool upper = blk >= kHalfBlocks;
        uint32_t off = (blk - (upper ? kHalfBlocks : 0)) * 1024u + 16u * opaque_lane();   // byte of the half
        if (valid < kTileTok && (int)(off / kRowBytes) + (upper ? kChunk : 0) >= valid) off %= kRowBytes;
        dma16(off, upper ? src1 : src0, lds_addr(dst + blk * 1024));
      }
    } else {
      const uint8_t* src = base + (int64_t)k * kTileBytes;
#pragma unroll
      for (int j = 0; j < kBlocksPerWave; ++j) {
        const int blk = wave + kWaves * j;
        uint32_t off = blk * 1024u + 16u * opaque_lane();   // byte of the tile this lane moves
        if (valid < kTileTok && off / kRowBytes >= (uint32_t)valid) off %= kRowBytes;
        dma16(off, src, lds_addr(dst + blk * 1024));
      }
    }
  };

  const uint8_t* qbase = a.k + (tile0 + cbeg) * a.k_tile;   // dense quantised rows: the split's first chunk tile
  // ---- quantised rows: copy of tile k's two packed chunk tiles, as stored,
  //      into staging buffer k % 2.  The 16-byte pieces of the pair are
  //      numbered chunk 0 first; wave w copies pieces [2 N w / 4, 2 N (w+1)
  //      / 4) (N pieces per chunk tile), kQCopies instructions of up to 64
  //      consecutive pieces each, so every wave issues the same number.  A
  //      pair whose second chunk holds no row of the slice copies its first
  //      chunk twice (the conversion zeroes those rows).
  auto stage = [&](int k) {
    if constexpr (FMT != 0) {
      constexpr int N = kQPieces<FMT>;
      const int valid = min(kTileTok, ntok - k * kTileTok);
      const uint8_t* c0p;
      const uint8_t* c1p;
      if constexpr (PAGED) {
        c0p = src0;
        c1p = src1;
      } else {
        c0p = qbase + (int64_t)(2 * k) * a.k_tile;
        c1p = valid > kChunk ? c0p + a.k_tile : c0p;
      }
      uint8_t* dst = &s_stage[k & 1][0];
      // the wave index as a scalar, so the piece range and the LDS
      // destinations are scalar values too (as vector values they were
      // spilled to scratch and reloaded behind a wait for every load)
      const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      const int pbeg = 2 * N * wv / kWaves, pend = 2 * N * (wv + 1) / kWaves;
      // dense cache: both chunk tiles within 4 GiB of the first, so one
      // scalar base and 32-bit lane offsets (recomputed here from the lane,
      // not kept live across the loop as per-lane 64-bit addresses)
      const uint32_t gap = (uint32_t)(c1p - c0p) - 16u * N;   // the second chunk's offset past piece N
#pragma unroll
      for (int i = 0; i < kQCopies<FMT>; ++i) {
        const int first = pbeg + 64 * i;
        const int pc = first + (PAGED ? lane : opaque_lane());
        if (pc < pend) {
          if constexpr (PAGED) dma16a(pc < N ? c0p + 16 * pc : c1p + 16 * (pc - N), lds_addr(dst + 16 * first));
          else dma16(16u * pc + (pc < N ? 0u : gap), c0p, lds_addr(dst + 16 * first));
        }
      }
    }
  };
  // ---- quantised rows: staging buffer of tile k -> bf16 buffer k % kNB in
  //      the bf16 tile layout (row m's 16-byte piece q at piece position
  //      q ^ mla_swz(m)); rows at or past the slice end become zeros.  fp8:
  //      the codes (e4m3 values are bf16 values), the two group scales kept
  //      in s_qscale for the softmax, which folds them into the scores and
  //      into P; MXFP4: e2m1 x 2^(E-127), exact in bf16.  Each thread
  //      converts 9 of the tile's 32 x 72 pieces of 8 elements.
  //      The work is split into reads and conversions of three pieces at a
  //      time (cvt_load, cvt_store) so that it can run as one phase (all
  //      reads first: the LDS round trips overlap) or between the products.
  struct CvtAt {
    const lds_u8* src;    // the thread's first code piece in the staging buffer
    const lds_u8* esrc;   // MXFP4: its first e8m0 byte
    lds_u8* dst;          // its first piece in the bf16 buffer
    bool live;            // the thread's row holds a token of the slice
  };
  auto cvt_at = [&](int k) {
    // Thread t converts row t / 8, pieces q0 + 8 j (q0 = t % 8, j = 0 .. 8):
    // the row, its swizzle and its chunk are the thread's own, so a piece's
    // source and destination are the thread's bases plus 8 j pieces (the
    // swizzle permutes within groups of 8, so piece q0 + 8 j lands at
    // (q0 ^ swizzle) + 8 j).  A wave's eight rows and eight pieces per row
    // read 64 different LDS banks (MXFP4) or two rows per bank group (fp8).
    constexpr int kCodeRow = FMT == 1 ? kDk : kDk / 2;   // code bytes per row
    const lds_u8* st = (const lds_u8*)&s_stage[k & 1][0];
    const int t = opaque_tid();
    const int m = t >> 3, q0 = t & 7;
    CvtAt c;
    c.src = st + (m >> 4) * kQChunk<FMT> + (m & 15) * kCodeRow + (FMT == 1 ? 8 : 4) * q0;
    c.esrc = st + (m >> 4) * kQChunk<FMT> + kQCodes<FMT> + (m & 15) * (kDk / 32) + (q0 >> 2);
    c.dst = (lds_u8*)&s_tile[k % kNB][0] + m * kRowBytes + 16 * (q0 ^ mla_swz(m));
    c.live = m < min(kTileTok, ntok - k * kTileTok);
    return c;
  };
  struct CvtRegs {
    uint32_t q[3][FMT == 1 ? 2 : 1];   // codes of three pieces
    uint32_t e[3];                     // MXFP4: their e8m0 bytes
  };
  auto cvt_load = [&](const CvtAt& c, int j0, CvtRegs& r) {   // reads of pieces j0 .. j0 + 2 (in the staging buffer either way)
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if constexpr (FMT == 1) {
        const uint2 c8 = *(const __attribute__((address_space(3))) uint2*)(c.src + 64 * (j0 + i));
        r.q[i][0] = c8.x;
        r.q[i][1] = c8.y;
      } else if constexpr (FMT == 2) {
        r.q[i][0] = *(const __attribute__((address_space(3))) uint32_t*)(c.src + 32 * (j0 + i));
        r.e[i] = c.esrc[2 * (j0 + i)];
      }
    }
  };
  auto cvt_store = [&](const CvtAt& c, int j0, const CvtRegs& r) {   // conversions and stores of pieces j0 .. j0 + 2
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      uint4 out = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (FMT == 1) {
        out = make_uint4(frag::fp8x2_to_bf16x2<false>(r.q[i][0]), frag::fp8x2_to_bf16x2<true>(r.q[i][0]),
                         frag::fp8x2_to_bf16x2<false>(r.q[i][1]), frag::fp8x2_to_bf16x2<true>(r.q[i][1]));
      } else if constexpr (FMT == 2) {
        const float sc = __uint_as_float(r.e[i] << 23);   // 2^(E-127); E = 0 reads as 0, E = 255 as +inf
        out = make_uint4(frag::fp4x2_to_bf16x2<0>(r.q[i][0], sc), frag::fp4x2_to_bf16x2<1>(r.q[i][0], sc),
                         frag::fp4x2_to_bf16x2<2>(r.q[i][0], sc), frag::fp4x2_to_bf16x2<3>(r.q[i][0], sc));
      }
      if (!c.live) out = make_uint4(0u, 0u, 0u, 0u);   // rows past the slice end: zeros
      *(lds_u4*)(c.dst + 128 * (j0 + i)) = out;
    }
  };
  // fp8: the two group scales of tile k for the softmax (a group with no row
  // of the slice: scale 1, its rows being zeros)
  auto cvt_scales = [&](int k) {
    if constexpr (FMT == 1) {
      const lds_u8* st = (const lds_u8*)&s_stage[k & 1][0];
      const int valid = min(kTileTok, ntok - k * kTileTok);
      const int t = opaque_tid();
      if (t < 2)
        s_qscale[k % kNB][t] =
            16 * t < valid ? *(const __attribute__((address_space(3))) float*)(st + t * kQChunk<FMT> + kQCodes<FMT>)
                           : 1.0f;
    }
  };
  // the whole conversion of tile k as one phase: all nine reads, then the
  // conversions (one piece at a time waited for nine round trips in a row)
  auto convert = [&](int k) {
    if constexpr (FMT != 0) {
      const CvtAt c = cvt_at(k);
      CvtRegs r[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) cvt_load(c, 3 * j, r[j]);
#pragma unroll
      for (int j = 0; j < 3; ++j) cvt_store(c, 3 * j, r[j]);
      cvt_scales(k);
    }
  };

  f32x16 acc[kVBlocks];
#pragma unroll
  for (int i = 0; i < kVBlocks; ++i) acc[i] = f32x16{};
  float mref = -INFINITY;   // reference max of head 32 wave + col (base 2)
  float lsum = 0.f;         // sum of P over this lane's tokens (exact)
  float lsum_mfma = 0.f;    // the same over the bf16-rounded P
  const float c2 = a.c2;

  // Score view: row col, piece 2 s + half, swizzled by the row; steps s and
  // s + 4 differ by 8 pieces (128 B): four bases plus immediate offsets.
  int k_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int pc = 2 * s + half;
    k_off[s] = kRowBytes * col + 16 * ((pc & ~7) | ((pc & 7) ^ mla_swz(col)));
  }
  // Value view for ds_read_b64_tr_b16: lane i16 of its 16-lane group reads
  // row 16 u + 4 half + i16 / 4 (+ 8 for the second half of the k-step),
  // columns 32 nb + 16 cb + 4 (i16 % 4) .. +3, i.e. piece
  // 4 nb + 2 cb + (i16 % 4) / 2.  nb and nb + 2 differ by 8 pieces; rows r
  // and r + 16 share the swizzle: two bases for each of the two row halves.
  const int i16 = lane & 15;
  const int cb = (lane >> 4) & 1;
  int v_off[2][2];   // [row half][nb & 1]
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int vrow = 4 * half + (i16 >> 2) + 8 * hh;
    const int swv = mla_swz(vrow);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int pc = 4 * e + 2 * cb + ((i16 & 3) >> 1);
      v_off[hh][e] = kRowBytes * vrow + 16 * ((pc & ~7) | ((pc & 7) ^ swv)) + 8 * (i16 & 1);
    }
  }

  // ---- the two products of a tile, as steps that can be interleaved
  auto kread = [&](const lds_u8* tb, int s) { return *(const lds_u4*)(tb + k_off[s & 3] + 128 * (s >> 2)); };
  auto vread = [&](const lds_u8* tb, int i) {   // i = 16 u + nb
    const int nb = i & 15;
    const int rel = 128 * (nb >> 1) + kRowBytes * 16 * (i >> 4);
    const uint2 lo =
        __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tb + v_off[0][nb & 1] + rel)));
    const uint2 hi =
        __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tb + v_off[1][nb & 1] + rel)));
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };

  // ---- online softmax (base 2) of one tile's scores against a fixed
  //      reference max per head: the first tile's max.  P = 2^(s - mref) is
  //      then not bounded by 1 but by 2^kHeadroom as long as no later score
  //      exceeds the reference by more than kHeadroom; bf16 P and the fp32
  //      sums hold such values exactly as well as values below 1.  A score
  //      beyond that (seen by any wave) restarts the run with the larger
  //      reference, so the accumulator never needs rescaling.  The result is
  //      unchanged: O and the sums share the reference, and
  //      LSE = mref + log2(sum).  P goes out as bf16 pairs in pk.
  uint32_t pk[8];
  uint32_t pr[8];   // SPLITP: bf16 of the rounding residuals of P, same layout
  float mseen = -INFINITY;   // largest scaled score seen in this run (base 2)
  bool res = false;          // SPLITP: the tile softmax last ran on needs the residual products (wave-uniform)
  auto softmax = [&](f32x16 sc, int k) {
    const int valid = min(kTileTok, ntok - k * kTileTok);
    // fp8 rows: the group scale of rows 0-15 (registers 0-7) and 16-31 (8-15)
    float gs[2] = {1.0f, 1.0f};
    if constexpr (FMT == 1) {
      gs[0] = s_qscale[k % kNB][0];
      gs[1] = s_qscale[k % kNB][1];
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] *= gs[i >> 3];
    }
    if (valid < kTileTok) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * half + (i & 3) >= valid) sc[i] = -INFINITY;
    }
    float cm = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) cm = fmaxf(cm, sc[i]);
    cm = max_xor32(cm) * c2;
    mseen = fmaxf(mseen, cm);
    if (mref == -INFINITY) mref = cm;   // first tile of the run (at least one valid token)
    float p[16];
    float psg[2] = {0.f, 0.f}, pm = 0.f;   // sums of P over rows 0-15 and 16-31
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c2, -mref));
      psg[i >> 3] += p[i];
      pm = fmaxf(pm, p[i]);
    }
    lsum += psg[0] + psg[1];
    // the lane's running sum covers half of its head's tokens so far, so the
    // two lanes' sum bounds the head's final sum from below
    if constexpr (SPLITP) res = __any(pm > kResFrac * sum_xor32(lsum));
    if constexpr (FMT == 1) {
      // fp8 rows: each group's scale folded into its weights, the rounded
      // products divided by it normalise O (a zero scale: the weights
      // unrounded, the values being 0)
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        float rs = 0.f;
#pragma unroll
        for (int i = 4 * grp; i < 4 * grp + 4; ++i) {
          const bf16x2 pb2 = {(__bf16)(p[2 * i] * gs[grp]), (__bf16)(p[2 * i + 1] * gs[grp])};
          pk[i] = __builtin_bit_cast(uint32_t, pb2);
          rs = __builtin_amdgcn_fdot2_f32_bf16(pb2, kOnes2, rs, false);
        }
        // (the hardware reciprocal: a normalising sum needs no correctly
        // rounded quotient)
        lsum_mfma += gs[grp] != 0.f ? rs * __builtin_amdgcn_rcpf(gs[grp]) : psg[grp];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x2 pb2 = {(__bf16)p[2 * i], (__bf16)p[2 * i + 1]};
        pk[i] = __builtin_bit_cast(uint32_t, pb2);
        // the rounded values the matrix product uses, summed for the normalisation
        lsum_mfma = __builtin_amdgcn_fdot2_f32_bf16(pb2, kOnes2, lsum_mfma, false);
      }
    }
    if (SPLITP && res) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r0 = p[2 * i] - __uint_as_float(pk[i] << 16);
        const float r1 = p[2 * i + 1] - __uint_as_float(pk[i] & 0xffff0000u);
        const bf16x2 rb2 = {(__bf16)r0, (__bf16)r1};
        pr[i] = __builtin_bit_cast(uint32_t, rb2);
        lsum_mfma = __builtin_amdgcn_fdot2_f32_bf16(rb2, kOnes2, lsum_mfma, false);
      }
    }
  };

  // ---- tiles, software-pipelined: iteration k accumulates tile k's values
  //      (O^T += V^T P^T, 32 products into 16 independent accumulators)
  //      interleaved with tile k + 1's scores (S^T = K Q^T, a chain of 36),
  //      then runs tile k + 1's softmax; iteration -1 only scores tile 0.
  //      Tiles 0-2 are copied up front and tile k + 3 into the buffer of
  //      tile k - 1 once every wave is past it (the barrier).  Loads
  //      complete in issue order, so tile k + 1 has landed once only tile
  //      k + 2's copy may still be pending.  Each barrier also publishes
  //      every wave's overflow flag for the tile scored before it.
  // One iteration: wait for tile k + 1 and publish the overflow flags, then
  // the interleaved products.  CUR: tile k's values exist (k >= 0); NEXT:
  // tile k + 1 exists.  Returns true when some wave asks for a restart.
  auto iteration = [&](auto cur_t, auto next_t, int k) -> bool {
    constexpr bool CUR = decltype(cur_t)::value;
    constexpr bool NEXT = decltype(next_t)::value;
    const bool res_k = SPLITP && CUR && res;   // tile k's softmax asked for the residual products
    const int par = k & 1;
    const bool over = __any(mseen > mref + kHeadroom);   // all lanes vote, outside the lane-0 branch
    if (lane == 0) s_over[par][wave] = over ? 1u : 0u;
    if constexpr (FMT == 0) {
      if (CUR && k + 3 < ntiles) prep(k + 3);   // pool lookups complete in the barrier's wait
      if (k + 2 < ntiles) wait_barrier<kBlocksPerWave>();
      else wait_barrier<0>();
    } else {
      // quantised rows: the barrier publishes tile k + 1's conversion and
      // tile k + 2's staging copy (the only copy in flight)
      if (k + 3 < ntiles) prep(k + 3);
      wait_barrier<0>();
    }
    // a restart asked for by some wave.  Quantised rows act on it at the end
    // of the iteration (its work is then discarded), so the flags' LDS round
    // trip does not hold up the iteration (the copy issued below lands before
    // the restart's first barrier; a wave reads these flags before the
    // barrier of the next iteration, and the next write to them is two
    // barriers on): MXFP4 rows 2,236-2,258 -> 2,188-2,198 us on one box; bf16
    // rows, bound by the board's power, measured no gain and return at once.
    const bool stop = (s_over[par][0] | s_over[par][1] | s_over[par][2] | s_over[par][3]) != 0;
    if (FMT == 0 && stop) return true;
    if constexpr (FMT == 0) {
      if (CUR && k + 3 < ntiles) load_tile(k + 3);
    } else {
      if (k + 3 < ntiles) stage(k + 3);    // into the staging buffer tile k + 1 left
      cvt_scales(k + 2);
    }
    // quantised rows: tile k + 2 is converted into the bf16 buffer tile k - 1
    // left in three parts between the products below (past the last tile it
    // converts zeros into a buffer no tile uses any more)
    CvtAt cv;
    CvtRegs cr;
    if constexpr (FMT != 0) cv = cvt_at(k + 2);
    const lds_u8* tv = (const lds_u8*)&s_tile[(k + kNB) % kNB][0];
    const lds_u8* tk = (const lds_u8*)&s_tile[(k + 1) % kNB][0];
    f32x16 sc;
    uint4 kv[kKPre + 1];
    uint4 vv[3];
    if (NEXT) {
#pragma unroll
      for (int s = 0; s < kKPre; ++s) kv[s] = kread(tk, s);
    }
    if (CUR) {
      vv[0] = vread(tv, 0);
      vv[1] = vread(tv, 1);
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if constexpr (FMT != 0) {
        if (s % 12 == 0) cvt_load(cv, s / 4, cr);
        if (s % 12 == 4) cvt_store(cv, (s - 4) / 4, cr);
      }
      if (CUR && s < 2 * kVBlocks) {
        if (s + 2 < 2 * kVBlocks) vv[(s + 2) % 3] = vread(tv, s + 2);
        const int u = s >> 4;
        const bf16x8 pb =
            __builtin_bit_cast(bf16x8, make_uint4(pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]));
        acc[s & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv[s % 3]), pb, acc[s & 15],
                                                              0, 0, 0);
      }
      if (NEXT) {
        if (s + kKPre < kSteps) kv[(s + kKPre) % (kKPre + 1)] = kread(tk, s + kKPre);
        sc = s == 0 ? mfma_s0(__builtin_bit_cast(bf16x8, kv[0]), qf[0])
                    : mfma_s(__builtin_bit_cast(bf16x8, kv[s % (kKPre + 1)]), qf[s], sc);
      }
    }
    if (res_k) {   // tile k's residual products (uniform branch), its value fragments read again
      uint4 vr[3];
      vr[0] = vread(tv, 0);
      vr[1] = vread(tv, 1);
#pragma unroll
      for (int i = 0; i < 2 * kVBlocks; ++i) {
        if (i + 2 < 2 * kVBlocks) vr[(i + 2) % 3] = vread(tv, i + 2);
        const int u = i >> 4;
        const bf16x8 pl =
            __builtin_bit_cast(bf16x8, make_uint4(pr[4 * u], pr[4 * u + 1], pr[4 * u + 2], pr[4 * u + 3]));
        acc[i & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vr[i % 3]), pl, acc[i & 15],
                                                              0, 0, 0);
      }
    }
    if (NEXT) {
      // the last score step has drained; sc is an operand, so the compiler
      // schedules no read of it before these wait states
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sc));
      softmax(sc, k + 1);
    }
    return stop;
  };
  typedef std::integral_constant<bool, true> T;
  typedef std::integral_constant<bool, false> F;

  for (;;) {
    if constexpr (FMT == 0) {
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < ntiles) {
          prep(j);
          load_tile(j);
        }
    } else {
      // stage tiles 0 and 1, convert tile 0 once its copy has landed
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (j < ntiles) {
          prep(j);
          stage(j);
        }
      if (ntiles > 1) wait_barrier<kQCopies<FMT>>();
      else wait_barrier<0>();
      if (ntiles > 0) convert(0);
    }
    bool restart = ntiles > 0 && iteration(F{}, T{}, -1);
    for (int k = 0; !restart && k + 1 < ntiles; ++k) restart = iteration(T{}, T{}, k);
    if (!restart && ntiles > 0) restart = iteration(T{}, F{}, ntiles - 1);
    if (!restart) break;
    // a score outgrew the reference: every wave starts over from the first
    // tile with its largest score so far as the reference (rare: needs a
    // jump of 2^kHeadroom over the run's first tile)
    wait_barrier<0>();   // no copy is still writing a buffer; every wave has read the flags
#pragma unroll
    for (int i = 0; i < kVBlocks; ++i) acc[i] = f32x16{};
    lsum = 0.f;
    lsum_mfma = 0.f;
    mref = mseen;
  }

  // ---- finalize: head 32 wave + col, all 512 value columns
  lsum = sum_xor32(lsum);
  lsum_mfma = sum_xor32(lsum_mfma);
  const int G = a.G;
  const int hd = kHeadsPerWave * wave + col;   // head inside the group
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
  for (int nb = 0; nb < kVBlocks; ++nb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v = make_float4(acc[nb][4 * q4] * inv, acc[nb][4 * q4 + 1] * inv, acc[nb][4 * q4 + 2] * inv,
                                   acc[nb][4 * q4 + 3] * inv);
      *reinterpret_cast<float4*>(out_o + 32 * nb + 8 * q4 + 4 * half) = v;
    }
  }
  if (half == 0) *out_l = lsum > 0.f ? (mref + __log2f(lsum)) * kLn2 : -INFINITY;
#endif
}

}  // namespace

hipError_t launch_mla_partial(const PartialArgs& a, int dtype, hipStream_t st) {
  const int nwg = a.wg_begin[a.nb];
  if (nwg == 0) return hipSuccess;
  const dim3 grid(nwg), block(kThreads);
  if (dtype != HX_KV_BF16) {
    // quantised rows: P rounded once, the step's rows appended beforehand
    if (a.fused_append) return hipErrorInvalidValue;
    const bool paged = a.table != nullptr;
    if (dtype == HX_KV_FP8_E4M3) {
      if (paged) hipLaunchKernelGGL((mla_partial_kernel<true, false, false, 1>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((mla_partial_kernel<false, false, false, 1>), grid, block, 0, st, a);
    } else {
      if (paged) hipLaunchKernelGGL((mla_partial_kernel<true, false, false, 2>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((mla_partial_kernel<false, false, false, 2>), grid, block, 0, st, a);
    }
    return hipGetLastError();
  }
  const int v = (a.table ? 4 : 0) | (a.split_p ? 2 : 0) | (a.fused_append == 1 ? 1 : 0);
  switch (v) {
    case 0: hipLaunchKernelGGL((mla_partial_kernel<false, false, false, 0>), grid, block, 0, st, a); break;
    case 1: hipLaunchKernelGGL((mla_partial_kernel<false, false, true, 0>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((mla_partial_kernel<false, true, false, 0>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((mla_partial_kernel<false, true, true, 0>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((mla_partial_kernel<true, false, false, 0>), grid, block, 0, st, a); break;
    case 5: hipLaunchKernelGGL((mla_partial_kernel<true, false, true, 0>), grid, block, 0, st, a); break;
    case 6: hipLaunchKernelGGL((mla_partial_kernel<true, true, false, 0>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((mla_partial_kernel<true, true, true, 0>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace hx
