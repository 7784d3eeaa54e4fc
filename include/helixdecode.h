/*
 * helixdecode — KV-parallel (sequence-split) decode attention for one
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (the method's data-parallel hot path):
 *   "Helix Parallelism: Rethinking Sharding Strategies for Interactive
 *   Multi-Million-Token LLM Decoding" (fdeinterviews.com summary), paragraph
 *   on KV parallelism: the request's KV history is split along the sequence;
 *   every slice attends over its part and returns a partial output and a
 *   log-sum-exp; one exchange then combines the partials into the exact
 *   attention output.  Same page, paragraph on Helix's two layouts: new KV
 *   entries rotate across the slices every 16 tokens.  jaehun.me review,
 *   Prompt 1.3.2 "The Secret Weapon": the combine is
 *   O = sum_i O_i exp(LSE_i) / sum_i exp(LSE_i), exact.
 *
 * On one GPU every KV-parallel rank becomes one slice of an HBM-resident
 * cache, and the exchange becomes an in-HBM combine (hx_lse_combine).
 *
 * Short page names used in the citations of this library's sources:
 * "Helix summary" is the fdeinterviews.com page named above; "jaehun.me
 * review" the jaehun.me paper review of the same work (sections numbered
 * Prompt 1.1.1 ... 1.5.2 as on that page); "NVIDIA blog" the open-lab.net
 * NVIDIA technical blog post (Korean) on multi-million-token real-time
 * inference; "ifai.io article" the ifai.io news article on NVIDIA's Helix.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Every function returns an hx_status; HX_OK is 0.  Arguments are checked
 *    on the host before anything is launched; on error nothing is launched
 *    and hx_last_error() returns a message (thread-local, valid until the
 *    next call on the same thread).  Nothing throws across the ABI.
 *  - Pointers named "device" are device memory owned by the caller; the
 *    library never allocates, frees or keeps them.  Pointers named "host"
 *    are read before the call returns.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Device
 *    work is asynchronous and ordered on that stream only; the call does not
 *    synchronise.
 *  - Device pointers must be 16-byte aligned (HX_EINVAL otherwise).
 *  - HX_EHIP reports a HIP runtime error from the launch (e.g. no device).
 *
 * Layout words used below: B requests, Hkv KV heads, Hq query heads,
 * G = Hq / Hkv query heads per KV head, Dk / Dv key and value widths,
 * P slices, cap rows per slice plane (a multiple of 16).
 */
#ifndef HELIXDECODE_H
#define HELIXDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HX_OK = 0,
  HX_EINVAL = 1,       /* bad argument (null, misaligned, out of range) */
  HX_EUNSUPPORTED = 2, /* valid but not implemented (shape / dtype combo) */
  HX_EHIP = 3,         /* the HIP runtime reported an error */
  HX_ENOSPC = 4        /* a block pool has too few free blocks */
} hx_status;

typedef enum {
  HX_KV_BF16 = 0,     /* bf16 K and V */
  HX_KV_FP8_E4M3 = 1, /* OCP fp8 e4m3 codes, one fp32 scale per 16-row group */
  HX_KV_MXFP4 = 2     /* OCP MX FP4 (e2m1) codes, one e8m0 scale per 32 elements of a row */
} hx_kv_dtype;

/* Token-group size of the placement: the unit that rotates over slices. */
#define HX_CHUNK 16

/* hx_kv_desc.flags.  HX_FLAG_P_BF16: the MLA kernel's value product takes
 * the softmax weights P rounded once to bf16 everywhere, with an output
 * error of up to 2^-8 times half the range of V (measured up to 2e-3 on
 * N(0, 0.5) data with short slices).  By default P enters as a bf16 high
 * part plus the bf16 of its rounding residual (error about 2^-16 of V's
 * range) on every 32-token tile where some weight exceeds 2^-10 of its
 * head's running sum, and rounded once on the others, where each weight is
 * a tiny share of the total and the rounding errors average out (measured
 * at 1M tokens: 2,635 us against 3,112 us with the residual everywhere and
 * ~2,600 us with the flag, all within 4e-6 of the exact output).  GQA bf16
 * caches always split P (no measurable cost there); fp8 / MXFP4 caches
 * round it once. */
#define HX_FLAG_P_BF16 1

/* Describes one KV cache (one layer).  Supported combinations:
 *   GQA: Dk = Dv = 128, v_alias_k = 0, dtype any, 1 <= G <= 128 (groups of
 *        more than 16 query heads run a kernel that shares each tile pair
 *        among the workgroup's waves through LDS);
 *   MLA: Dk = 576, Dv = 512, v_alias_k = 1 (V is the first 512 columns of
 *        the K row: one latent KV head), dtype any, G = 128 (fp8 and MXFP4
 *        rows are converted to bf16 in LDS before the matrix products).
 * Other combinations return HX_EUNSUPPORTED. */
typedef struct {
  int32_t P;          /* slices (KV-parallel ranks), 1..64 */
  int32_t B;          /* requests, >= 1 */
  int32_t Hkv;        /* KV heads, >= 1 */
  int32_t Dk;         /* key width */
  int32_t Dv;         /* value width */
  int32_t v_alias_k;  /* 1: V = K[..., :Dv]; the V plane is absent */
  int32_t dtype;      /* hx_kv_dtype */
  int32_t flags;      /* 0 or HX_FLAG_P_BF16 */
  int64_t cap;        /* rows per slice plane, a positive multiple of 16 */
} hx_kv_desc;

/* Device pointers of the cache planes (all caller-owned):
 *   k, v      : codes, [P][B][Hkv][cap/16] chunk tiles of 16 rows each.  The
 *               byte order inside a tile is the library's (chosen so the
 *               attention kernels load matrix-core operands with 1 KiB
 *               coalesced reads); hx_kv_tile_offset() documents it.  Write
 *               with hx_kv_append, read rows back with hx_kv_dequant.
 *   k_scale,  : HX_KV_FP8_E4M3: float [P][B][Hkv][cap/16] (one per tile);
 *   v_scale     HX_KV_BF16: unused (NULL).
 * v and v_scale are NULL when v_alias_k = 1.
 * HX_KV_MXFP4 caches are one plane, passed as k (v, k_scale and v_scale
 * NULL): each [P][B][Hkv][cap/16] chunk tile of 2,176 bytes holds the K
 * codes (1,024 B), the V codes (1,024 B), then the e8m0 exponents of K and
 * of V (16 rows x D/32 bytes each, row-major), so the attention streams one
 * contiguous run per slice.
 * Quantised MLA caches (v_alias_k = 1, fp8 or MXFP4) are one plane too,
 * passed as k: each chunk tile holds the 16 latent rows' codes, row-major
 * (fp8: 576 bytes per row; MXFP4: 288 bytes, the even element in the low
 * nibble), then fp8: the group's float scale padded to 16 bytes (9,232 B
 * per tile); MXFP4: the rows' e8m0 bytes, 18 per row, row-major (4,896 B). */
typedef struct {
  void* k;
  void* v;
  void* k_scale;
  void* v_scale;
} hx_kv_cache;

/* Byte sizes the caller allocates for each plane (0: the plane is absent,
 * pass NULL), and the tile sizes. */
typedef struct {
  size_t k_bytes, v_bytes, k_scale_bytes, v_scale_bytes;
  size_t k_tile_bytes, v_tile_bytes; /* bytes of one 16-row chunk tile (packed caches: the whole packed tile) */
  int64_t n_max;                     /* largest context: P * cap */
} hx_kv_layout_info;

/* Thread-local message of the last failing call ("" if none). */
const char* hx_last_error(void);

/* Library version string. */
const char* hx_version(void);

/* Sizes of the cache planes for `desc`.  Host only; no device work. */
hx_status hx_kv_layout(const hx_kv_desc* desc, hx_kv_layout_info* out);

/* Placement (host only).  Token t (0-based, per request) belongs to the
 * 16-token group t / 16; groups are dealt to the P slices in turn starting
 * at slice 0, so *r = (t / 16) mod P and the local row is
 * *j = ((t / 16) / P) * 16 + t mod 16 (rows keep arrival order).
 * Sources: Helix summary, paragraph on Helix's two layouts (rotation every
 * 16 tokens); NVIDIA technical blog (open-lab.net, Korean), section on
 * distributed KV placement (tokens 1-16 on rank 0, 17-32 on rank 1). */
hx_status hx_slot(int64_t t, int32_t P, int32_t* r, int64_t* j);

/* Rows held by slice r when a request has n tokens (host only):
 * floor(n / 16P) * 16 + clamp(n - floor(n / 16P) * 16P - 16 r, 0, 16). */
hx_status hx_slice_len(int64_t n, int32_t P, int32_t r, int64_t* len);

/* Byte offset (times 2, plus 1 for the high nibble of an FP4 code) of
 * element (row m of the tile, column d) inside a chunk tile of the K
 * (which = 0) or V (which = 1) codes, or of the byte that starts its scale
 * (which = 2 for K, 3 for V: fp8 the tile's float, MXFP4 the e8m0 of
 * row m, columns d / 32 * 32 ..); offsets of an MXFP4 cache count from the
 * start of its packed tile, the others from the tile of their own plane.
 * HX_EINVAL for scales of a bf16 cache or V of an aliased one.  Host only;
 * documents the tile layout for callers that write tiles themselves. */
hx_status hx_kv_tile_offset(const hx_kv_desc* desc, int32_t which, int32_t m, int32_t d, int64_t* off2);

/* Append new tokens for every KV head, placing each by hx_slot: request b
 * gets count[b] consecutive tokens (count = NULL: n_new each, count[b] may
 * be 0) starting at token pos[b] (pos, count: host arrays [B]).
 * Inputs are device arrays in storage format, token-major, with n_new rows
 * per (request, head), of which request b uses the first count[b]:
 *   k_new [B][Hkv][n_new][Dk], v_new [B][Hkv][n_new][Dv] (v_new NULL if
 *   v_alias_k): bf16 -> 2 bytes per element; fp8 -> 1 byte; MXFP4 -> packed
 *   bytes [..][Dk/2], even element in the low nibble;
 *   k_scale_new / v_scale_new: fp8 -> float [B][Hkv][n_new], the scale of
 *   the 16-token group each token falls in.  A group whose first row is
 *   among the new tokens takes the scale of that row; a group that already
 *   holds rows keeps its stored scale, and new codes of such a group are
 *   read under it (the scales of its new tokens are not used), so they must
 *   have been made with that scale.  The scales are device data the host
 *   does not see, so a mismatch cannot be reported; hx_kv_append_bf16 and
 *   hx_decode_step_bf16 quantise on the device and keep each group's scale
 *   consistent by themselves.  MXFP4 -> uint8 e8m0 [B][Hkv][n_new][D/32];
 *   bf16 -> NULL.
 * Pure placement: the bytes are copied, never converted, so it is
 * bit-exact.  Rows outside [pos[b], pos[b] + count[b]) are left unchanged.
 * Requires n_new >= 1, 0 <= count[b] <= n_new, 0 <= pos[b] and
 * pos[b] + count[b] <= P * cap. */
hx_status hx_kv_append(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* k_new, const void* v_new,
                       const void* k_scale_new, const void* v_scale_new, const int64_t* pos, const int32_t* count,
                       int32_t n_new, void* stream);

/* Append new tokens given as bf16 values, quantising them into the cache's
 * storage format on the device (same placement, pos, count and n_new
 * conventions as hx_kv_append; the new KV rows of a decode step come out of
 * the QKV projection and are written round-robin as produced: Helix summary,
 * paragraph on Helix's two layouts).  k_new [B][Hkv][n_new][Dk] and v_new
 * [B][Hkv][n_new][Dv] are bf16 (device; v_new NULL if v_alias_k).
 *   bf16 cache: identical to hx_kv_append.
 *   fp8 e4m3 cache: per 16-token group of a (request, KV head, K or V),
 *     scale = amax / 448 (fp32; 1 for an all-zero group) and code = nearest
 *     e4m3 (ties to even) of x / scale clamped to +-448.  A group filled over
 *     several calls keeps a scale that only grows: when the new rows' amax
 *     exceeds 448 * stored scale (and the group holds a non-zero code), the
 *     scale becomes amax / 448 and the stored codes are re-encoded from
 *     their values times old / new scale; otherwise new rows use the stored
 *     scale.  A group written in one call gets exactly the per-group rule.
 *   MXFP4 cache: per 32 consecutive elements of a row, E = clamp(floor(
 *     log2 amax) - 2, -127, 127) + 127 and code = nearest e2m1 (ties to
 *     even, saturating at 6) of x / 2^(E-127); rows are independent.
 * Deterministic, so equal inputs give equal bytes.  Errors as hx_kv_append. */
hx_status hx_kv_append_bf16(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* k_new, const void* v_new,
                            const int64_t* pos, const int32_t* count, int32_t n_new, void* stream);

/* Decode rows [j0, j0 + n) of slice r, request b, KV head g into fp32:
 * k_out [n][Dk], v_out [n][Dv] (device; v_out may be NULL).  bf16: exact
 * widening; fp8: fp32 product code * scale rounded to nearest-even; MXFP4:
 * code * 2^(E-127), exact.  For tests and inspection, not the hot path. */
hx_status hx_kv_dequant(const hx_kv_desc* desc, const hx_kv_cache* cache, int32_t r, int32_t b, int32_t g,
                        int64_t j0, int64_t n, float* k_out, float* v_out, void* stream);

/* Workspace bytes hx_decode_attn_partial and hx_decode_attn need for `desc`
 * with Hq query heads (host only).  The workspace holds the partial results
 * of the splits each slice is cut into (and, for hx_decode_attn, the slice
 * partials); it needs no initialisation and its contents are scratch
 * between calls. */
hx_status hx_workspace_size(const hx_kv_desc* desc, int32_t Hq, size_t* bytes);

/* Zero a workspace (device) on `stream` (optional; for callers that want
 * deterministic bytes in it). */
hx_status hx_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Per-slice partial attention for one decode step, every slice in one
 * launch (Helix summary, paragraph on KV parallelism: each slice attends
 * over its part of the history and returns a partial output and a
 * log-sum-exp).
 *   q        device bf16 [B][Hq][Dk]; query head h uses KV head h / G.
 *   ctx_len  host int64 [B]: tokens of request b, 1 <= ctx_len[b] <= P*cap;
 *            slice r holds hx_slice_len(ctx_len[b], P, r) rows.
 *   scale    softmax scale applied to q.k (e.g. 1/sqrt(Dk)).
 *   o_part   device float [P][B][Hq][Dv]: O_r = sum_t softmax_r(s)_t V_t
 *            over slice r's tokens (normalised); 0 for an empty slice.
 *   lse_part device float [P][B][Hq]: LSE_r = ln sum_{t in r} exp(s_t)
 *            (natural log); -inf for an empty slice.
 *   ws       device workspace of hx_workspace_size bytes (see there).
 * A call launches the partial kernel and, when some slice is cut into
 * several splits, a small kernel that folds the splits of each slice.
 * Calls that share a workspace must be ordered (same stream). */
hx_status hx_decode_attn_partial(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* q, int32_t Hq,
                                 const int64_t* ctx_len, float scale, float* o_part, float* lse_part, void* ws,
                                 size_t ws_bytes, void* stream);

/* The whole decode step's attention in one call: the final O [B][Hq][Dv]
 * (fp32, normalised) and natural-log LSE [B][Hq] of every query head over
 * its request's full context, i.e. hx_decode_attn_partial followed by
 * hx_lse_combine (Helix summary, paragraph on KV parallelism; jaehun.me
 * review, Prompt 1.3.2), for callers that hold all slices on one GPU and do
 * not need the per-slice partials.  Same arguments and checks as
 * hx_decode_attn_partial, with o, lse (device, 16-byte aligned) in place of
 * o_part, lse_part; the slice partials live in the workspace.  Two kernel
 * launches: the partial pass, then one kernel that folds every slice's
 * partial (or its split records) into the final output with the LSE rule,
 * in place of the split fold and the combine. */
hx_status hx_decode_attn(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* q, int32_t Hq,
                         const int64_t* ctx_len, float scale, float* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream);

/* hx_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks, kernels and
 * results as hx_decode_attn (bit for bit); the scratch is the library's own
 * fixed array of 128 MiB per device (allocated when the library's code is
 * loaded on that device and held until the process ends), so the call
 * allocates nothing.  A call whose split records and slice partials need
 * more than 128 MiB returns HX_EINVAL (then use hx_decode_attn); every
 * workload up to 8 requests x 128 MLA heads x 2^20 tokens fits.  All calls on
 * one device share that device's scratch: calls that may overlap on one
 * device (other streams, other host threads) race and must be ordered by
 * the caller. */
hx_status hx_decode_attn_noalloc(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* q, int32_t Hq,
                                 const int64_t* ctx_len, float scale, float* o, float* lse, void* stream);

/* A whole decode step in one call for callers that hold all slices on one
 * GPU: append each request's n_new newest rows, then hx_decode_attn.  The
 * new rows are rows [ctx_len[b] - n_new, ctx_len[b]) of request b, given in
 * storage format as for hx_kv_append (k_new [B][Hkv][n_new][..] etc., count
 * = n_new for every request; requires ctx_len[b] >= n_new >= 1); O, LSE,
 * workspace and the other arguments as hx_decode_attn.  The append runs
 * inside the partial kernel: the workgroup that owns a new row's chunk tile
 * writes the row before it reads the tile (one launch fewer than append +
 * attention; the cache afterwards holds exactly what hx_kv_append writes).
 * MXFP4 caches take the append kernel first instead (their fused kernel was
 * slower than the launch it saves), and so do quantised MLA caches (their
 * kernel converts tiles in LDS before reading them); all arguments are
 * checked before the cache is written.  Helix summary, paragraphs on
 * Helix's two layouts (new KV written round-robin as produced) and on KV
 * parallelism. */
hx_status hx_decode_step(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* k_new, const void* v_new,
                         const void* k_scale_new, const void* v_scale_new, int32_t n_new, const void* q, int32_t Hq,
                         const int64_t* ctx_len, float scale, float* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream);

/* hx_decode_step with the step's new rows given as bf16 values (what the
 * QKV projection produces: k_new [B][Hkv][n_new][Dk], v_new
 * [B][Hkv][n_new][Dv], bf16, device; v_new NULL if v_alias_k), quantised
 * into the cache's format inside the partial kernel by the workgroup that
 * owns each new row's chunk tile, with the rules of hx_kv_append_bf16 (fp8:
 * a group's scale grows and its stored codes are re-encoded when the new
 * rows need it; MXFP4: per-row block exponents).  Two launches for any
 * format: the partial kernel (which quantises first), then the fold into O
 * and LSE.  The cache afterwards holds exactly what hx_kv_append_bf16
 * writes, and O / LSE equal hx_kv_append_bf16 followed by hx_decode_attn.
 * Quantised MLA caches take the quantising append kernel first (three
 * launches; all arguments are checked before the cache is written).
 * A bf16 cache takes the rows as storage format (= hx_decode_step).  Other
 * arguments, checks and errors as hx_decode_step.  Helix summary,
 * paragraphs on Helix's two layouts (new KV written round-robin as
 * produced) and on KV parallelism. */
hx_status hx_decode_step_bf16(const hx_kv_desc* desc, const hx_kv_cache* cache, const void* k_new, const void* v_new,
                              int32_t n_new, const void* q, int32_t Hq, const int64_t* ctx_len, float scale, float* o,
                              float* lse, void* ws, size_t ws_bytes, void* stream);

/* LSE-weighted combine of P partials (jaehun.me review, Prompt 1.3.2):
 *   m = max_r LSE_r, w_r = exp(LSE_r - m),
 *   o = sum_r w_r O_r / sum_r w_r,  lse = m + ln sum_r w_r.
 * o_part [P][B][Hq][Dv], lse_part [P][B][Hq] (device float) ->
 * o [B][Hq][Dv], lse [B][Hq] (device float).  All-empty rows (every
 * LSE_r = -inf) give o = 0, lse = -inf.  1 <= P <= 1024. */
hx_status hx_lse_combine(int32_t P, int32_t B, int32_t Hq, int32_t Dv, const float* o_part, const float* lse_part,
                         float* o, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * Block-pool (paged) caches
 *
 * The same placement (hx_slot) with a different storage: instead of a
 * [P][B][Hkv][cap/16] plane sized for the longest request, every slice of
 * every request is a list of 16-row blocks taken from one shared pool, so
 * requests grow independently and memory follows the tokens actually held
 * (the 16-token group is the placement unit and an even memory fill is what
 * the rotation is for: Helix summary, paragraph on Helix's two layouts).
 *
 * A block holds the 16-row chunk tiles of all Hkv KV heads for one (request,
 * slice, 16-row group).  Planes of a pool of N blocks (device, caller-owned,
 * sizes from hx_pool_layout):
 *   k, v       : [N][Hkv] chunk tiles, tile byte order as in the dense cache;
 *   k_scale,   : fp8: float [N][Hkv]; bf16: NULL.
 *   v_scale      v and v_scale are NULL when v_alias_k = 1.
 *   MXFP4: one plane k of [N][Hkv] packed 2,176-byte tiles as in the dense
 *   cache (v, k_scale, v_scale NULL).
 * block_table: device int32 [B][P][cap/16].  Entry (b, r, c) is the block
 *   holding local rows 16c .. 16c+15 of slice r of request b.  desc->cap is
 *   the longest slice a table row can describe (16 entries' worth of rows
 *   per entry), so contexts still satisfy ctx <= P * cap.  Every entry a call
 *   reads or writes (the groups of the rows it touches) must hold a block id
 *   in [0, N), and distinct (b, r, c) in use must hold distinct blocks; ids
 *   outside [0, N) are clamped into it on the device (wrong rows, never an
 *   access outside the planes).  Entries of groups past a slice's rows are
 *   never read.  hx_block_pool_* below maintain such a table on the host.
 * ------------------------------------------------------------------------ */
typedef struct {
  hx_kv_cache planes;          /* k, v, k_scale, v_scale of the pool */
  const int32_t* block_table;  /* device [B][P][cap/16] */
  int32_t num_blocks;          /* N >= 1 */
  int32_t reserved;            /* must be 0 */
} hx_kv_pool;

/* Plane sizes of a pool of num_blocks blocks for `desc` (host only);
 * n_max = P * cap, the longest context the block table can describe. */
hx_status hx_pool_layout(const hx_kv_desc* desc, int32_t num_blocks, hx_kv_layout_info* out);

/* hx_kv_append, hx_kv_append_bf16 and hx_kv_dequant on a pool cache: same
 * arguments, placement, encoding and errors, with the rows addressed through
 * the block table (HX_EINVAL also for a null or misaligned table or
 * num_blocks < 1). */
hx_status hx_kv_append_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* k_new, const void* v_new,
                             const void* k_scale_new, const void* v_scale_new, const int64_t* pos,
                             const int32_t* count, int32_t n_new, void* stream);
hx_status hx_kv_append_bf16_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* k_new,
                                  const void* v_new, const int64_t* pos, const int32_t* count, int32_t n_new,
                                  void* stream);
hx_status hx_kv_dequant_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, int32_t r, int32_t b, int32_t g,
                              int64_t j0, int64_t n, float* k_out, float* v_out, void* stream);

/* hx_decode_attn_partial and hx_decode_attn on a pool cache (same
 * arguments, outputs, workspace and errors).  The kernels are the dense
 * ones with tile addresses taken from the block table, so for equal rows
 * the results are bit-identical to the dense cache's. */
hx_status hx_decode_attn_partial_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* q, int32_t Hq,
                                       const int64_t* ctx_len, float scale, float* o_part, float* lse_part, void* ws,
                                       size_t ws_bytes, void* stream);
hx_status hx_decode_attn_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* q, int32_t Hq,
                               const int64_t* ctx_len, float scale, float* o, float* lse, void* ws, size_t ws_bytes,
                               void* stream);

/* hx_decode_step and hx_decode_step_bf16 on a pool cache (the new rows'
 * blocks must be listed). */
hx_status hx_decode_step_bf16_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* k_new,
                                    const void* v_new, int32_t n_new, const void* q, int32_t Hq,
                                    const int64_t* ctx_len, float scale, float* o, float* lse, void* ws,
                                    size_t ws_bytes, void* stream);
hx_status hx_decode_step_paged(const hx_kv_desc* desc, const hx_kv_pool* pool, const void* k_new, const void* v_new,
                               const void* k_scale_new, const void* v_scale_new, int32_t n_new, const void* q,
                               int32_t Hq, const int64_t* ctx_len, float scale, float* o, float* lse, void* ws,
                               size_t ws_bytes, void* stream);

/* Host-side block allocator for a pool of num_blocks blocks: a free list
 * that hands out the most recently freed block first (initially 0, 1, ...).
 * The handle is an opaque host object; calls on one handle are serialised
 * internally.  The tables it edits are host arrays int32 [B][P][cap/16] in
 * the layout of hx_kv_pool.block_table, with -1 marking an entry without a
 * block; the caller copies them to the device table. */
typedef struct hx_block_pool hx_block_pool;

hx_status hx_block_pool_create(int32_t num_blocks, hx_block_pool** out);
void hx_block_pool_destroy(hx_block_pool* pool);
hx_status hx_block_pool_free_count(const hx_block_pool* pool, int32_t* n_free);

/* Make request b's lists cover a context of n tokens: every entry (b, r, c)
 * with c < ceil(hx_slice_len(n, P, r) / 16) that holds -1 gets a free block;
 * entries already holding a block keep it.  Every entry of request b's
 * lists other than -1 must be a block handed to request b, and no block may
 * be listed twice (else HX_EINVAL, as for hx_block_pool_release).  All or
 * nothing: on any error nothing changes; with too few free blocks
 * HX_ENOSPC is returned.  *n_taken (may be NULL)
 * receives the number of blocks handed out.  0 <= n <= P * cap. */
hx_status hx_block_pool_reserve(hx_block_pool* pool, const hx_kv_desc* desc, int32_t* table_host, int32_t b,
                                int64_t n, int32_t* n_taken);

/* Return every block of request b's lists to the pool and set its entries to
 * -1 (a finished request).  An entry (other than -1) that is not a block
 * handed to request b, or a block listed twice, is HX_EINVAL and leaves the
 * pool and the table unchanged. */
hx_status hx_block_pool_release(hx_block_pool* pool, const hx_kv_desc* desc, int32_t* table_host, int32_t b);

/* ------------------------------------------------------------------------
 * Launch trace (for profiling; not needed to use the library)
 *
 * hx_trace_begin records a start event on `stream` and opens a trace; until
 * hx_trace_end, every kernel the library launches (from any thread) is
 * followed by a HIP event recorded on that launch's stream, for up to
 * `capacity` (1 .. 2^20) launches.  hx_trace_end waits for the last event,
 * closes the trace and reports, for launch i, its kernel's name (`names`:
 * host char [capacity][32], NUL-terminated: "gqa_partial",
 * "gqa_wide_partial", "mla_partial", "split_fold", "fold_combine",
 * "lse_combine", "append", "quant_append", "dequant") and ms[i] (host float
 * [capacity]): the time from the previous event (the start event for i = 0)
 * to the end of launch i, which is the launch's duration when every traced
 * launch is on `stream` and nothing else runs on it in between.  *n
 * receives the number of launches.  HX_ENOSPC: more launches than
 * `capacity` (the first `capacity` are reported); HX_EINVAL: a trace is
 * already open (begin) or none is (end).  Events are host-side HIP objects
 * created by hx_trace_begin and destroyed by hx_trace_end; do not open a
 * trace around HIP graph capture.
 * ------------------------------------------------------------------------ */
hx_status hx_trace_begin(int32_t capacity, void* stream);
/* Adds the caller's own entry `name` (at most 31 characters kept) to the
 * open trace, recorded on `stream` now: it ends the interval of whatever
 * the caller ran on the stream since the previous entry (HX_EINVAL when no
 * trace is open). */
hx_status hx_trace_mark(const char* name, void* stream);
hx_status hx_trace_end(int32_t* n, float* ms, char* names);

/* ------------------------------------------------------------------------
 * Read probe (a measurement aid; not needed to use the library)
 *
 * Every kernel of the decode path is bound by reading the KV cache from HBM
 * once, so its rate is best judged against what a plain read reaches on the
 * same device.  hx_read_probe reads `nbytes` (a positive multiple of 16) of
 * device memory at `src` (16-byte aligned) once, in 16-byte non-temporal
 * loads per lane (1 KiB per wave-wide load, as the attention kernels load
 * their tiles), and writes to out[i] (device uint32 [HX_READ_PROBE_BLOCKS])
 * the XOR of the 32-bit words workgroup i read.  Asynchronous on `stream`;
 * a traced launch is named "read_probe".  HX_EINVAL: null or misaligned
 * pointer, or nbytes not a positive multiple of 16.
 * ------------------------------------------------------------------------ */
#define HX_READ_PROBE_BLOCKS 1024
hx_status hx_read_probe(const void* src, int64_t nbytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HELIXDECODE_H */
