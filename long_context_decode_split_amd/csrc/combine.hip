// LSE-weighted combine of per-slice partials (jaehun.me review, Prompt 1.3.2,
// boxed formula O = sum_r O_r e^{LSE_r} / sum_r e^{LSE_r}), evaluated after
// scaling numerator and denominator by e^{-max_r LSE_r}.  It stands in for the
// all-to-all plus rescale between KV-parallel ranks (Helix summary, paragraph
// on KV parallelism): on one GPU the partials are already in HBM.
//
// One workgroup per (request, query head) row; the P log-sum-exps are read
// once into LDS, and each thread folds its columns of O in base 2.

#include "hx_common.h"

namespace hx {
namespace {

constexpr int kThreads = 128;
constexpr int kMaxP = 1024;
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;

__global__ __launch_bounds__(kThreads) void lse_combine_kernel(int P, int rows, int Dv, const float* __restrict__ o_part,
                                                               const float* __restrict__ lse_part, float* __restrict__ o,
                                                               float* __restrict__ lse) {
  __shared__ float s_w[kMaxP];
  __shared__ float s_red[kThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  // max over the slices
  float m = -INFINITY;
  for (int r = tid; r < P; r += kThreads) {
    const float l = lse_part[(int64_t)r * rows + row];
    s_w[r] = l;
    m = fmaxf(m, l);
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  m = s_red[0];
  for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, s_red[w]);
  __syncthreads();
  // weights 2^((LSE_r - m) log2 e); an empty slice (-inf) weighs 0
  float den = 0.f;
  const bool all_empty = m == -INFINITY;
  for (int r = tid; r < P; r += kThreads) {
    const float w = all_empty ? 0.f : __builtin_amdgcn_exp2f((s_w[r] - m) * kLog2e);
    s_w[r] = w;
  }
  __syncthreads();
  for (int r = 0; r < P; ++r) den += s_w[r];
  for (int d = tid; d < Dv; d += kThreads) {
    float num = 0.f;
    for (int r = 0; r < P; ++r) {
      const float w = s_w[r];
      if (w != 0.f) num += w * o_part[((int64_t)r * rows + row) * Dv + d];
    }
    o[(int64_t)row * Dv + d] = den > 0.f ? num / den : 0.f;
  }
  if (tid == 0) lse[row] = den > 0.f ? m + __log2f(den) * kLn2 : -INFINITY;
}

// Fold of the split records of one slice into the slice's partial, by the
// same LSE rule: one workgroup per (slice, query head), threads over value
// columns.  The split LSEs and weights live in LDS; each thread keeps eight
// splits' loads in flight at a time.
constexpr int kFoldThreads = 128;

__global__ __launch_bounds__(kFoldThreads) void split_fold_kernel(const PartialArgs a) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[kFoldThreads / 64];
  const int G = a.G, Dv = a.Dv, P = a.P;
  const int f = blockIdx.x;
  int bl = 0;
  while (bl + 1 < a.nb && a.fold_begin[bl + 1] <= f) ++bl;
  const int nsplit = a.nsplit[bl];
  int rem = f - a.fold_begin[bl];
  const int hd = rem % G;
  rem /= G;
  const int r = rem % P;
  const int g = rem / P;
  const int b = a.b0 + bl;
  const int64_t rec0 = a.wg_begin[bl] + (int64_t)(g * P + r) * nsplit;
  const int tid = threadIdx.x;

  float m = -INFINITY;
  for (int sp = tid; sp < nsplit; sp += kFoldThreads) {
    const float l = a.ws_lse[(rec0 + sp) * G + hd];
    s_w[sp] = l;
    m = fmaxf(m, l);
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  m = s_red[0];
#pragma unroll
  for (int w = 1; w < kFoldThreads / 64; ++w) m = fmaxf(m, s_red[w]);
  __syncthreads();
  const bool empty = m == -INFINITY;
  for (int sp = tid; sp < nsplit; sp += kFoldThreads)
    s_w[sp] = empty ? 0.f : __builtin_amdgcn_exp2f((s_w[sp] - m) * kLog2e);
  __syncthreads();
  float den = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) den += s_w[sp];

  const float* src = a.ws_o + (rec0 * G + hd) * (int64_t)Dv;
  const int64_t rstride = (int64_t)G * Dv;   // floats between split records
  float* dst = a.o_part + (((int64_t)r * a.Btot + b) * a.Hq + g * G + hd) * Dv;
  for (int d = tid; d < Dv; d += kFoldThreads) {
    float num = 0.f;
    int sp = 0;
    for (; sp + 8 <= nsplit; sp += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[(sp + u) * rstride + d];
#pragma unroll
      for (int u = 0; u < 8; ++u) num += s_w[sp + u] * v[u];
    }
    for (; sp < nsplit; ++sp) num += s_w[sp] * src[sp * rstride + d];
    dst[d] = den > 0.f ? num / den : 0.f;
  }
  if (tid == 0)
    a.lse_part[((int64_t)r * a.Btot + b) * a.Hq + g * G + hd] = den > 0.f ? m + __log2f(den) * kLn2 : -INFINITY;
}

// hx_decode_attn's completion: one workgroup per (request, query head) of
// the launch folds the partial of every (slice, split) of its group by the
// same LSE rule, straight into the final output: for a slice with one split
// the partial kernel wrote the slice output, otherwise the split records.
constexpr int kFcThreads = 256;
constexpr int kFcMaxItems = kMaxSplits * 64;   // P * nsplit (P <= 64)

__global__ __launch_bounds__(kFcThreads) void fold_combine_kernel(const PartialArgs a, float* __restrict__ o,
                                                                  float* __restrict__ lse) {
  __shared__ float s_w[kFcMaxItems];
  __shared__ float s_red[kFcThreads / 64];
  const int G = a.G, Dv = a.Dv, P = a.P;
  const int f = blockIdx.x;
  const int bl = f / a.Hq;
  const int hq = f % a.Hq;
  const int g = hq / G, hd = hq % G;
  const int b = a.b0 + bl;
  const int nsplit = a.nsplit[bl];
  const int items = P * nsplit;
  const int64_t rec0 = a.wg_begin[bl] + (int64_t)g * P * nsplit;   // records of (request, KV head g), slice-major
  const int tid = threadIdx.x;
  auto item_lse = [&](int i) -> float {
    return nsplit == 1 ? a.lse_part[((int64_t)i * a.Btot + b) * a.Hq + hq] : a.ws_lse[(rec0 + i) * G + hd];
  };
  auto item_o4 = [&](int i, int d) -> float4 {
    const float* p = nsplit == 1 ? a.o_part + (((int64_t)i * a.Btot + b) * a.Hq + hq) * Dv + d
                                 : a.ws_o + ((rec0 + i) * G + hd) * Dv + d;
    return *reinterpret_cast<const float4*>(p);
  };
  float m = -INFINITY;
  for (int i = tid; i < items; i += kFcThreads) {
    const float l = item_lse(i);
    s_w[i] = l;
    m = fmaxf(m, l);
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  m = s_red[0];
#pragma unroll
  for (int w = 1; w < kFcThreads / 64; ++w) m = fmaxf(m, s_red[w]);
  __syncthreads();
  const bool empty = m == -INFINITY;
  for (int i = tid; i < items; i += kFcThreads) s_w[i] = empty ? 0.f : __builtin_amdgcn_exp2f((s_w[i] - m) * kLog2e);
  __syncthreads();
  float den = 0.f;
  for (int i = 0; i < items; ++i) den += s_w[i];
  // threads split the items into groups; each thread sums 4 consecutive
  // columns of its group's items with independent 16-byte loads (every
  // record and slice output is written, so weight-0 items add exact zeros),
  // then the groups' sums are added in LDS
  const int lanes = Dv / 4;                  // threads per item group
  const int groups = kFcThreads / lanes;     // Dv = 128: 8, Dv = 512: 2
  const int grp = tid / lanes, d4 = 4 * (tid % lanes);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (grp < groups) {
    int i = grp;
    for (; i + 3 * groups < items; i += 4 * groups) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = item_o4(i + u * groups, d4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = s_w[i + u * groups];
        acc.x += w * v[u].x;
        acc.y += w * v[u].y;
        acc.z += w * v[u].z;
        acc.w += w * v[u].w;
      }
    }
    for (; i < items; i += groups) {
      const float4 v = item_o4(i, d4);
      const float w = s_w[i];
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
  }
  __shared__ float4 s_acc[kFcThreads];
  s_acc[tid] = acc;
  __syncthreads();
  if (grp == 0) {
    for (int q = 1; q < groups; ++q) {
      const float4 t = s_acc[q * lanes + tid];
      acc.x += t.x;
      acc.y += t.y;
      acc.z += t.z;
      acc.w += t.w;
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    float4* out = reinterpret_cast<float4*>(o + ((int64_t)b * a.Hq + hq) * Dv + d4);
    *out = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (tid == 0) lse[(int64_t)b * a.Hq + hq] = den > 0.f ? m + __log2f(den) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_fold_combine(const PartialArgs& a, float* o, float* lse, hipStream_t st) {
  const int nf = a.nb * a.Hq;
  if (nf == 0) return hipSuccess;
  for (int i = 0; i < a.nb; ++i)
    if (a.nsplit[i] * a.P > kFcMaxItems) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fold_combine_kernel, dim3(nf), dim3(kFcThreads), 0, st, a, o, lse);
  return hipGetLastError();
}

hipError_t launch_split_fold(const PartialArgs& a, hipStream_t st) {
  const int nf = a.fold_begin[a.nb];
  if (nf == 0) return hipSuccess;
  hipLaunchKernelGGL(split_fold_kernel, dim3(nf), dim3(kFoldThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_lse_combine(int P, int B, int Hq, int Dv, const float* o_part, const float* lse_part, float* o,
                              float* lse, hipStream_t st) {
  const int rows = B * Hq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_combine_kernel, dim3(rows), dim3(kThreads), 0, st, P, rows, Dv, o_part, lse_part, o, lse);
  return hipGetLastError();
}

}  // namespace hx
