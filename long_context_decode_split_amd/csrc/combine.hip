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

}  // namespace

hipError_t launch_lse_combine(int P, int B, int Hq, int Dv, const float* o_part, const float* lse_part, float* o,
                              float* lse, hipStream_t st) {
  const int rows = B * Hq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_combine_kernel, dim3(rows), dim3(kThreads), 0, st, P, rows, Dv, o_part, lse_part, o, lse);
  return hipGetLastError();
}

}  // namespace hx
