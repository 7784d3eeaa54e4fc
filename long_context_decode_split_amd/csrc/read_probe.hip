// A plain streaming read of a device buffer, as a measurement aid: the rate
// it reaches is the practical HBM read ceiling that the attention kernels'
// rates are compared with (every attention kernel here is bound by reading
// the KV cache once).  As the attention kernels stream a slice, each
// workgroup reads one contiguous run of the buffer; each lane reads 16 bytes
// with the non-temporal policy (the kernels' policy for KV rows), so each
// wave-wide load reads 1 KiB contiguous, and a workgroup keeps kUnroll loads
// per lane (kUnroll x 4 KiB) in flight.  The XOR of everything read goes to
// out[block] so no read is dead.

#include "hx_common.h"

namespace hx {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// 1,024 workgroups of 4 waves with 4 loads per lane in flight: the fastest
// of unroll 4 / 8 / 16 x 1,024 / 2,048 / 4,096 workgroups on MI355X (4 GiB:
// 6.7 - 7.0 TB/s, all within 5% of each other)
#ifndef HX_READ_PROBE_UNROLL
#define HX_READ_PROBE_UNROLL 4
#endif
constexpr int kThreadsRP = 256;
constexpr int kUnroll = HX_READ_PROBE_UNROLL;

__global__ __launch_bounds__(kThreadsRP) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                uint32_t* __restrict__ out) {
  // run of this workgroup: [beg, end) in 16-byte units, whole 4 KiB rows
  constexpr int64_t kRow = kThreadsRP;
  const int64_t rows = (n16 + kRow - 1) / kRow;
  const int64_t per = (rows + gridDim.x - 1) / gridDim.x;
  const int64_t beg = min(n16, (int64_t)blockIdx.x * per * kRow);
  const int64_t end = min(n16, beg + per * kRow);
  int64_t i = beg + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kUnroll - 1) * kRow < end; i += kUnroll * kRow) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kRow);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += kRow) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
  __shared__ uint32_t s_x[kThreadsRP / 64];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kThreadsRP / 64; ++w) r ^= s_x[w];
    out[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* src, int64_t nbytes, uint32_t* out, int nblocks, hipStream_t st) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(nblocks), dim3(kThreadsRP), 0, st, (const u32x4*)src, nbytes / 16, out);
  return hipGetLastError();
}

}  // namespace hx
