// HBM stream kernels used to measure this GPU's practical bandwidth ceilings beside the
// hot path (a measurement library, separate from libbutler and its ABI).
//
//   butler_measure_read  : every byte of a buffer read once with 16-byte loads, nothing
//                          written but one word per workgroup (the reads feed an xor that
//                          the compiler cannot drop)
//   butler_measure_copy  : a plain copy, 16-byte loads and stores
//
// Each workgroup streams one contiguous slice of the buffer (DRAM pages stay open), with
// `unroll` loads of 16 bytes per lane in flight before the first is used.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

template <int U>
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, long long n16,
                                                   uint32_t* __restrict__ sink) {
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long lo = (long long)blockIdx.x * per;
  const long long hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  long long i = lo + threadIdx.x;
  for (; i + 256LL * (U - 1) < hi; i += 256LL * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + 256LL * u];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += 256) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t s[4];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

template <int U>
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, long long n16) {
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long lo = (long long)blockIdx.x * per;
  const long long hi = lo + per < n16 ? lo + per : n16;
  long long i = lo + threadIdx.x;
  for (; i + 256LL * (U - 1) < hi; i += 256LL * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + 256LL * u];
#pragma unroll
    for (int u = 0; u < U; ++u) dst[i + 256LL * u] = v[u];
  }
  for (; i < hi; i += 256) dst[i] = src[i];
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned src) with `blocks` workgroups of 256
// threads and `unroll` in {1, 2, 4, 8, 16} loads per lane in flight; sink holds `blocks`
// words.  Returns 0, or -1 on bad arguments, -4 on a launch error.
int butler_measure_read(void* stream, const void* src, size_t bytes, uint32_t* sink, int blocks,
                        int unroll) {
  if (!src || !sink || bytes % 16 || ((uintptr_t)src & 15) || blocks <= 0) return -1;
  const long long n16 = (long long)(bytes / 16);
  hipStream_t s = (hipStream_t)stream;
  const dim3 g((unsigned)blocks), b(256);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(read_kernel<1>, g, b, 0, s, (const uint4*)src, n16, sink); break;
    case 2: hipLaunchKernelGGL(read_kernel<2>, g, b, 0, s, (const uint4*)src, n16, sink); break;
    case 4: hipLaunchKernelGGL(read_kernel<4>, g, b, 0, s, (const uint4*)src, n16, sink); break;
    case 8: hipLaunchKernelGGL(read_kernel<8>, g, b, 0, s, (const uint4*)src, n16, sink); break;
    case 16: hipLaunchKernelGGL(read_kernel<16>, g, b, 0, s, (const uint4*)src, n16, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Copies `bytes` (a multiple of 16, both pointers 16-byte aligned, not overlapping).
int butler_measure_copy(void* stream, const void* src, void* dst, size_t bytes, int blocks,
                        int unroll) {
  if (!src || !dst || bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15) ||
      blocks <= 0)
    return -1;
  const long long n16 = (long long)(bytes / 16);
  hipStream_t s = (hipStream_t)stream;
  const dim3 g((unsigned)blocks), b(256);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(copy_kernel<1>, g, b, 0, s, (const uint4*)src, (uint4*)dst, n16); break;
    case 2: hipLaunchKernelGGL(copy_kernel<2>, g, b, 0, s, (const uint4*)src, (uint4*)dst, n16); break;
    case 4: hipLaunchKernelGGL(copy_kernel<4>, g, b, 0, s, (const uint4*)src, (uint4*)dst, n16); break;
    case 8: hipLaunchKernelGGL(copy_kernel<8>, g, b, 0, s, (const uint4*)src, (uint4*)dst, n16); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
