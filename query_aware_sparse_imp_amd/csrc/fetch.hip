// Selected-row fetch from a KV cache kept in host memory (TokenButler arXiv abstract: the
// predictor's selection cuts decode latency against dense attention whose KV cache is
// offloaded to the CPU, because only the selected tokens' rows have to reach the GPU).
// The cache sits in pinned host memory that the GPU maps; this kernel reads the selected
// K and V rows across the host link (zero copy: no staging copy of the whole cache) and
// packs them per selected set, in set order, into device memory, where the attention
// then reads them at HBM speed.  It also takes a device-resident cache (a plain gather).
//
// One workgroup per (selection row, chunk of 1024 16-byte pieces per tensor).  Consecutive
// threads take consecutive pieces of a row, so each row leaves as one contiguous request;
// every thread issues its index loads, then all of its K and V loads, before any store.
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr int kFtThreads = 256;
constexpr int kFtPieces = 1024;                  // 16-byte pieces per workgroup and tensor
constexpr int kFtU = kFtPieces / kFtThreads;     // pieces per thread and tensor

// PPR: 16-byte pieces per cache row (D * element size / 16)
template <int PPR>
__global__ __launch_bounds__(kFtThreads) void fetch_rows_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
    const uint4* __restrict__ k, const uint4* __restrict__ v, uint4* __restrict__ k_sel,
    uint4* __restrict__ v_sel, int rows, int kvdiv, int L_cap, int cap) {
  constexpr int PPB = kFtPieces / PPR;           // list positions per workgroup
  const int row = blockIdx.x % rows, chunk = blockIdx.x / rows;
  const int n = min(count[row], cap);
  const int p0 = chunk * PPB;
  if (p0 >= n) return;
  const int total = min(PPB, n - p0) * PPR;      // pieces of this workgroup, >= 1
  const size_t src0 = (size_t)(row / kvdiv) * L_cap;
  const int32_t* irow = idx + (size_t)row * cap + p0;
  // token of every piece; positions past the end repeat the last piece (loaded, not stored)
  // and indices outside [0, L_cap) are clamped so a bad list never reads past the cache
  int tok[kFtU];
#pragma unroll
  for (int u = 0; u < kFtU; ++u) {
    const int q = min((int)threadIdx.x + u * kFtThreads, total - 1);
    tok[u] = (int)min((unsigned)irow[q / PPR], (unsigned)(L_cap - 1));
  }
  uint4 rk[kFtU], rv[kFtU];
#pragma unroll
  for (int u = 0; u < kFtU; ++u) {
    const int q = min((int)threadIdx.x + u * kFtThreads, total - 1);
    const size_t off = (src0 + tok[u]) * PPR + q % PPR;
    rk[u] = k[off];
    rv[u] = v[off];
  }
  uint4* kd = k_sel + ((size_t)row * cap + p0) * PPR;
  uint4* vd = v_sel + ((size_t)row * cap + p0) * PPR;
#pragma unroll
  for (int u = 0; u < kFtU; ++u) {
    const int q = (int)threadIdx.x + u * kFtThreads;
    if (q < total) {
      kd[q] = rk[u];
      vd[q] = rv[u];
    }
  }
}

}  // namespace

long long fetch_rows_blocks(long long rows, int cap, int row_bytes) {
  const int ppr = row_bytes / 16;
  const int ppb = kFtPieces / ppr;
  return rows * ((cap + ppb - 1) / ppb);
}

hipError_t launch_fetch_rows(hipStream_t s, const int32_t* idx, const int32_t* count,
                             const void* k, const void* v, void* k_sel, void* v_sel, int rows,
                             int kvdiv, int row_bytes, int L_cap, int cap) {
  const long long blocks = fetch_rows_blocks(rows, cap, row_bytes);
#define BUTLER_FT(PPR)                                                                       \
  if (row_bytes == PPR * 16) {                                                               \
    hipLaunchKernelGGL(fetch_rows_kernel<PPR>, dim3((unsigned)blocks), dim3(kFtThreads), 0, s, \
                       idx, count, (const uint4*)k, (const uint4*)v, (uint4*)k_sel,          \
                       (uint4*)v_sel, rows, kvdiv, L_cap, cap);                              \
    return hipGetLastError();                                                                \
  }
  BUTLER_FT(8) BUTLER_FT(16) BUTLER_FT(32)
#undef BUTLER_FT
  return hipErrorInvalidValue;
}

}  // namespace butler
