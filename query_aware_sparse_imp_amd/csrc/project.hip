// K_imp = K . W_K for cached key rows [pos0, pos0 + n_new) of every (b, KV head).
// TokenButler model card, Method: post-RoPE keys projected to d' by a learned D x d'
// matrix, appended once per generated token.
//
// One thread per output element (row, j).  W_K (at most 128 x 32) lives in LDS as
// float; a key row is read in 16-byte chunks that the DP threads of a row share
// (same address -> one request).  Products and sums run in float64, where every
// partial sum of bf16 x bf16 products is exact, and the result is rounded once into
// the storage type -- K_imp is the correctly rounded K . W_K.
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

template <typename T> struct Acc { using type = double; };

__device__ __forceinline__ void store_elem(bf16_t* p, double v) { *p = d2bf(v); }
__device__ __forceinline__ void store_elem(float* p, double v) { *p = (float)v; }

template <typename T, int D, int DP>
__global__ __launch_bounds__(256) void project_keys_kernel(const T* __restrict__ k,
                                                           const T* __restrict__ w,
                                                           T* __restrict__ kimp, int L_cap,
                                                           int pos0, int n_new,
                                                           long long rows_total) {
  using A = typename Acc<T>::type;
  constexpr int EPL = Vec16<T>::N;
  constexpr int RPB = 256 / DP;
  __shared__ float wsh[D * DP];
  const int j = threadIdx.x % DP;
  const int rsub = threadIdx.x / DP;
  const long long stride = (long long)gridDim.x * RPB;
  long long row = (long long)blockIdx.x * RPB + rsub;
  // the first key row is requested before W_K is staged, so both round trips overlap
  float kv[D / EPL][EPL];
  auto load_row = [&](long long rw) {
    const long long bg = rw / n_new, t = pos0 + rw % n_new;
    const T* kr = k + (bg * L_cap + t) * D;
#pragma unroll
    for (int c = 0; c < D / EPL; ++c) Vec16<T>::load(kr + c * EPL, kv[c]);
  };
  if (row < rows_total) load_row(row);
  // W_K in 16-byte pieces, all issued before any is used
  {
    constexpr int EPL16 = Vec16<T>::N;
    constexpr int NPIECE = D * DP / EPL16;
    constexpr int PER = (NPIECE + 255) / 256;
    float wv[PER][EPL16];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int pc = threadIdx.x + u * 256;
      if (pc < NPIECE) Vec16<T>::load(w + pc * EPL16, wv[u]);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int pc = threadIdx.x + u * 256;
      if (pc < NPIECE) {
#pragma unroll
        for (int e = 0; e < EPL16; ++e) wsh[pc * EPL16 + e] = wv[u][e];
      }
    }
  }
  __syncthreads();
  while (row < rows_total) {
    // four independent float64 sums (every partial sum is exact, so their order does not
    // change the result)
    A acc4[4] = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < D / EPL; ++c) {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        acc4[c & 3] = fma((A)kv[c][e], (A)wsh[(c * EPL + e) * DP + j], acc4[c & 3]);
    }
    const A acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    const long long bg = row / n_new, t = pos0 + row % n_new;
    store_elem(kimp + (bg * L_cap + t) * DP + j, acc);
    row += stride;
    if (row < rows_total) load_row(row);
  }
}

template <typename T, int D, int DP>
hipError_t launch_t(hipStream_t s, const void* k, const void* w, void* kimp, int B, int Hkv,
                    int L_cap, int pos0, int n_new) {
  const long long rows = (long long)B * Hkv * n_new;
  constexpr int RPB = 256 / DP;
  long long blocks = (rows + RPB - 1) / RPB;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((project_keys_kernel<T, D, DP>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (const T*)k, (const T*)w, (T*)kimp, L_cap, pos0, n_new, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_project_keys(hipStream_t s, int dtype, const void* k, const void* w,
                               void* kimp, int B, int Hkv, int L_cap, int D, int dp,
                               int pos0, int n_new) {
#define BUTLER_PROJ(T, DD, PP)                                                     \
  if (D == DD && dp == PP)                                                         \
    return launch_t<T, DD, PP>(s, k, w, kimp, B, Hkv, L_cap, pos0, n_new);
  if (dtype == 1) {
    BUTLER_PROJ(bf16_t, 128, 32) BUTLER_PROJ(bf16_t, 128, 16)
    BUTLER_PROJ(bf16_t, 64, 32) BUTLER_PROJ(bf16_t, 64, 16)
  } else {
    BUTLER_PROJ(float, 128, 32) BUTLER_PROJ(float, 128, 16)
    BUTLER_PROJ(float, 64, 32) BUTLER_PROJ(float, 64, 16)
  }
#undef BUTLER_PROJ
  return hipErrorInvalidValue;
}

}  // namespace butler
