// K_imp = K . W_K for cached key rows [pos0, pos0 + n_new) of every (b, KV head).
// TokenButler model card, Method: post-RoPE keys projected to d' by a learned D x d'
// matrix, appended once per generated token.
//
// One thread per output element (row, j).  W_K (at most 128 x 32) lives in LDS as
// float; a key row is read in 16-byte chunks that the DP threads of a row share
// (same address -> one request).  bf16 rows accumulate in float32 (the products of
// two bf16 values are exact in float32), float32 rows in float64; the result is
// rounded once into the storage type.
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

template <typename T> struct Acc { using type = float; };
template <> struct Acc<float> { using type = double; };

__device__ __forceinline__ void store_elem(bf16_t* p, float v) { *p = f2bf(v); }
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
  for (int i = threadIdx.x; i < D * DP; i += 256) wsh[i] = load_elem(w + i);
  __syncthreads();
  const int j = threadIdx.x % DP;
  const int rsub = threadIdx.x / DP;
  for (long long row = (long long)blockIdx.x * RPB + rsub; row < rows_total;
       row += (long long)gridDim.x * RPB) {
    const long long bg = row / n_new;
    const long long t = pos0 + row % n_new;
    const T* kr = k + (bg * L_cap + t) * D;
    A acc = 0;
#pragma unroll 4
    for (int c = 0; c < D / EPL; ++c) {
      float kv[EPL];
      Vec16<T>::load(kr + c * EPL, kv);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc += (A)kv[e] * (A)wsh[(c * EPL + e) * DP + j];
    }
    store_elem(kimp + (bg * L_cap + t) * DP + j, acc);
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
