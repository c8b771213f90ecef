// K_imp = K . W_K for cached key rows [pos0, pos0 + n_new) of every (b, KV head).
// TokenButler model card, Method: post-RoPE keys projected to d' by a learned D x d'
// matrix, appended once per generated token.
//
// Few rows (decode appends): one thread per output element (row, j).  W_K (at most
// 128 x 32) lives in LDS as
// float; a key row is read in 16-byte chunks that the DP threads of a row share
// (same address -> one request).  Products and sums run in float64, where every
// partial sum of bf16 x bf16 products is exact, and the result is rounded once into
// the storage type -- K_imp is the correctly rounded K . W_K.
#include <type_traits>

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


// Bulk rows (prefill, set-up; bf16): the same exact dot products on the matrix cores,
// v_mfma_f64_16x16x4f64 over 16 key rows x 16 outputs (A lane l = K[row l%16][d],
// B lane l = W_K[d][col l%16], accumulator r of lane l = row 4r + l/16, col l%16).  The
// d index is permuted so that lane group g4 = l/16 feeds d = (D/4) g4 + s at step s: a
// lane reads its row's D/4 consecutive elements with 16-byte loads, and keeps its W_K
// column slice in VGPRs for the whole sweep.  Every product and partial sum is exact in
// float64, so the order of the MFMA accumulation gives the same bits as the oracle.
typedef __attribute__((ext_vector_type(4))) double f64x4p_t;

template <int D, int DP>
__global__ __launch_bounds__(256) void project_keys_mfma_kernel(const bf16_t* __restrict__ k,
                                                                const bf16_t* __restrict__ w,
                                                                bf16_t* __restrict__ kimp,
                                                                int L_cap, int pos0, int n_new,
                                                                long long rows_total) {
  constexpr int S = D / 4;      // MFMA steps per 16-row tile (d values per lane group)
  constexpr int JT = DP / 16;   // 16-column tiles
  const int lane = threadIdx.x & 63;
  const int ql = lane & 15, g4 = lane >> 4;
  // this lane's W_K slice: W_K[S*g4 + s][16 jt + ql]
  float wv[JT][S];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int st = 0; st < S; ++st) wv[jt][st] = bf2f(w[(S * g4 + st) * DP + 16 * jt + ql]);
  const long long nwaves = (long long)gridDim.x * 4;
  for (long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); tile * 16 < rows_total;
       tile += nwaves) {
    // A operand: key row tile*16 + ql (clamped), elements S*g4 .. S*g4 + S
    const long long ra = min(tile * 16 + ql, rows_total - 1);
    const long long bga = ra / n_new, ta = pos0 + ra % n_new;
    const bf16_t* kr = k + (bga * L_cap + ta) * D + S * g4;
    float kv[S];
#pragma unroll
    for (int c = 0; c < S / 8; ++c) Vec16<bf16_t>::load(kr + 8 * c, kv + 8 * c);
    f64x4p_t acc[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[jt] = f64x4p_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
        acc[jt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kv[st], (double)wv[jt][st],
                                                       acc[jt], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const long long row = tile * 16 + 4 * r + g4;
      if (row >= rows_total) continue;
      const long long bg = row / n_new, t = pos0 + row % n_new;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
        kimp[(bg * L_cap + t) * DP + 16 * jt + ql] = d2bf(acc[jt][r]);
    }
  }
}

template <typename T, int D, int DP>
hipError_t launch_t(hipStream_t s, const void* k, const void* w, void* kimp, int B, int Hkv,
                    int L_cap, int pos0, int n_new) {
  const long long rows = (long long)B * Hkv * n_new;
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (n_new >= 16) {
      long long blocks = (rows / 16 + 3) / 4;   // four 16-row tiles per workgroup
      if (blocks > 4096) blocks = 4096;
      if (blocks < 1) blocks = 1;
      hipLaunchKernelGGL((project_keys_mfma_kernel<D, DP>), dim3((unsigned)blocks), dim3(256), 0,
                         s, (const bf16_t*)k, (const bf16_t*)w, (bf16_t*)kimp, L_cap, pos0,
                         n_new, rows);
      return hipGetLastError();
    }
  }
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
