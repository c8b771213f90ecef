// Producer f_theta at a producer layer (TokenButler model card, Method):
//   Q_imp = relu(LN(H) . W1) . W2, reshaped to [B, Hq, G, Lq, d'].
// Steps: (1) LN rows -> bf16 x_hat; (2) GEMM x_hat . W1 split over K into float32
// partial sums; (3) fixed-order reduction of the partials + ReLU -> bf16 a;
// (4) GEMM a . W2; (5) reduction + bf16 store scattered into the Q_imp layout.
// With one split the epilogue runs inside the GEMM.  The GEMM tile is 32 rows x 64
// columns, K staged through LDS 32 at a time; a thread owns 1 row x 8 columns.
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr int kLnThreads = 256;
constexpr int kTM = 32, kTN = 64, kTK = 32;
constexpr int kGemmThreads = 256;

__global__ __launch_bounds__(kLnThreads) void ln_rows_kernel(const bf16_t* __restrict__ h,
                                                             bf16_t* __restrict__ xhat, int E,
                                                             float eps) {
  const long long row = blockIdx.x;
  const bf16_t* hr = h + row * E;
  __shared__ float tmp[kLnThreads / 64];
  float s = 0.f;
  for (int j = threadIdx.x; j < E; j += kLnThreads) s += bf2f(hr[j]);
  const float mean = block_sum_f<kLnThreads>(s, tmp) / (float)E;
  float v = 0.f;
  for (int j = threadIdx.x; j < E; j += kLnThreads) {
    const float d = bf2f(hr[j]) - mean;
    v = fmaf(d, d, v);
  }
  const float var = block_sum_f<kLnThreads>(v, tmp) / (float)E;
  const float rstd = 1.0f / sqrtf(var + eps);
  for (int j = threadIdx.x; j < E; j += kLnThreads)
    xhat[row * E + j] = f2bf((bf2f(hr[j]) - mean) * rstd);
}

// Output placement of GEMM results.
struct Epilogue {
  int mode;   // 0: float32 partial [split][M][N]; 1: relu + bf16 row-major; 2: bf16 Q_imp scatter
  int Lq, Hq, G, dp;
};

__device__ __forceinline__ void store_out(const Epilogue& ep, void* out, int M, int N, int m,
                                          int n, float acc) {
  if (ep.mode == 1) {
    ((bf16_t*)out)[(long long)m * N + n] = f2bf(fmaxf(acc, 0.f));
  } else {
    // column n = (head*G + slot)*dp + i, row m = b*Lq + t
    const int b = m / ep.Lq, t = m - b * ep.Lq;
    const int head = n / (ep.G * ep.dp);
    const int rem = n - head * ep.G * ep.dp;
    const int slot = rem / ep.dp, i = rem - slot * ep.dp;
    ((bf16_t*)out)[((((long long)b * ep.Hq + head) * ep.G + slot) * ep.Lq + t) * ep.dp + i] =
        f2bf(acc);
  }
}

__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bm, void* out, int M, int N, int K,
    int k_per_split, Epilogue ep) {
  const int n0 = blockIdx.x * kTN, m0 = blockIdx.y * kTM, split = blockIdx.z;
  const int k0 = split * k_per_split, k1 = min(K, k0 + k_per_split);
  __shared__ float As[kTM][kTK + 1];
  __shared__ float Bs[kTK][kTN];
  const int r = threadIdx.x / 8, c = (threadIdx.x % 8) * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int kk = k0; kk < k1; kk += kTK) {
    // A tile: 32 x 32, 4 elements per thread
    for (int e = threadIdx.x; e < kTM * kTK; e += kGemmThreads) {
      const int ar = e / kTK, ac = e % kTK;
      const int gm = m0 + ar, gk = kk + ac;
      As[ar][ac] = (gm < M && gk < k1) ? bf2f(A[(long long)gm * K + gk]) : 0.f;
    }
    // B tile: 32 x 64, 8 elements (16 bytes) per thread
    {
      const int br = threadIdx.x / 8, bc = (threadIdx.x % 8) * 8;
      const int gk = kk + br;
      float tmp[8];
      if (gk < k1) {
        Vec16<bf16_t>::load(Bm + (long long)gk * N + n0 + bc, tmp);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) tmp[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) Bs[br][bc + j] = tmp[j];
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < kTK; ++k) {
      const float a = As[r][k];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(a, Bs[k][c + j], acc[j]);
    }
    __syncthreads();
  }
  const int m = m0 + r;
  if (m >= M) return;
  if (ep.mode == 0) {
    float* P = (float*)out + ((long long)split * M + m) * N + n0 + c;
#pragma unroll
    for (int j = 0; j < 8; ++j) P[j] = acc[j];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) store_out(ep, out, M, N, m, n0 + c + j, acc[j]);
  }
}

__global__ void reduce_splits_kernel(const float* __restrict__ P, void* out, int M, int N,
                                     int nsplit, Epilogue ep) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long long)M * N) return;
  float acc = 0.f;
  for (int s = 0; s < nsplit; ++s) acc += P[(long long)s * M * N + e];
  store_out(ep, out, M, N, (int)(e / N), (int)(e % N), acc);
}

int splits_for(int M, int N, int K) {
  const int tiles = ((M + kTM - 1) / kTM) * (N / kTN);
  int s = 1;
  while (tiles * s < 512 && K / (s * 2) >= 256) s *= 2;
  return s;
}

hipError_t gemm(hipStream_t st, const bf16_t* A, const bf16_t* Bm, void* out, float* partial,
                int M, int N, int K, Epilogue ep) {
  const int ns = splits_for(M, N, K);
  const int kps = ((K / ns) + kTK - 1) / kTK * kTK;
  dim3 grid(N / kTN, (M + kTM - 1) / kTM, ns);
  if (ns == 1) {
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(kGemmThreads), 0, st, A, Bm, out, M, N, K,
                       kps, ep);
  } else {
    Epilogue pe = ep;
    pe.mode = 0;
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(kGemmThreads), 0, st, A, Bm, (void*)partial,
                       M, N, K, kps, pe);
    const long long tot = (long long)M * N;
    hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0,
                       st, partial, out, M, N, ns, ep);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t produce_workspace(int M, int E, int F, int N2) {
  const size_t xs = align256((size_t)M * E * 2);
  const size_t as = align256((size_t)M * F * 2);
  const size_t p1 = (size_t)splits_for(M, F, E) * M * F * 4;
  const size_t p2 = (size_t)splits_for(M, N2, F) * M * N2 * 4;
  const size_t need_p1 = splits_for(M, F, E) > 1 ? p1 : 0;
  const size_t need_p2 = splits_for(M, N2, F) > 1 ? p2 : 0;
  return xs + as + align256(need_p1 > need_p2 ? need_p1 : need_p2);
}

hipError_t launch_produce(hipStream_t s, const void* h, const void* w1, const void* w2,
                          void* q_imp, int B, int Lq, int E, int F, int Hq, int G, int dp,
                          float eps, void* ws) {
  const int M = B * Lq, N2 = Hq * G * dp;
  bf16_t* xhat = (bf16_t*)ws;
  bf16_t* act = (bf16_t*)((char*)ws + align256((size_t)M * E * 2));
  float* partial = (float*)((char*)act + align256((size_t)M * F * 2));
  hipLaunchKernelGGL(ln_rows_kernel, dim3(M), dim3(kLnThreads), 0, s, (const bf16_t*)h, xhat, E,
                     eps);
  Epilogue e1{1, Lq, Hq, G, dp};
  hipError_t err = gemm(s, xhat, (const bf16_t*)w1, act, partial, M, F, E, e1);
  if (err != hipSuccess) return err;
  Epilogue e2{2, Lq, Hq, G, dp};
  return gemm(s, act, (const bf16_t*)w2, q_imp, partial, M, N2, F, e2);
}

}  // namespace butler
