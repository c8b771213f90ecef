// Producer f_theta at a producer layer (TokenButler model card, Method):
//   Q_imp = relu(LN(H) . W1) . W2, reshaped to [B, Hq, G, Lq, d'].
// Steps: (1) LN rows -> bf16 x_hat; (2) GEMM x_hat . W1 split over K into float32
// partial sums; (3) fixed-order reduction of the partials + ReLU -> bf16 a;
// (4) GEMM a . W2; (5) reduction + bf16 store scattered into the Q_imp layout.
// With one split the epilogue runs inside the GEMM.
//
// Two GEMM kernels.  Blocks of rows (prefill: M = B*Lq >= 64) run on the matrix cores:
// a 128 x 128 tile per workgroup, 64 x 64 per wave as 2 x 2 v_mfma_f32_32x32x16_bf16
// tiles, K staged through LDS 32 at a time, double-buffered, with a ring of four
// register stages so three K tiles are in flight from memory.  The MFMA wants eight
// consecutive K values per lane for both operands; the activations are K-contiguous, the
// weights [K, N] are N-contiguous, so the weight tile is transposed on its way into LDS:
// two K rows are packed into one 32-bit word per column.  A few rows (decode: one
// hidden state per sequence) take the VALU kernel -- 32 rows x 64 columns per workgroup,
// a thread owns 1 row x 8 columns -- since there the weights stream once from HBM and
// the matrix cores would idle.  Up to 4 rows take a weight-streaming GEMV instead (below).
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr int kLnThreads = 256;
constexpr int kTM = 32, kTN = 64, kTK = 32;
constexpr int kGemmThreads = 256;

// One row per workgroup: the row is held in VGPRs (16-byte pieces, all requested before
// the first reduction), mean and variance from block sums, then the bf16 x_hat.
__global__ __launch_bounds__(kLnThreads) void ln_rows_kernel(const bf16_t* __restrict__ h,
                                                             bf16_t* __restrict__ xhat, int E,
                                                             float eps) {
  constexpr int kPieces = 4;   // rows up to 256 * 8 * 4 = 8192 elements
  const long long row = blockIdx.x;
  const bf16_t* hr = h + row * E;
  __shared__ float tmp[kLnThreads / 64];
  float hv[kPieces][8];
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int e0 = (threadIdx.x + kLnThreads * u) * 8;
    if (e0 < E) {
      Vec16<bf16_t>::load(hr + e0, hv[u]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[u][e] = 0.f;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kPieces; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += hv[u][e];
  const float mean = block_sum_f<kLnThreads>(s, tmp) / (float)E;
  float v = 0.f;
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    if ((threadIdx.x + kLnThreads * u) * 8 >= E) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = hv[u][e] - mean;
      v = fmaf(d, d, v);
    }
  }
  const float var = block_sum_f<kLnThreads>(v, tmp) / (float)E;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int e0 = (threadIdx.x + kLnThreads * u) * 8;
    if (e0 >= E) continue;
    uint4 o;
    uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ow[e] = (uint32_t)f2bf((hv[u][2 * e] - mean) * rstd) |
              ((uint32_t)f2bf((hv[u][2 * e + 1] - mean) * rstd) << 16);
    *reinterpret_cast<uint4*>(xhat + row * E + e0) = o;
  }
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


// ---------------------------------------------------------------------------
// matrix-core GEMM
// ---------------------------------------------------------------------------

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8v_t;
typedef __attribute__((ext_vector_type(16))) float f32x16v_t;

constexpr int kMM = 128, kMN = 128, kMK = 32;
constexpr int kMThreads = 256;
constexpr int kMPf = 4;        // register stages of the K loop (even: LDS buffers alternate)
constexpr int kAS = kMK + 8;   // LDS row stride in bf16 of the A tile and the transposed B tile

__global__ __launch_bounds__(kMThreads) void gemm_mfma_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bm, void* out, int M, int N, int K,
    int k_per_split, Epilogue ep) {
  const int n0 = blockIdx.x * kMN, m0 = blockIdx.y * kMM, split = blockIdx.z;
  const int k0 = split * k_per_split, k1 = min(K, k0 + k_per_split);
  __shared__ __align__(16) bf16_t As[2][kMM * kAS];
  __shared__ __align__(16) bf16_t Bt[2][kMN * kAS];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  // staging roles: A chunks c = tid, tid + 256 are row c/4, K columns 8*(c%4) .. +8; for B
  // the thread takes K rows 2p, 2p+1 and columns 8g .. 8g+7 of the tile
  const int p = tid & 15, g = tid >> 4;
  const int c0 = tid, c1 = tid + kMThreads;
  const bf16_t* a0 = A + (long long)min(m0 + (c0 >> 2), M - 1) * K + (c0 & 3) * 8;
  const bf16_t* a1 = A + (long long)min(m0 + (c1 >> 2), M - 1) * K + (c1 & 3) * 8;  // rows past M: computed, never stored
  const bf16_t* bp = Bm + (long long)(2 * p) * N + n0 + 8 * g;
  const int as0 = (c0 >> 2) * kAS + (c0 & 3) * 8, as1 = (c1 >> 2) * kAS + (c1 & 3) * 8;
  // a ring of kMPf = 4 register stages: tiles t+1 .. t+3 are in flight from memory while
  // tile t is multiplied; every load is unconditional (the ring runs past the last tile on
  // clamped addresses), so each wait is for exactly one stage
  uint4 ra0_0, ra1_0, rb0_0, rb1_0, ra0_1, ra1_1, rb0_1, rb1_1;
  uint4 ra0_2, ra1_2, rb0_2, rb1_2, ra0_3, ra1_3, rb0_3, rb1_3;
#define BUTLER_GLOAD(st, kk)                                                     \
  do {                                                                           \
    ra0_##st = *reinterpret_cast<const uint4*>(a0 + (kk));                      \
    ra1_##st = *reinterpret_cast<const uint4*>(a1 + (kk));                      \
    rb0_##st = *reinterpret_cast<const uint4*>(bp + (long long)(kk) * N);       \
    rb1_##st = *reinterpret_cast<const uint4*>(bp + (long long)(kk) * N + N);   \
  } while (0)
  // column 8g+2q gets the low halves of both K rows, column 8g+2q+1 the high halves
#define BUTLER_PACK(q, x0, x1)                                                   \
  bw[(8 * g + 2 * (q)) * (kAS / 2) + p] = ((x0) & 0xffffu) | ((x1) << 16);      \
  bw[(8 * g + 2 * (q) + 1) * (kAS / 2) + p] = ((x0) >> 16) | ((x1) & 0xffff0000u)
#define BUTLER_LSTORE(st, buf)                                                   \
  do {                                                                           \
    *reinterpret_cast<uint4*>(&As[buf][as0]) = ra0_##st;                        \
    *reinterpret_cast<uint4*>(&As[buf][as1]) = ra1_##st;                        \
    uint32_t* bw = reinterpret_cast<uint32_t*>(Bt[buf]);                        \
    BUTLER_PACK(0, rb0_##st.x, rb1_##st.x);                                      \
    BUTLER_PACK(1, rb0_##st.y, rb1_##st.y);                                      \
    BUTLER_PACK(2, rb0_##st.z, rb1_##st.z);                                      \
    BUTLER_PACK(3, rb0_##st.w, rb1_##st.w);                                      \
  } while (0)
  f32x16v_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int T = (k1 - k0) / kMK;   // a multiple of kMPf (checked on the host)
  BUTLER_GLOAD(0, k0);
  BUTLER_GLOAD(1, k0 + min(1, T - 1) * kMK);
  BUTLER_GLOAD(2, k0 + min(2, T - 1) * kMK);
  BUTLER_GLOAD(3, k0 + min(3, T - 1) * kMK);
  BUTLER_LSTORE(0, 0);
  __syncthreads();
  const int lr = lane & 31, lk = 8 * (lane >> 5);
  auto mma = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kMK / 16; ++ks) {
      bf16x8v_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8v_t*>(&As[buf][(wm * 64 + i * 32 + lr) * kAS + ks * 16 + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8v_t*>(&Bt[buf][(wn * 64 + j * 32 + lr) * kAS + ks * 16 + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  // tile t: multiply from LDS buffer t % 2, store tile t+1 (register stage (t+1) % 4) into
  // the other buffer (past the end: written, never read), refill stage t % 4 with tile t+4
#define BUTLER_STEP(st, nx)                                                       \
  do {                                                                            \
    mma((st) & 1);                                                                \
    BUTLER_LSTORE(nx, ((st) & 1) ^ 1);                                            \
    BUTLER_GLOAD(st, k0 + min(t0 + (st) + kMPf, T - 1) * kMK);                    \
    __syncthreads();                                                              \
  } while (0)
  for (int t0 = 0; t0 < T; t0 += kMPf) {
    BUTLER_STEP(0, 1);
    BUTLER_STEP(1, 2);
    BUTLER_STEP(2, 3);
    BUTLER_STEP(3, 0);
  }
#undef BUTLER_STEP
#undef BUTLER_GLOAD
#undef BUTLER_PACK
#undef BUTLER_LSTORE
  // accumulator r of tile (i, j): row 8(r/4) + 4(lane/32) + r%4, column lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int n = n0 + wn * 64 + j * 32 + lr;
        if (m >= M) continue;
        if (ep.mode == 0) ((float*)out)[((long long)split * M + m) * N + n] = acc[i][j][r];
        else store_out(ep, out, M, N, m, n, acc[i][j][r]);
      }
}

bool use_mfma(int M, int N, int K) {
  return M >= 64 && N % kMN == 0 && K % (kMK * kMPf) == 0;
}

int mfma_splits(int M, int N, int K) {
  const int tiles = ((M + kMM - 1) / kMM) * (N / kMN);
  int s = 1;
  while (tiles * s < 256 && K / (s * 2) >= 512 && (K / (s * 2)) % (kMK * kMPf) == 0) s *= 2;
  return s;
}

__global__ void reduce_splits_kernel(const float* __restrict__ P, void* out, int M, int N,
                                     int nsplit, Epilogue ep) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long long)M * N) return;
  float acc = 0.f;
  for (int s = 0; s < nsplit; ++s) acc += P[(long long)s * M * N + e];
  store_out(ep, out, M, N, (int)(e / N), (int)(e % N), acc);
}

int valu_splits(int M, int N, int K) {
  const int tiles = ((M + kTM - 1) / kTM) * (N / kTN);
  int s = 1;
  while (tiles * s < 512 && K / (s * 2) >= 256) s *= 2;
  return s;
}

int splits_for(int M, int N, int K) {
  return use_mfma(M, N, K) ? mfma_splits(M, N, K) : valu_splits(M, N, K);
}

hipError_t gemm(hipStream_t st, const bf16_t* A, const bf16_t* Bm, void* out, float* partial,
                int M, int N, int K, Epilogue ep) {
  const bool mf = use_mfma(M, N, K);
  const int ns = splits_for(M, N, K);
  const int kt = mf ? kMK : kTK;
  const int kps = ((K / ns) + kt - 1) / kt * kt;
  Epilogue pe = ep;
  if (ns > 1) pe.mode = 0;
  void* dst = (ns > 1) ? (void*)partial : out;
  if (mf) {
    dim3 grid(N / kMN, (M + kMM - 1) / kMM, ns);
    hipLaunchKernelGGL(gemm_mfma_kernel, grid, dim3(kMThreads), 0, st, A, Bm, dst, M, N, K, kps,
                       pe);
  } else {
    dim3 grid(N / kTN, (M + kTM - 1) / kTM, ns);
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(kGemmThreads), 0, st, A, Bm, dst, M, N, K,
                       kps, pe);
  }
  if (ns > 1) {
    const long long tot = (long long)M * N;
    hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0,
                       st, partial, out, M, N, ns, ep);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// decode rows (M <= 4): weight-streaming GEMV in three kernels
// ---------------------------------------------------------------------------
//   1  every workgroup normalises the M rows itself (LN statistics over E, then the bf16
//      x_hat of its 64-row K slice), multiplies its slice of W1 (64 K rows x 256 columns,
//      16-byte loads, all issued first) and writes float32 partial sums per K slice;
//   2  every workgroup sums the first layer's partials of its K slice in slice order,
//      applies ReLU and the bf16 rounding, and multiplies its slice of W2 the same way;
//   3  the second layer's partials are summed in slice order, rounded to bf16 and
//      scattered into the Q_imp layout.
// The weights stream from HBM once; everything else is small and stays in L2.

constexpr int kGvThreads = 256;
constexpr int kGvCols = 256;      // columns per workgroup: 32 groups of 8
constexpr int kGvK = 64;          // K rows per workgroup: 8 per thread row
constexpr int kGvMaxM = 4;

// x (float, the M rows of this K slice, in LDS) times W[k0 .. k0+64, n0 .. n0+256):
// float32 partials to part[slice][m][n].
__device__ __forceinline__ void gemv_slice(const float (*xs)[kGvK], const uint4 (&wv)[kGvK / 8],
                                           float* __restrict__ part, int M, int N, int n0,
                                           int slice, float* red) {
  const int cg = threadIdx.x & 31, kr = threadIdx.x >> 5;
  float acc[kGvMaxM][8];
#pragma unroll
  for (int m = 0; m < kGvMaxM; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;
#pragma unroll
  for (int j = 0; j < kGvK / 8; ++j) {
    Raw16 r;
    r.v = wv[j];
    float wf[8];
    unpack16<bf16_t>(r, wf);
#pragma unroll
    for (int m = 0; m < kGvMaxM; ++m) {
      if (m >= M) break;
      const float x = xs[m][kr + 8 * j];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[m][e] = fmaf(x, wf[e], acc[m][e]);
    }
  }
  // the 8 thread rows meet in LDS, summed in row order
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[kr * kGvCols + cg * 8 + e] = acc[m][e];
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) s += red[q * kGvCols + threadIdx.x];
    part[((long long)slice * M + m) * N + n0 + threadIdx.x] = s;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kGvThreads) void gemv_ln_w1_kernel(const bf16_t* __restrict__ h,
                                                                 const bf16_t* __restrict__ W,
                                                                 float* __restrict__ part, int M,
                                                                 int K, int N, float eps) {
  const int n0 = blockIdx.x * kGvCols, slice = blockIdx.y, k0 = slice * kGvK;
  const int cg = threadIdx.x & 31, kr = threadIdx.x >> 5;
  uint4 wv[kGvK / 8];
#pragma unroll
  for (int j = 0; j < kGvK / 8; ++j)
    wv[j] = *reinterpret_cast<const uint4*>(W + (long long)(k0 + kr + 8 * j) * N + n0 + 8 * cg);
  __shared__ float xs[kGvMaxM][kGvK];
  __shared__ float red[8 * kGvCols];
  __shared__ float tmp[kGvThreads / 64];
  for (int m = 0; m < M; ++m) {
    // the row is held in registers: 16-byte pieces, all requested before the reductions
    const bf16_t* hr = h + (long long)m * K;
    constexpr int kPieces = 4;   // rows up to 256 * 8 * 4 = 8192 elements
    float hv[kPieces][8];
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const int e0 = (threadIdx.x + kGvThreads * u) * 8;
      if (e0 < K) {
        Vec16<bf16_t>::load(hr + e0, hv[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[u][e] = 0.f;
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < kPieces; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += hv[u][e];
    const float mean = block_sum_f<kGvThreads>(sum, tmp) / (float)K;
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      if ((threadIdx.x + kGvThreads * u) * 8 >= K) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = hv[u][e] - mean;
        v = fmaf(d, d, v);
      }
    }
    const float rstd = 1.0f / sqrtf(block_sum_f<kGvThreads>(v, tmp) / (float)K + eps);
    if (threadIdx.x < kGvK) xs[m][threadIdx.x] = bf2f(f2bf((bf2f(hr[k0 + threadIdx.x]) - mean) * rstd));
  }
  __syncthreads();
  gemv_slice(xs, wv, part, M, N, n0, slice, red);
}

__global__ __launch_bounds__(kGvThreads) void gemv_relu_w2_kernel(const float* __restrict__ part1,
                                                                   int nslice1,
                                                                   const bf16_t* __restrict__ W,
                                                                   float* __restrict__ part, int M,
                                                                   int K, int N) {
  const int n0 = blockIdx.x * kGvCols, slice = blockIdx.y, k0 = slice * kGvK;
  const int cg = threadIdx.x & 31, kr = threadIdx.x >> 5;
  uint4 wv[kGvK / 8];
#pragma unroll
  for (int j = 0; j < kGvK / 8; ++j)
    wv[j] = *reinterpret_cast<const uint4*>(W + (long long)(k0 + kr + 8 * j) * N + n0 + 8 * cg);
  __shared__ float xs[kGvMaxM][kGvK];
  __shared__ float red[8 * kGvCols];
  // first-layer activations of this K slice: partials summed in slice order, ReLU, bf16
  const int m = threadIdx.x / kGvK, kk = threadIdx.x % kGvK;
  if (m < M) {
    float a = 0.f;
    for (int s0 = 0; s0 < nslice1; s0 += 16) {
      float pv[16];   // sixteen slices requested at once, summed in slice order
#pragma unroll
      for (int u = 0; u < 16; ++u)
        pv[u] = part1[((long long)min(s0 + u, nslice1 - 1) * M + m) * K + k0 + kk];
#pragma unroll
      for (int u = 0; u < 16; ++u) a += (s0 + u < nslice1) ? pv[u] : 0.f;
    }
    xs[m][kk] = bf2f(f2bf(fmaxf(a, 0.f)));
  }
  __syncthreads();
  gemv_slice(xs, wv, part, M, N, n0, slice, red);
}

__global__ void gemv_out_kernel(const float* __restrict__ part2, int nslice2, bf16_t* q_imp,
                                int M, int N, Epilogue ep) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long long)M * N) return;
  const int m = (int)(e / N), n = (int)(e % N);
  float a = 0.f;
  for (int s0 = 0; s0 < nslice2; s0 += 16) {
    float pv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) pv[u] = part2[((long long)min(s0 + u, nslice2 - 1) * M + m) * N + n];
#pragma unroll
    for (int u = 0; u < 16; ++u) a += (s0 + u < nslice2) ? pv[u] : 0.f;
  }
  store_out(ep, q_imp, M, N, m, n, a);
}

bool use_gemv(int M, int E, int F, int N2) {
  return M <= kGvMaxM && E <= kGvThreads * 8 * 4 && E % 8 == 0 && E % kGvK == 0 && F % kGvK == 0 && F % kGvCols == 0 &&
         N2 % kGvCols == 0;
}


}  // namespace

size_t produce_workspace(int M, int E, int F, int N2) {
  if (use_gemv(M, E, F, N2))
    return align256((size_t)(E / kGvK) * M * F * 4) + align256((size_t)(F / kGvK) * M * N2 * 4);
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
  if (use_gemv(M, E, F, N2)) {
    float* p1 = (float*)ws;
    float* p2 = (float*)((char*)ws + align256((size_t)(E / kGvK) * M * F * 4));
    hipLaunchKernelGGL(gemv_ln_w1_kernel, dim3(F / kGvCols, E / kGvK), dim3(kGvThreads), 0, s,
                       (const bf16_t*)h, (const bf16_t*)w1, p1, M, E, F, eps);
    hipLaunchKernelGGL(gemv_relu_w2_kernel, dim3(N2 / kGvCols, F / kGvK), dim3(kGvThreads), 0, s,
                       (const float*)p1, E / kGvK, (const bf16_t*)w2, p2, M, F, N2);
    const long long tot = (long long)M * N2;
    hipLaunchKernelGGL(gemv_out_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s,
                       (const float*)p2, F / kGvK, (bf16_t*)q_imp, M, N2,
                       Epilogue{2, Lq, Hq, G, dp});
    return hipGetLastError();
  }
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
