// Producer f_theta at a producer layer (TokenButler model card, Method):
//   Q_imp = relu(LN(H) . W1^T) . W2^T, reshaped to [B, Hq, G, Lq, d'].
// The weights come in the [out, in] layout of a PyTorch Linear (W1 [F, E], W2 [N2, F]),
// K-contiguous like the activations, so both MFMA operands read eight consecutive K
// values per lane straight from the same kind of LDS tile, and a GEMV reads whole weight
// rows with 16-byte loads.
// Steps: (1) LN rows -> bf16 x_hat; (2) GEMM x_hat . W1^T split over K into float32
// partial sums; (3) fixed-order reduction of the partials + ReLU -> bf16 a;
// (4) GEMM a . W2^T; (5) reduction + bf16 store scattered into the Q_imp layout.
// With one split the epilogue runs inside the GEMM.
//
// GEMM kernels.  Blocks of rows (prefill: M = B*Lq >= 64) run on the matrix cores: a
// 128 x 128 tile per workgroup, 64 x 64 per wave as 2 x 2 v_mfma_f32_32x32x16_bf16 tiles,
// K staged through LDS 64 at a time.  gemm_dma_kernel (every shape whose operands fit
// 32-bit byte offsets) loads each stage straight into LDS with buffer loads, in a ring of
// two stages (two workgroups per CU), takes its tile from an XCD-aware order, and keeps
// the accumulators transposed so its epilogue packs four columns per LDS write;
// gemm_mfma_kernel (the rest) stages through registers.  bf16 results leave through an
// LDS stage as 16-byte row chunks (contiguous in both the row-major activation and the
// Q_imp layout).  Other shapes with more than 4 rows take the VALU kernel -- 32 rows x 64
// columns per workgroup, a thread owns 1 row x 8 columns.  Up to 4 rows (decode: one
// hidden state per sequence) take a weight-streaming GEMV instead (below).
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr int kLnThreads = 256;
constexpr int kTM = 32, kTN = 64, kTK = 32;
constexpr int kGemmThreads = 256;

// Two floats -> two bf16 (rounded to nearest even) in one 32-bit word, low half first:
// the hardware's packed conversion.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2v_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

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
      ow[e] = pack_bf16x2((hv[u][2 * e] - mean) * rstd, (hv[u][2 * e + 1] - mean) * rstd);
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
    // B tile: 32 K x 64 columns from the [N, K] weights, 8 K values (16 bytes) per thread
    {
      const int bn = threadIdx.x / 4, bk = (threadIdx.x % 4) * 8;
      const int gk = kk + bk;
      float tmp[8];
      if (gk + 8 <= k1) {
        Vec16<bf16_t>::load(Bm + (long long)(n0 + bn) * K + gk, tmp);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          tmp[j] = (gk + j < k1) ? bf2f(Bm[(long long)(n0 + bn) * K + gk + j]) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) Bs[bk + j][bn] = tmp[j];
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

constexpr int kMM = 128, kMN = 128;
constexpr int kMThreads = 256;

// 128 x 128 tiles, 64 x 64 per wave as 2 x 2 v_mfma_f32_32x32x16_bf16 tiles.  K is staged
// through LDS 64 at a time, double-buffered, with two register stages so the next tile
// is in flight from memory while one is multiplied (16 MFMAs per wave between barriers;
// a ring of four stages measured slower).
// LDS rows of 72 bf16 (144 B) keep the 16-byte operand reads of 16 consecutive rows on
// distinct banks.  bf16 results leave through an LDS stage in 16-byte row chunks.
#ifndef BUTLER_GEMM_STAGES
#define BUTLER_GEMM_STAGES 2
#endif
constexpr int kM2K = 64;
constexpr int kM2St = BUTLER_GEMM_STAGES;   // register stages of the K loop (2 or 4)
static_assert(kM2St == 2 || kM2St == 4, "stage ring");
constexpr int kA2S = kM2K + 8;

__global__ __launch_bounds__(kMThreads) void gemm_mfma_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bm, void* out, int M, int N, int K,
    int k_per_split, Epilogue ep) {
  const int n0 = blockIdx.x * kMN, m0 = blockIdx.y * kMM, split = blockIdx.z;
  const int k0 = split * k_per_split, k1 = min(K, k0 + k_per_split);
  __shared__ __align__(16) bf16_t As[2][kMM * kA2S];
  __shared__ __align__(16) bf16_t Bs[2][kMN * kA2S];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  // staging roles, the same for both operands: chunk c = tid + 256 i (i < 4) is tile row
  // c / 8, K columns 8 (c % 8) .. +8
  const int r0 = tid >> 3, kc = (tid & 7) * 8;   // rows r0 + 32 i
  // rows past M: computed on clamped addresses, never stored
  const bf16_t* ap = A + (long long)min(m0 + r0, M - 1) * K + kc;
  const bf16_t* ap1 = A + (long long)min(m0 + r0 + 32, M - 1) * K + kc;
  const bf16_t* ap2 = A + (long long)min(m0 + r0 + 64, M - 1) * K + kc;
  const bf16_t* ap3 = A + (long long)min(m0 + r0 + 96, M - 1) * K + kc;
  const bf16_t* bp = Bm + (long long)(n0 + r0) * K + kc;
  const long long b_step = (long long)32 * K;
  const int lo = r0 * kA2S + kc, lo_step = 32 * kA2S;
  uint4 ra0_0, ra1_0, ra2_0, ra3_0, rb0_0, rb1_0, rb2_0, rb3_0;
  uint4 ra0_1, ra1_1, ra2_1, ra3_1, rb0_1, rb1_1, rb2_1, rb3_1;
  uint4 ra0_2, ra1_2, ra2_2, ra3_2, rb0_2, rb1_2, rb2_2, rb3_2;
  uint4 ra0_3, ra1_3, ra2_3, ra3_3, rb0_3, rb1_3, rb2_3, rb3_3;
#define BUTLER_GLOAD(st, kk)                                                     \
  do {                                                                           \
    ra0_##st = *reinterpret_cast<const uint4*>(ap + (kk));                      \
    ra1_##st = *reinterpret_cast<const uint4*>(ap1 + (kk));                     \
    ra2_##st = *reinterpret_cast<const uint4*>(ap2 + (kk));                     \
    ra3_##st = *reinterpret_cast<const uint4*>(ap3 + (kk));                     \
    rb0_##st = *reinterpret_cast<const uint4*>(bp + (kk));                      \
    rb1_##st = *reinterpret_cast<const uint4*>(bp + b_step + (kk));             \
    rb2_##st = *reinterpret_cast<const uint4*>(bp + 2 * b_step + (kk));         \
    rb3_##st = *reinterpret_cast<const uint4*>(bp + 3 * b_step + (kk));         \
  } while (0)
#define BUTLER_LSTORE(st, buf)                                                   \
  do {                                                                           \
    *reinterpret_cast<uint4*>(&As[buf][lo]) = ra0_##st;                         \
    *reinterpret_cast<uint4*>(&As[buf][lo + lo_step]) = ra1_##st;               \
    *reinterpret_cast<uint4*>(&As[buf][lo + 2 * lo_step]) = ra2_##st;           \
    *reinterpret_cast<uint4*>(&As[buf][lo + 3 * lo_step]) = ra3_##st;           \
    *reinterpret_cast<uint4*>(&Bs[buf][lo]) = rb0_##st;                         \
    *reinterpret_cast<uint4*>(&Bs[buf][lo + lo_step]) = rb1_##st;               \
    *reinterpret_cast<uint4*>(&Bs[buf][lo + 2 * lo_step]) = rb2_##st;           \
    *reinterpret_cast<uint4*>(&Bs[buf][lo + 3 * lo_step]) = rb3_##st;           \
  } while (0)
  f32x16v_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int T = (k1 - k0) / kM2K;   // a multiple of kM2St (checked on the host)
  BUTLER_GLOAD(0, k0);
  BUTLER_GLOAD(1, k0 + min(1, T - 1) * kM2K);
  if constexpr (kM2St == 4) {
    BUTLER_GLOAD(2, k0 + min(2, T - 1) * kM2K);
    BUTLER_GLOAD(3, k0 + min(3, T - 1) * kM2K);
  }
  BUTLER_LSTORE(0, 0);
  __syncthreads();
  const int lr = lane & 31, lk = 8 * (lane >> 5);
#define BUTLER_MMA(buf)                                                                      \
  do {                                                                                       \
    _Pragma("unroll") for (int ks = 0; ks < kM2K / 16; ++ks) {                               \
      bf16x8v_t a[2], b[2];                                                                  \
      _Pragma("unroll") for (int i = 0; i < 2; ++i)                                          \
        a[i] = *reinterpret_cast<const bf16x8v_t*>(&As[buf][(wm * 64 + i * 32 + lr) * kA2S + ks * 16 + lk]); \
      _Pragma("unroll") for (int j = 0; j < 2; ++j)                                          \
        b[j] = *reinterpret_cast<const bf16x8v_t*>(&Bs[buf][(wn * 64 + j * 32 + lr) * kA2S + ks * 16 + lk]); \
      _Pragma("unroll") for (int i = 0; i < 2; ++i)                                          \
        _Pragma("unroll") for (int j = 0; j < 2; ++j)                                        \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0); \
    }                                                                                        \
  } while (0)
  // tile t: multiply from LDS buffer t % 2, store tile t+1 (register stage (t+1) % kM2St)
  // into the other buffer (past the end: written, never read), refill stage t % kM2St with
  // tile t + kM2St
#define BUTLER_STEP(st, nx)                                                       \
  do {                                                                            \
    BUTLER_MMA((st) & 1);                                                         \
    BUTLER_LSTORE(nx, ((st) & 1) ^ 1);                                            \
    BUTLER_GLOAD(st, k0 + min(t0 + (st) + kM2St, T - 1) * kM2K);                  \
    __syncthreads();                                                              \
  } while (0)
  for (int t0 = 0; t0 < T; t0 += kM2St) {
    if constexpr (kM2St == 4) {
      BUTLER_STEP(0, 1);
      BUTLER_STEP(1, 2);
      BUTLER_STEP(2, 3);
      BUTLER_STEP(3, 0);
    } else {
      BUTLER_STEP(0, 1);
      BUTLER_STEP(1, 0);
    }
  }
#undef BUTLER_STEP
#undef BUTLER_MMA
#undef BUTLER_GLOAD
#undef BUTLER_LSTORE
  // accumulator r of tile (i, j): row 8(r/4) + 4(lane/32) + r%4, column lane%32
  if (ep.mode == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int n = n0 + wn * 64 + j * 32 + lr;
          if (m < M) ((float*)out)[((long long)split * M + m) * N + n] = acc[i][j][r];
        }
    return;
  }
  // bf16 results go through LDS so every lane stores 16 contiguous bytes: the tile in
  // [128][136] bf16 over the (now idle) A buffers, then 8 consecutive columns per chunk,
  // which stay inside one (head, slot) run of d' values in the Q_imp layout
  constexpr int CS = kMN + 8;
  bf16_t* Cs = &As[0][0];
  static_assert(kMM * CS <= 2 * kMM * kA2S, "output stage fits the A buffers");
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float v = (ep.mode == 1) ? fmaxf(acc[i][j][r], 0.f) : acc[i][j][r];
        Cs[rr * CS + wn * 64 + j * 32 + lr] = f2bf(v);
      }
  __syncthreads();
  const int cc = tid & 15;   // 16-byte chunk of the row: columns 8 cc .. 8 cc + 7
#pragma unroll
  for (int i = 0; i < kMM / 16; ++i) {
    const int rr = (tid >> 4) + 16 * i;
    const int m = m0 + rr;
    if (m >= M) continue;
    const uint4 val = *reinterpret_cast<const uint4*>(&Cs[rr * CS + 8 * cc]);
    const int n = n0 + 8 * cc;
    bf16_t* dst;
    if (ep.mode == 1) {
      dst = (bf16_t*)out + (long long)m * N + n;
    } else {
      // column n = (head*G + slot)*dp + i, row m = b*Lq + t
      const int b = m / ep.Lq, t = m - b * ep.Lq;
      const int head = n / (ep.G * ep.dp);
      const int rem = n - head * ep.G * ep.dp;
      const int slot = rem / ep.dp, i0 = rem - slot * ep.dp;
      dst = (bf16_t*)out + ((((long long)b * ep.Hq + head) * ep.G + slot) * ep.Lq + t) * ep.dp + i0;
    }
    *reinterpret_cast<uint4*>(dst) = val;
  }
}

// The same tiles and wave layout fed by LDS-direct buffer loads: each stage of 64 K values
// (16 KB of A, 16 KB of B) goes from memory straight into LDS (buffer_load_dwordx4 ... lds,
// no VGPR staging, no LDS store instructions), S stages in a ring, so S - 1 stages are in
// flight while one is multiplied; one barrier per stage.  A wave's load writes 1 KB of LDS
// in lane order: eight tile rows of 128 bytes.  The lane picks which 16-byte chunk of its
// row it fetches so that chunk c of tile row r sits in slot c ^ ((r >> 1) & 7): the
// operand reads of 16 consecutive rows (one LDS cycle of a 16-byte read) then hit 16
// distinct 16-byte bank groups.  Rows past M are read clamped and never stored.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kDK = 64;                                 // K per stage
constexpr int kDTile = kMM * kDK * 2;                   // bytes of one operand tile
constexpr int kDLoads = kDTile / (kMThreads * 16);      // 16-byte loads per lane and operand
static_assert(2 * kDLoads == 8, "wait_vm counts a stage as eight loads per lane");

// s_waitcnt bounding only the vector-memory counter (expcnt, lgkmcnt left at their maximum)
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// s_waitcnt lgkmcnt(0) alone: this wave's LDS accesses have completed
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// wait until at most n_left (0, 8 or 16: whole stages) of this wave's loads are in flight
__device__ __forceinline__ void wait_vm(int n_left) {
  if (n_left >= 16) wait_vm_n<16>();
  else if (n_left >= 8) wait_vm_n<8>();
  else wait_vm_n<0>();
}

// Which tile a workgroup takes.  Workgroup w runs on XCD w % 8, and each XCD has its own
// L2: with xcd set, the XCDs split the (split, row block, column tile) space into 8
// rectangles of xs x xm x xn, and XCD x takes every tile of rectangle x, so its L2 fetches
// only those rows of A and of B (for the producer at 2048 rows: 6 MB per XCD instead of
// nearly all 25 MB).
struct TileMap {
  int nm, nn, ns;    // row blocks, column tiles, K splits
  int xm, xn, xs;    // how the 8 XCDs divide each (xcd != 0)
  int xcd;
};

__device__ __forceinline__ void tile_of(const TileMap& t, int w, int& mb, int& nb, int& s) {
  if (!t.xcd) {
    nb = w % t.nn;
    mb = (w / t.nn) % t.nm;
    s = w / (t.nn * t.nm);
    return;
  }
  const int x = w & 7, j = w >> 3;
  const int rn = t.nn / t.xn, rm = t.nm / t.xm, rs = t.ns / t.xs;
  nb = (x % t.xn) * rn + j % rn;
  mb = ((x / t.xn) % t.xm) * rm + (j / rn) % rm;
  s = (x / (t.xn * t.xm)) * rs + j / (rn * rm);
}

template <int S>
__global__ __launch_bounds__(kMThreads) void gemm_dma_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bm, void* out, int M, int N, int K,
    int k_per_split, Epilogue ep, TileMap tm) {
  static_assert(S >= 2 && S <= 4, "stage ring");
  __shared__ __align__(16) unsigned char sm[S * 2 * kDTile];
  int mb, nb, split;
  tile_of(tm, blockIdx.x, mb, nb, split);
  const int n0 = nb * kMN, m0 = mb * kMM;
  const int k0 = split * k_per_split;
  const int T = k_per_split / kDK;   // >= S - 1 (checked on the host)
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, M * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)Bm, (short)0, N * K * 2, 0x00020000);
  // load j of this lane: tile row 32 wid + 8 j + lane / 8, slot lane % 8
  int va[kDLoads], vb[kDLoads];
#pragma unroll
  for (int j = 0; j < kDLoads; ++j) {
    const int r = 32 * wid + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    va[j] = (min(m0 + r, M - 1) * K + 8 * c) * 2;
    vb[j] = ((n0 + r) * K + 8 * c) * 2;
  }
  lds_void_t* lds = (lds_void_t*)sm;
  const auto issue = [&](int t) {
    const int so = (k0 + t * kDK) * 2;
    unsigned char* base = sm + (t % S) * 2 * kDTile + wid * (kDLoads * 1024);
#pragma unroll
    for (int j = 0; j < kDLoads; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(base + j * 1024), 16, va[j], so, 0, 0);
#pragma unroll
    for (int j = 0; j < kDLoads; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(base + kDTile + j * 1024), 16, vb[j], so, 0, 0);
  };
  (void)lds;
  // operand reads: tile row (wm or wn) * 64 + 32 i + lane % 32, logical chunk 2 ks + lane / 32
  const int f = (lane >> 1) & 7, h = lane >> 5;
  int rowa[2], rowb[2], slot[kDK / 16];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    rowa[i] = (wm * 64 + i * 32 + (lane & 31)) * 128;
    rowb[i] = kDTile + (wn * 64 + i * 32 + (lane & 31)) * 128;
  }
#pragma unroll
  for (int ks = 0; ks < kDK / 16; ++ks) slot[ks] = 16 * ((2 * ks + h) ^ f);
  f32x16v_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);
  for (int t = 0; t < T; ++t) {
    // this wave's loads of stage t have landed once at most the later stages' are left
    wait_vm(min(S - 2, T - 1 - t) * 2 * kDLoads);
    // every wave's stage t is in LDS and every wave is done with stage t-1.  __syncthreads
    // would also wait for the later stages' loads (its fence covers the LDS-direct writes),
    // so: this wave's LDS reads completed, then the hardware barrier between two compiler
    // barriers, so no LDS access moves across it.
    wait_lds();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + S - 1 < T) issue(t + S - 1);
    const unsigned char* st = sm + (t % S) * 2 * kDTile;
#pragma unroll
    for (int ks = 0; ks < kDK / 16; ++ks) {
      bf16x8v_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const bf16x8v_t*>(st + rowa[i] + slot[ks]);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const bf16x8v_t*>(st + rowb[j] + slot[ks]);
      // weights as the first operand: the accumulators hold C^T, so a lane's four
      // consecutive accumulators are four consecutive output columns of one row
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
    // the next k-step's four operands read ahead of this k-step's four products
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int ks = 0; ks < kDK / 16 - 1; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
  // accumulator r of tile (i, j): row m0 + 64 wm + 32 i + lane % 32, column
  // n0 + 64 wn + 32 j + 8 (r / 4) + 4 (lane / 32) + r % 4
  const int lr = lane & 31, h4 = 4 * (lane >> 5);
  if (ep.mode == 0) {
    float* P = (float*)out + (long long)split * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = m0 + wm * 64 + i * 32 + lr;
      if (m >= M) continue;
      float* prow = P + (long long)m * N + n0 + wn * 64 + h4;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(prow + j * 32 + 8 * g) =
              make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                          acc[i][j][4 * g + 3]);
    }
    return;
  }
  // bf16 results through LDS ([128][136] over the ring, 8-byte writes of four columns),
  // then 16-byte row chunks to memory
  constexpr int CS = kMN + 8;
  bf16_t* Cs = reinterpret_cast<bf16_t*>(sm);
  static_assert(kMM * CS * 2 <= S * 2 * kDTile, "output stage fits the ring");
  __syncthreads();   // every wave is done reading the last stage
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (ep.mode == 1) ? fmaxf(acc[i][j][4 * g + e], 0.f) : acc[i][j][4 * g + e];
        *reinterpret_cast<uint2*>(&Cs[(wm * 64 + i * 32 + lr) * CS + wn * 64 + j * 32 + 8 * g + h4]) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
  __syncthreads();
  const int cc = tid & 15;   // this thread's 16-byte chunk: columns n0 + 8 cc .. + 7
  const int r0 = tid >> 4;   // rows r0 + 16 i
  const int n = n0 + 8 * cc;
  if (ep.mode == 1) {
#pragma unroll
    for (int i = 0; i < kMM / 16; ++i) {
      const int m = m0 + r0 + 16 * i;
      if (m >= M) break;
      *reinterpret_cast<uint4*>((bf16_t*)out + (long long)m * N + n) =
          *reinterpret_cast<const uint4*>(&Cs[(r0 + 16 * i) * CS + 8 * cc]);
    }
    return;
  }
  // Q_imp layout: column n = (head G + slot) d' + i0, row m = b Lq + t; the chunk stays
  // inside one (head, slot) run.  The column part is fixed per thread; (b, t) steps by 16
  // rows at a time.
  const int head = n / (ep.G * ep.dp);
  const int rem = n - head * ep.G * ep.dp;
  const int slot2 = rem / ep.dp, i0 = rem - slot2 * ep.dp;
  int bb = (m0 + r0) / ep.Lq, tt = (m0 + r0) - bb * ep.Lq;
#pragma unroll
  for (int i = 0; i < kMM / 16; ++i) {
    const int m = m0 + r0 + 16 * i;
    if (m >= M) break;
    bf16_t* dst = (bf16_t*)out +
                  ((((long long)bb * ep.Hq + head) * ep.G + slot2) * ep.Lq + tt) * ep.dp + i0;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&Cs[(r0 + 16 * i) * CS + 8 * cc]);
    tt += 16;
    while (tt >= ep.Lq) {
      tt -= ep.Lq;
      ++bb;
    }
  }
}

constexpr int kMGran = kM2St * kM2K;   // K granule of a split

#ifndef BUTLER_GEMM_DMA_STAGES
#define BUTLER_GEMM_DMA_STAGES 2
#endif
constexpr int kDStages = BUTLER_GEMM_DMA_STAGES;   // 0: register-staged kernel only
constexpr int kDRing = kDStages >= 2 ? kDStages : 2;   // the LDS-direct kernel's ring

// The LDS-direct kernel addresses its operands with 32-bit byte offsets and needs at least
// S - 1 stages of K in a split.
bool use_dma(int M, int N, int K, int kps) {
  return kDStages >= 2 && (long long)M * K * 2 < (1LL << 31) &&
         (long long)N * K * 2 < (1LL << 31) && kps % kDK == 0 && kps / kDK >= kDStages - 1;
}

// The XCD split of the tiles with the least L2 fill: per XCD, its splits' share of K times
// (row blocks + column tiles) of its rectangle.  Without a split into 8 equal rectangles,
// the plain order.
TileMap tile_map(int nm, int nn, int ns) {
  TileMap best{nm, nn, ns, 1, 1, 1, 0};
  long long best_cost = -1;
  for (int xs = 1; xs <= 8; xs *= 2)
    for (int xm = 1; xs * xm <= 8; xm *= 2) {
      const int xn = 8 / (xs * xm);
      if (ns % xs || nm % xm || nn % xn) continue;
      const long long cost = (long long)(ns / xs) * (nm / xm + nn / xn);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best = TileMap{nm, nn, ns, xm, xn, xs, 1};
      }
    }
  return best;
}

bool use_mfma(int M, int N, int K) {
  return M >= 64 && N % kMN == 0 && K % kMGran == 0;
}

int mfma_splits(int M, int N, int K) {
  const int tiles = ((M + kMM - 1) / kMM) * (N / kMN);
  int s = 1;
  while (tiles * s < 256 && K / (s * 2) >= 512 && (K / (s * 2)) % kMGran == 0) s *= 2;
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

// The same eight columns at a time (N and d' are multiples of 8, so the eight share a row
// and a (head, slot) run of the Q_imp layout): 32-byte partial loads per split, summed in
// the same order, and one 16-byte store.
__global__ void reduce_splits8_kernel(const float* __restrict__ P, void* out, int M, int N,
                                      int nsplit, Epilogue ep) {
  const long long e = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (e >= (long long)M * N) return;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* ps = P + (long long)s * M * N + e;
    const float4 a = *reinterpret_cast<const float4*>(ps);
    const float4 b = *reinterpret_cast<const float4*>(ps + 4);
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
  if (ep.mode == 1)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = fmaxf(acc[c], 0.f);
  const uint4 o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                             pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  const int m = (int)(e / N), n = (int)(e - (long long)m * N);
  bf16_t* dst;
  if (ep.mode == 1) {
    dst = (bf16_t*)out + e;
  } else {
    const int b = m / ep.Lq, t = m - b * ep.Lq;
    const int head = n / (ep.G * ep.dp);
    const int rem = n - head * ep.G * ep.dp;
    const int slot = rem / ep.dp, i = rem - slot * ep.dp;
    dst = (bf16_t*)out + ((((long long)b * ep.Hq + head) * ep.G + slot) * ep.Lq + t) * ep.dp + i;
  }
  *reinterpret_cast<uint4*>(dst) = o;
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
  const int kt = mf ? kMGran : kTK;
  const int kps = ((K / ns) + kt - 1) / kt * kt;
  Epilogue pe = ep;
  if (ns > 1) pe.mode = 0;
  void* dst = (ns > 1) ? (void*)partial : out;
  if (mf) {
    dim3 grid(N / kMN, (M + kMM - 1) / kMM, ns);
    if (use_dma(M, N, K, kps)) {
      const TileMap tm = tile_map((M + kMM - 1) / kMM, N / kMN, ns);
      const unsigned nwg = (unsigned)grid.x * grid.y * grid.z;
      hipLaunchKernelGGL(gemm_dma_kernel<kDRing>, dim3(nwg),
                         dim3(kMThreads), 0, st, A, Bm, dst, M, N, K, kps, pe, tm);
    } else
      hipLaunchKernelGGL(gemm_mfma_kernel, grid, dim3(kMThreads), 0, st, A, Bm, dst, M, N, K,
                         kps, pe);
  } else {
    dim3 grid(N / kTN, (M + kTM - 1) / kTM, ns);
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(kGemmThreads), 0, st, A, Bm, dst, M, N, K,
                       kps, pe);
  }
  if (ns > 1) {
    const long long tot = (long long)M * N;
    if (N % 8 == 0 && (ep.mode != 2 || ep.dp % 8 == 0))
      hipLaunchKernelGGL(reduce_splits8_kernel, dim3((unsigned)((tot / 8 + 255) / 256)), dim3(256),
                         0, st, partial, out, M, N, ns, ep);
    else
      hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0,
                         st, partial, out, M, N, ns, ep);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// decode rows (M <= 4): weight-streaming GEMV in two kernels
// ---------------------------------------------------------------------------
//   1  every workgroup normalises the M rows itself (LN statistics over E, then bf16
//      x_hat into LDS) while its weight rows are in flight; a wave owns one row n of W1
//      (K-contiguous: lane l reads K values 8l + 512j .. +8 with 16-byte loads, all issued
//      first), dots it with the M rows, reduces across the wave, applies ReLU and writes
//      the bf16 activation a[m][n];
//   2  the same for W2 over the activations, the results rounded to bf16 and scattered
//      into the Q_imp layout.
// The weights stream from HBM once and no partial sums leave a wave.

constexpr int kGvThreads = 256;     // 4 waves, one weight row each
constexpr int kGvRows = kGvThreads / 64;
constexpr int kGvMaxM = 4;
constexpr int kGvMaxK = 8192;

// Loads of weight row n (K-contiguous), NL 16-byte pieces per lane; pieces past K read
// the row's last piece and are dropped in gv_dot.
template <int NL>
__device__ __forceinline__ void gv_load(uint4 (&wv)[NL], const bf16_t* __restrict__ W, int n,
                                        int K, int lane) {
  const bf16_t* wr = W + (long long)n * K;
#pragma unroll
  for (int j = 0; j < NL; ++j) wv[j] = *reinterpret_cast<const uint4*>(wr + min(8 * lane + 512 * j, K - 8));
}

// The M dot products of the held weight row with the bf16 rows xs[m][0..K) in LDS, summed
// across the wave (every lane gets the sums).
template <int NL>
__device__ __forceinline__ void gv_dot(const uint4 (&wv)[NL], const bf16_t* xs, int M, int K,
                                       int lane, float (&acc)[kGvMaxM]) {
#pragma unroll
  for (int m = 0; m < kGvMaxM; ++m) acc[m] = 0.f;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int k = 8 * lane + 512 * j;
    if (k >= K) continue;
    Raw16 r;
    r.v = wv[j];
    float wf[8];
    unpack16<bf16_t>(r, wf);
#pragma unroll
    for (int m = 0; m < kGvMaxM; ++m) {
      if (m >= M) break;
      Raw16 xr;
      xr.v = *reinterpret_cast<const uint4*>(xs + m * K + k);
      float xf[8];
      unpack16<bf16_t>(xr, xf);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[m] = fmaf(xf[e], wf[e], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < kGvMaxM; ++m)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc[m] += __shfl_xor(acc[m], o, 64);
}

template <int NL>
__global__ __launch_bounds__(kGvThreads) void gemv_ln_w1_kernel(const bf16_t* __restrict__ h,
                                                                 const bf16_t* __restrict__ W,
                                                                 bf16_t* __restrict__ act, int M,
                                                                 int K, int N, float eps) {
  extern __shared__ __align__(16) bf16_t xs[];   // [M][K]
  __shared__ float tmp[kGvThreads / 64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = min(blockIdx.x * kGvRows + wid, N - 1);
  uint4 wv[NL];
  gv_load<NL>(wv, W, n, K, lane);
  for (int m = 0; m < M; ++m) {
    // the row is held in registers: 16-byte pieces, all requested before the reductions
    const bf16_t* hr = h + (long long)m * K;
    constexpr int kPieces = kGvMaxK / (kGvThreads * 8);
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
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const int e0 = (threadIdx.x + kGvThreads * u) * 8;
      if (e0 >= K) continue;
      uint4 o;
      uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ow[e] = (uint32_t)f2bf((hv[u][2 * e] - mean) * rstd) |
                ((uint32_t)f2bf((hv[u][2 * e + 1] - mean) * rstd) << 16);
      *reinterpret_cast<uint4*>(xs + m * K + e0) = o;
    }
  }
  __syncthreads();
  float acc[kGvMaxM];
  gv_dot<NL>(wv, xs, M, K, lane, acc);
  const int nn = blockIdx.x * kGvRows + wid;
  if (lane < M && nn < N) {
    float a = acc[0];
#pragma unroll
    for (int m = 1; m < kGvMaxM; ++m) a = (lane == m) ? acc[m] : a;
    act[(long long)lane * N + nn] = f2bf(fmaxf(a, 0.f));
  }
}

template <int NL>
__global__ __launch_bounds__(kGvThreads) void gemv_w2_kernel(const bf16_t* __restrict__ act,
                                                             const bf16_t* __restrict__ W,
                                                             bf16_t* q_imp, int M, int K, int N,
                                                             Epilogue ep) {
  extern __shared__ __align__(16) bf16_t xs[];   // [M][K]
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = min(blockIdx.x * kGvRows + wid, N - 1);
  uint4 wv[NL];
  gv_load<NL>(wv, W, n, K, lane);
  for (int e0 = threadIdx.x * 8; e0 < M * K; e0 += kGvThreads * 8)
    *reinterpret_cast<uint4*>(xs + e0) = *reinterpret_cast<const uint4*>(act + e0);
  __syncthreads();
  float acc[kGvMaxM];
  gv_dot<NL>(wv, xs, M, K, lane, acc);
  const int nn = blockIdx.x * kGvRows + wid;
  if (lane < M && nn < N) {
    float a = acc[0];
#pragma unroll
    for (int m = 1; m < kGvMaxM; ++m) a = (lane == m) ? acc[m] : a;
    store_out(ep, q_imp, M, N, lane, nn, a);
  }
}

bool use_gemv(int M, int E, int F, int N2) {
  (void)N2;
  return M <= kGvMaxM && E <= kGvMaxK && F <= kGvMaxK && E % 8 == 0 && F % 8 == 0;
}

// 16-byte pieces per lane for a row of K elements, rounded up to a launched instance
int gv_loads(int K) {
  const int nl = (K + 511) / 512;
  return nl <= 2 ? 2 : nl <= 4 ? 4 : nl <= 8 ? 8 : 16;
}

}  // namespace

size_t produce_workspace(int M, int E, int F, int N2) {
  if (use_gemv(M, E, F, N2)) return align256((size_t)M * F * 2);
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
    bf16_t* act = (bf16_t*)ws;
    const Epilogue e2{2, Lq, Hq, G, dp};
#define BUTLER_GV1(NL)                                                                       \
  hipLaunchKernelGGL(gemv_ln_w1_kernel<NL>, dim3((F + kGvRows - 1) / kGvRows), dim3(kGvThreads), \
                     (size_t)M * E * 2, s, (const bf16_t*)h, (const bf16_t*)w1, act, M, E, F, eps)
#define BUTLER_GV2(NL)                                                                       \
  hipLaunchKernelGGL(gemv_w2_kernel<NL>, dim3((N2 + kGvRows - 1) / kGvRows), dim3(kGvThreads), \
                     (size_t)M * F * 2, s, (const bf16_t*)act, (const bf16_t*)w2, (bf16_t*)q_imp, M, F, \
                     N2, e2)
    switch (gv_loads(E)) {
      case 2: BUTLER_GV1(2); break;
      case 4: BUTLER_GV1(4); break;
      case 8: BUTLER_GV1(8); break;
      default: BUTLER_GV1(16); break;
    }
    switch (gv_loads(F)) {
      case 2: BUTLER_GV2(2); break;
      case 4: BUTLER_GV2(4); break;
      case 8: BUTLER_GV2(8); break;
      default: BUTLER_GV2(16); break;
    }
#undef BUTLER_GV1
#undef BUTLER_GV2
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
