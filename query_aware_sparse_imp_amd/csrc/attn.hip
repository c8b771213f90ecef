// Attention over the selected tokens only (TokenButler model card, intro and Method:
// the full KV cache is kept, each step attends to the selected subset).
//
// Decode (index lists): split-K flash decoding.  The selected list of one (b, KV
// head, query row) is cut into slices of kTokensPerSplit positions, one workgroup per
// slice.  Inside a workgroup D/8 lanes cover one 2*D-byte key row (16 bytes each), so
// a wave gathers 64/(D/8) selected rows per load instruction, straight into VGPRs;
// all R query heads of the GQA group are served by the same gathered rows.  Logits,
// the online softmax (base 2) and the P.V accumulation run in float32.  Each slice
// writes (max, sum, acc[D]) per head; the workgroup that finishes last (an atomic
// ticket per row) merges the slices in slice order and writes the output, then resets
// its ticket to zero for the next call.
//
// Prefill (bitmask rows): one workgroup per query row expands the row's bitmask into
// an ascending LDS index list and runs the same gather loop over it.
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kTokensPerSplit = 256;
constexpr int kAttnUnroll = 4;
constexpr int kMaxBitmaskL = 16384;

template <typename T, int D, int R>
struct Geo {
  static constexpr int EPL = Vec16<T>::N;   // elements per lane
  static constexpr int LPR = D / EPL;       // lanes per key row
  static constexpr int TPW = 64 / LPR;      // rows per wave step
};

// Online-softmax state of R heads for this lane's slice of D.
template <int R, int EPL>
struct SoftState {
  float m[R], l[R], acc[R][EPL];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      m[r] = neg_inf();
      l[r] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[r][e] = 0.f;
    }
  }
  // merge another state (m2, l2, a2) into this one
  __device__ __forceinline__ void merge(int r, float m2, float l2, const float* a2) {
    if (m2 == neg_inf()) return;
    const float mn = fmaxf(m[r], m2);
    const float a = (m[r] == neg_inf()) ? 0.f : fast_exp2(m[r] - mn);
    const float b = fast_exp2(m2 - mn);
    l[r] = l[r] * a + l2 * b;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[r][e] = acc[r][e] * a + a2[e] * b;
    m[r] = mn;
  }
};

// Processes list positions p = p0, p0 + stride, ... < p1 (this lane group's share).
template <typename T, int D, int R, typename ListT>
__device__ __forceinline__ void gather_attend(const T* __restrict__ kb, const T* __restrict__ vb,
                                              ListT list, int L_cap, int p0, int p1, int stride,
                                              const float (&qr)[R][Geo<T, D, R>::EPL],
                                              SoftState<R, Geo<T, D, R>::EPL>& st) {
  using G = Geo<T, D, R>;
  constexpr int EPL = G::EPL, LPR = G::LPR, U = kAttnUnroll;
  for (int p = p0; p < p1; p += stride * U) {
    float kv[U][EPL], vv[U][EPL];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pu = p + u * stride;
      ok[u] = pu < p1;
      if (ok[u]) {
        // indices outside [0, L_cap) never leave the cache (they read row L_cap - 1)
        const long long t = (long long)min((unsigned)list[pu], (unsigned)(L_cap - 1));
        Vec16<T>::load(kb + t * D, kv[u]);
        Vec16<T>::load(vb + t * D, vv[u]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) { kv[u][e] = 0.f; vv[u][e] = 0.f; }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float z[U];
      float mx = st.m[r];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaf(qr[r][e], kv[u][e], a);
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) a += __shfl_xor(a, o, 64);
        z[u] = ok[u] ? a : neg_inf();
        mx = fmaxf(mx, z[u]);
      }
      const float alpha = (st.m[r] == neg_inf()) ? 0.f : fast_exp2(st.m[r] - mx);
      st.l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) st.acc[r][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pz = ok[u] ? fast_exp2(z[u] - mx) : 0.f;
        st.l[r] += pz;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.acc[r][e] = fmaf(pz, vv[u][e], st.acc[r][e]);
      }
      st.m[r] = (mx == neg_inf()) ? st.m[r] : mx;
    }
  }
}

// Reduces the states of all lane groups of the block into LDS arrays
// red_m/red_l [R], red_acc [R][D] (valid after return, all threads synced).
template <typename T, int D, int R>
__device__ __forceinline__ void block_reduce_state(SoftState<R, Geo<T, D, R>::EPL>& st,
                                                   float* sm, float* sl, float* sacc,
                                                   float* red_m, float* red_l,
                                                   float* red_acc) {
  using G = Geo<T, D, R>;
  constexpr int EPL = G::EPL, LPR = G::LPR;
  constexpr int NW = kAttnThreads / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int pe = lane % LPR;
  // lane groups within the wave (same pe, different rows)
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(st.m[r], o, 64);
      const float l2 = __shfl_xor(st.l[r], o, 64);
      float a2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(st.acc[r][e], o, 64);
      // merge in a fixed order regardless of which lane holds which side
      SoftState<1, EPL> lo, hi;
      const bool mine_low = (lane & o) == 0;
      lo.m[0] = mine_low ? st.m[r] : m2;  lo.l[0] = mine_low ? st.l[r] : l2;
      hi.m[0] = mine_low ? m2 : st.m[r];  hi.l[0] = mine_low ? l2 : st.l[r];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        lo.acc[0][e] = mine_low ? st.acc[r][e] : a2[e];
        hi.acc[0][e] = mine_low ? a2[e] : st.acc[r][e];
      }
      lo.merge(0, hi.m[0], hi.l[0], hi.acc[0]);
      st.m[r] = lo.m[0];
      st.l[r] = lo.l[0];
#pragma unroll
      for (int e = 0; e < EPL; ++e) st.acc[r][e] = lo.acc[0][e];
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (pe == 0) { sm[wid * R + r] = st.m[r]; sl[wid * R + r] = st.l[r]; }
#pragma unroll
      for (int e = 0; e < EPL; ++e) sacc[(wid * R + r) * D + pe * EPL + e] = st.acc[r][e];
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < R * D; j += kAttnThreads) {
    const int r = j / D, d = j % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w * R + r]);
    float lsum = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm[w * R + r];
      const float f = (mw == neg_inf()) ? 0.f : fast_exp2(mw - M);
      lsum += sl[w * R + r] * f;
      a += sacc[(w * R + r) * D + d] * f;
    }
    red_acc[j] = a;
    if (d == 0) { red_m[r] = M; red_l[r] = lsum; }
  }
  __syncthreads();
}

template <typename T, int D, int R>
__device__ __forceinline__ void load_q(const T* q, long long qoff_head0, long long head_stride,
                                       int pe, float scale_log2,
                                       float (&qr)[R][Geo<T, D, R>::EPL]) {
  constexpr int EPL = Geo<T, D, R>::EPL;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float tmp[EPL];
    Vec16<T>::load(q + qoff_head0 + r * head_stride + pe * EPL, tmp);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[r][e] = tmp[e] * scale_log2;
  }
}

template <typename T, int D, int R>
__global__ __launch_bounds__(kAttnThreads) void attn_idx_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, float* __restrict__ out,
    float* __restrict__ part, int* __restrict__ tickets, int Hq, int Hkv, int Lq, int L_cap,
    int cap, float scale_log2, int nsplit) {
  using G = Geo<T, D, R>;
  constexpr int EPL = G::EPL, LPR = G::LPR, TPW = G::TPW;
  constexpr int NW = kAttnThreads / 64;
  const int row = blockIdx.y, split = blockIdx.x;
  const int bg = row / Lq, i = row - bg * Lq;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int sub = lane / LPR, pe = lane % LPR;

  float qr[R][EPL];
  load_q<T, D, R>(q, (((long long)b * Hq + g * R) * Lq + i) * D, (long long)Lq * D, pe,
                  scale_log2, qr);
  const int n = min(count[row], cap);
  const int p_start = split * kTokensPerSplit;
  const int p_end = min(p_start + kTokensPerSplit, n);
  SoftState<R, EPL> st;
  st.init();
  const T* kb = k + (long long)bg * L_cap * D + pe * EPL;
  const T* vb = v + (long long)bg * L_cap * D + pe * EPL;
  gather_attend<T, D, R>(kb, vb, idx + (long long)row * cap, L_cap, p_start + wid * TPW + sub, p_end,
                         NW * TPW, qr, st);

  __shared__ float sm[NW * R], sl[NW * R], sacc[NW * R * D];
  __shared__ float red_m[R], red_l[R], red_acc[R * D];
  block_reduce_state<T, D, R>(st, sm, sl, sacc, red_m, red_l, red_acc);

  float* my = part + ((long long)row * nsplit + split) * R * (D + 2);
  for (int j = threadIdx.x; j < R * D; j += kAttnThreads) my[(j / D) * (D + 2) + 2 + j % D] = red_acc[j];
  if (threadIdx.x < R) {
    my[threadIdx.x * (D + 2)] = red_m[threadIdx.x];
    my[threadIdx.x * (D + 2) + 1] = red_l[threadIdx.x];
  }
  __threadfence();
  __syncthreads();
  __shared__ int sh_last;
  if (threadIdx.x == 0) {
    const int t = __hip_atomic_fetch_add(&tickets[row], 1, __ATOMIC_ACQ_REL,
                                         __HIP_MEMORY_SCOPE_AGENT);
    sh_last = (t == nsplit - 1);
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();
  const float* base = part + (long long)row * nsplit * R * (D + 2);
  for (int j = threadIdx.x; j < R * D; j += kAttnThreads) {
    const int r = j / D, d = j % D;
    float M = neg_inf();
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, base[((long long)s * R + r) * (D + 2)]);
    float lsum = 0.f, a = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float* ps = base + ((long long)s * R + r) * (D + 2);
      const float f = (ps[0] == neg_inf()) ? 0.f : fast_exp2(ps[0] - M);
      lsum += ps[1] * f;
      a += ps[2 + d] * f;
    }
    out[(((long long)b * Hq + g * R + r) * Lq + i) * D + d] = (lsum > 0.f) ? a / lsum : 0.f;
  }
  if (threadIdx.x == 0) tickets[row] = 0;
}

// Bitmask rows: one workgroup per (b, KV head, query row).
template <typename T, int D, int R>
__global__ __launch_bounds__(kAttnThreads) void attn_bitmask_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const uint32_t* __restrict__ bitmask, float* __restrict__ out, int Hq, int Hkv, int Lq,
    int L, int L_cap, int q_pos0, float scale_log2) {
  using G = Geo<T, D, R>;
  constexpr int EPL = G::EPL, LPR = G::LPR, TPW = G::TPW;
  constexpr int NW = kAttnThreads / 64;
  const int row = blockIdx.x;
  const int bg = row / Lq, i = row - bg * Lq;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int sub = lane / LPR, pe = lane % LPR;
  const int nwords = (L + 31) / 32;
  const int L_r = min(q_pos0 + i + 1, L);
  const int nwords_act = (L_r + 31) / 32;
  __shared__ int list[kMaxBitmaskL];
  __shared__ int tmp[NW];
  const uint32_t* brow = bitmask + (long long)row * nwords;
  int carry = 0;
  for (int w0 = 0; w0 < nwords_act; w0 += kAttnThreads) {
    const int w = w0 + threadIdx.x;
    uint32_t bits = 0;
    if (w < nwords_act) {
      bits = brow[w];
      const int lim = L_r - w * 32;  // tokens after the row's own position never count
      if (lim < 32) bits &= (lim <= 0) ? 0u : ((1u << lim) - 1u);
    }
    int tot;
    int pos = carry + block_exclusive_sum<kAttnThreads>(__popc(bits), tot, tmp);
    for (uint32_t e = bits; e; e &= e - 1) list[pos++] = w * 32 + (__ffs(e) - 1);
    carry += tot;
  }
  __syncthreads();
  float qr[R][EPL];
  load_q<T, D, R>(q, (((long long)b * Hq + g * R) * Lq + i) * D, (long long)Lq * D, pe,
                  scale_log2, qr);
  SoftState<R, EPL> st;
  st.init();
  const T* kb = k + (long long)bg * L_cap * D + pe * EPL;
  const T* vb = v + (long long)bg * L_cap * D + pe * EPL;
  gather_attend<T, D, R>(kb, vb, (const int*)list, L_cap, wid * TPW + sub, carry, NW * TPW, qr, st);
  __shared__ float sm[NW * R], sl[NW * R], sacc[NW * R * D];
  __shared__ float red_m[R], red_l[R], red_acc[R * D];
  block_reduce_state<T, D, R>(st, sm, sl, sacc, red_m, red_l, red_acc);
  for (int j = threadIdx.x; j < R * D; j += kAttnThreads) {
    const int r = j / D, d = j % D;
    out[(((long long)b * Hq + g * R + r) * Lq + i) * D + d] =
        (red_l[r] > 0.f) ? red_acc[j] / red_l[r] : 0.f;
  }
}

int nsplit_for(int cap) { return (cap + kTokensPerSplit - 1) / kTokensPerSplit; }

template <typename T, int D, int R>
hipError_t idx_t(hipStream_t s, const void* q, const void* k, const void* v,
                 const int32_t* idx, const int32_t* count, float* out, int B, int Hq, int Hkv,
                 int Lq, int L_cap, int cap, float scale, void* ws) {
  const int nsplit = nsplit_for(cap);
  const long long rows = (long long)B * Hkv * Lq;
  int* tickets = (int*)ws;
  float* part = (float*)((char*)ws + ((rows * sizeof(int) + 255) / 256) * 256);
  hipLaunchKernelGGL((attn_idx_kernel<T, D, R>), dim3(nsplit, (unsigned)rows),
                     dim3(kAttnThreads), 0, s, (const T*)q, (const T*)k, (const T*)v, idx,
                     count, out, part, tickets, Hq, Hkv, Lq, L_cap, cap,
                     scale * 1.4426950408889634f, nsplit);
  return hipGetLastError();
}

template <typename T, int D, int R>
hipError_t bm_t(hipStream_t s, const void* q, const void* k, const void* v,
                const uint32_t* bitmask, float* out, int B, int Hq, int Hkv, int Lq, int L,
                int L_cap, int q_pos0, float scale) {
  const long long rows = (long long)B * Hkv * Lq;
  hipLaunchKernelGGL((attn_bitmask_kernel<T, D, R>), dim3((unsigned)rows), dim3(kAttnThreads),
                     0, s, (const T*)q, (const T*)k, (const T*)v, bitmask, out, Hq, Hkv, Lq,
                     L, L_cap, q_pos0, scale * 1.4426950408889634f);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace(int B, int Hq, int Hkv, int D, int Lq, int L, int cap) {
  (void)L;
  const long long rows = (long long)B * Hkv * Lq;
  const int R = Hq / Hkv;
  const size_t tick = ((rows * sizeof(int) + 255) / 256) * 256;
  return tick + (size_t)rows * nsplit_for(cap) * R * (D + 2) * sizeof(float);
}

#define BUTLER_ATTN_DISPATCH(FN, ...)                                              \
  do {                                                                             \
    const int R = Hq / Hkv;                                                        \
    if (dtype == 1) {                                                              \
      if (D == 128) {                                                              \
        if (R == 1) return FN<bf16_t, 128, 1>(__VA_ARGS__);                        \
        if (R == 2) return FN<bf16_t, 128, 2>(__VA_ARGS__);                        \
        if (R == 4) return FN<bf16_t, 128, 4>(__VA_ARGS__);                        \
        if (R == 8) return FN<bf16_t, 128, 8>(__VA_ARGS__);                        \
      } else if (D == 64) {                                                        \
        if (R == 1) return FN<bf16_t, 64, 1>(__VA_ARGS__);                         \
        if (R == 2) return FN<bf16_t, 64, 2>(__VA_ARGS__);                         \
        if (R == 4) return FN<bf16_t, 64, 4>(__VA_ARGS__);                         \
        if (R == 8) return FN<bf16_t, 64, 8>(__VA_ARGS__);                         \
      }                                                                            \
    } else {                                                                       \
      if (D == 128) {                                                              \
        if (R == 1) return FN<float, 128, 1>(__VA_ARGS__);                         \
        if (R == 2) return FN<float, 128, 2>(__VA_ARGS__);                         \
        if (R == 4) return FN<float, 128, 4>(__VA_ARGS__);                         \
        if (R == 8) return FN<float, 128, 8>(__VA_ARGS__);                         \
      } else if (D == 64) {                                                        \
        if (R == 1) return FN<float, 64, 1>(__VA_ARGS__);                          \
        if (R == 2) return FN<float, 64, 2>(__VA_ARGS__);                          \
        if (R == 4) return FN<float, 64, 4>(__VA_ARGS__);                          \
        if (R == 8) return FN<float, 64, 8>(__VA_ARGS__);                          \
      }                                                                            \
    }                                                                              \
    return hipErrorInvalidValue;                                                   \
  } while (0)

hipError_t launch_attn_idx(hipStream_t s, int dtype, const void* q, const void* k,
                           const void* v, const int32_t* idx, const int32_t* count,
                           float* out, int B, int Hq, int Hkv, int D, int Lq, int L_cap,
                           int cap, float scale, void* ws) {
  BUTLER_ATTN_DISPATCH(idx_t, s, q, k, v, idx, count, out, B, Hq, Hkv, Lq, L_cap, cap, scale, ws);
}

hipError_t launch_attn_bitmask(hipStream_t s, int dtype, const void* q, const void* k,
                               const void* v, const uint32_t* bitmask, float* out, int B,
                               int Hq, int Hkv, int D, int Lq, int L, int L_cap, int q_pos0,
                               float scale, void* ws) {
  (void)ws;
  BUTLER_ATTN_DISPATCH(bm_t, s, q, k, v, bitmask, out, B, Hq, Hkv, Lq, L, L_cap, q_pos0, scale);
}

}  // namespace butler
