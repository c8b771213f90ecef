// Device building blocks of the decode attention, shared by the split-K attention
// kernels and the selection pass that attends its own chunk:
//   Geo / SoftState   per-lane layout and online-softmax state (max, sum, acc) per head;
//   merge_pair        merges two base-2 online-softmax states;
//   block_reduce      merges the lanes of each wave, then the waves through LDS, in a
//                     fixed order;
//   MfTile / mf_load / mf_compute
//                     one 16-token tile on the matrix cores: v_mfma_f32_16x16x32_bf16 with
//                     the 16 gathered key rows as A and the group's heads as the B
//                     columns, online softmax per head (a 16-lane row per head stream,
//                     DPP row_newbcast across the row), P.V on the VALU in float32.
#pragma once
#include "common.h"

namespace butler {
namespace {

template <typename T, int D, int R>
struct Geo {
  static constexpr int EPL = Vec16<T>::N;          // elements per lane
  static constexpr int LPR = D / EPL;              // lanes per key row
  static constexpr int TPW = 64 / LPR;             // rows per wave step
  static constexpr int STEPS = 32 / TPW;           // steps per wave per round
  static constexpr int UB = STEPS < 8 ? STEPS : 8; // rows per lane group per batch
};

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
};

template <int EPL>
__device__ __forceinline__ void merge_pair(float& m, float& l, float* acc, float m2, float l2,
                                           const float* a2) {
  if (m2 == neg_inf()) return;
  if (m == neg_inf()) {
    m = m2; l = l2;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = a2[e];
    return;
  }
  const float mn = fmaxf(m, m2);
  const float fa = fast_exp2(m - mn), fb = fast_exp2(m2 - mn);
  l = l * fa + l2 * fb;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * fa + a2[e] * fb;
  m = mn;
}

// Merges the lane groups of each wave (fixed order, identical in both lanes of a pair),
// then the waves through LDS.  On return, red_m/red_l [R] and red_acc [R*D] hold the
// workgroup's state; all threads have synchronised.
template <typename T, int D, int R, int NT>
__device__ __forceinline__ void block_reduce(SoftState<R, Geo<T, D, R>::EPL>& st, float* s_m,
                                             float* s_l, float* s_acc, float* red_m,
                                             float* red_l, float* red_acc) {
  using G = Geo<T, D, R>;
  constexpr int EPL = G::EPL, LPR = G::LPR;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int pe = lane % LPR;
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
    const bool low = (lane & o) == 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float m2 = __shfl_xor(st.m[r], o, 64);
      const float l2 = __shfl_xor(st.l[r], o, 64);
      float a2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(st.acc[r][e], o, 64);
      if (low) {
        merge_pair<EPL>(st.m[r], st.l[r], st.acc[r], m2, l2, a2);
      } else {
        float m = m2, l = l2, acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = a2[e];
        merge_pair<EPL>(m, l, acc, st.m[r], st.l[r], st.acc[r]);
        st.m[r] = m; st.l[r] = l;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.acc[r][e] = acc[e];
      }
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (pe == 0) { s_m[wid * R + r] = st.m[r]; s_l[wid * R + r] = st.l[r]; }
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[(wid * R + r) * D + pe * EPL + e] = st.acc[r][e];
    }
  }
  __syncthreads();
  constexpr int NWV = NT / 64;
  for (int j = threadIdx.x; j < R * D; j += NT) {
    const int r = j / D, d = j - r * D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, s_m[w * R + r]);
    float lsum = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = s_m[w * R + r];
      const float f = (mw == neg_inf()) ? 0.f : fast_exp2(mw - M);
      lsum += s_l[w * R + r] * f;
      a += s_acc[(w * R + r) * D + d] * f;
    }
    red_acc[j] = a;
    if (d == 0) { red_m[r] = M; red_l[r] = lsum; }
  }
  __syncthreads();
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

template <int H>
__device__ __forceinline__ float row_bcast(float x) { return dpp_f<0x150 + H>(x); }

__device__ __forceinline__ float row_bcast_rt(float x, int h) {
  switch (h) {
    case 0: return row_bcast<0>(x);
    case 1: return row_bcast<1>(x);
    case 2: return row_bcast<2>(x);
    case 3: return row_bcast<3>(x);
    case 4: return row_bcast<4>(x);
    case 5: return row_bcast<5>(x);
    case 6: return row_bcast<6>(x);
    default: return row_bcast<7>(x);
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

struct MfTile {
  uint4 k[4], v[4];
};

// Rows of the tile at list positions base .. base+15: lane (quad, pe) takes K columns
// kk*32 + 8*quad of row pe, and V columns 8*pe of rows 4*quad + r.  Every position of the
// staged list holds a valid cache row (past the end: a selected row, masked out of the
// softmax), so the loads need no guard and the compiler can count them exactly.
__device__ __forceinline__ void mf_load(MfTile& tl, const int* s_list, int base,
                                        const bf16_t* kb, const bf16_t* vb, int quad, int pe) {
  constexpr int D = 128;
  const int tk = s_list[base + pe];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    tl.k[kk] = *reinterpret_cast<const uint4*>(kb + (long long)tk * D + kk * 32 + 8 * quad);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tv = s_list[base + 4 * quad + r];
    tl.v[r] = *reinterpret_cast<const uint4*>(vb + (long long)tv * D + 8 * pe);
  }
}

// lim = how many of rows 4*quad .. 4*quad+3 of the tile are real list entries
template <int R>
__device__ __forceinline__ void mf_compute(const MfTile& tl, const bf16x8_t (&qf)[4], int lim,
                                           float scale_log2, float& m, float& l,
                                           float (&acc)[R][8]) {
  f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tl.k[kk]), qf[kk], c, 0, 0, 0);
  // lane (quad, pe): logits of rows 4*quad + r for head pe
  float z[4], mt = neg_inf();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    z[r] = (r < lim) ? c[r] * scale_log2 : neg_inf();
    mt = fmaxf(mt, z[r]);
  }
  const float mn = fmaxf(m, mt);
  const float alpha = (mn == neg_inf()) ? 1.f : fast_exp2(m - mn);
  float pz[4], ps = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pz[r] = (r < lim) ? fast_exp2(z[r] - mn) : 0.f;
    ps += pz[r];
  }
  l = l * alpha + ps;
  m = mn;
  float vv[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    Raw16 rv;
    rv.v = tl.v[r];
    unpack16<bf16_t>(rv, vv[r]);
  }
#pragma unroll
  for (int h = 0; h < R; ++h) {
    const float a = row_bcast_rt(alpha, h);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] *= a;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = row_bcast_rt(pz[r], h);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vv[r][e], acc[h][e]);
    }
  }
}

}  // namespace
}  // namespace butler
