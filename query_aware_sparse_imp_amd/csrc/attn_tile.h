// Device building blocks of the decode attention, shared by the split-K attention
// kernels and the selection pass that attends its own chunk:
//   Geo / SoftState   per-lane layout and online-softmax state (max, sum, acc) per head;
//   merge_pair        merges two base-2 online-softmax states;
//   block_reduce      merges the lanes of each wave, then the waves through LDS, in a
//                     fixed order;
//   MfTile / mf_load / PvStream
//                     one 16-token tile on the matrix cores: v_mfma_f32_16x16x32_bf16 with
//                     the 16 gathered key rows as A and the group's heads as the B
//                     columns gives the logits; online softmax per head and wave; P.V on
//                     v_mfma_f32_16x16x16_bf16 with the probabilities in bf16.
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

// Merges the waves' states (s_m, s_l [wave][head], s_acc [wave][head][D] in LDS) in wave
// order into red_m/red_l [R] and red_acc [R*D]; synchronises before and after.
template <int D, int R, int NT>
__device__ __forceinline__ void merge_waves(const float* s_m, const float* s_l, const float* s_acc,
                                            float* red_m, float* red_l, float* red_acc) {
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
  merge_waves<D, R, NT>(s_m, s_l, s_acc, red_m, red_l, red_acc);
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

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

// P.V on the matrix cores.  One online-softmax stream per head and wave: lane (quad, pe)
// serves head pe, and the 16 rows of a tile share the head's running max (a max over the
// four 16-lane rows).  The tile's probabilities, rounded to bf16, are as they stand the B
// operand of v_mfma_f32_16x16x16_bf16 (B[k][n] = P[row k][head n] sits in lane 16(k/4)+n,
// element k%4); the A operand V^T[i][k] = V[row k][8i + e] for one e comes from the lane's
// four value rows, element e of each, by two byte permutes.  Accumulator o[e] then holds,
// in lane (quad, pe), head pe at d = 8(4 quad + t) + e, t = 0..3.
typedef __attribute__((ext_vector_type(4))) short s16x4_t;

struct PvStream {
  float m, l;      // running max (shared by the four rows) and this row's partial sum
  f32x4_t o[8];

  __device__ __forceinline__ void init() {
    m = neg_inf();
    l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // lim = how many of rows 4*quad .. 4*quad+3 of the tile are real list entries
  __device__ __forceinline__ void compute(const MfTile& tl, const bf16x8_t (&qf)[4], int lim,
                                          float scale_log2) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tl.k[kk]), qf[kk], c, 0, 0, 0);
    float z[4], mt = neg_inf();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = (r < lim) ? c[r] * scale_log2 : neg_inf();
      mt = fmaxf(mt, z[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);
    const float alpha = (mn == neg_inf()) ? 1.f : fast_exp2(m - mn);
    float p[4], ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = (r < lim) ? fast_exp2(z[r] - mn) : 0.f;
      ps += p[r];
    }
    l = l * alpha + ps;
    m = mn;
    if (__ballot(alpha != 1.f)) {   // the max moved for some head of the wave
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int t = 0; t < 4; ++t) o[e][t] *= alpha;
    }
    s16x4_t pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) pb[r] = __builtin_bit_cast(short, (__bf16)p[r]);
    const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&tl.v[0]);
    const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&tl.v[1]);
    const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&tl.v[2]);
    const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&tl.v[3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
      const uint32_t lo = __builtin_amdgcn_perm(v1[e >> 1], v0[e >> 1], sel);
      const uint32_t hi = __builtin_amdgcn_perm(v3[e >> 1], v2[e >> 1], sel);
      const s16x4_t a = __builtin_bit_cast(s16x4_t, make_uint2(lo, hi));
      o[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[e], 0, 0, 0);
    }
  }

  // the wave's state of head h -> LDS (s_m, s_l [wave][h], s_acc [wave][h][128]), then the
  // waves merged in order into red_m, red_l, red_acc
  template <int R, int NT>
  __device__ __forceinline__ void reduce(float* s_m, float* s_l, float* s_acc, float* red_m,
                                         float* red_l, float* red_acc) {
    constexpr int D = 128;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int quad = lane >> 4, pe = lane & 15;
    float lt = l;
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (pe < R) {
      if (quad == 0) {
        s_m[wid * R + pe] = m;
        s_l[wid * R + pe] = lt;
      }
      float* dst = s_acc + (wid * R + pe) * D + 32 * quad;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        *reinterpret_cast<float4*>(dst + 8 * t) = make_float4(o[0][t], o[1][t], o[2][t], o[3][t]);
        *reinterpret_cast<float4*>(dst + 8 * t + 4) = make_float4(o[4][t], o[5][t], o[6][t], o[7][t]);
      }
    }
    merge_waves<D, R, NT>(s_m, s_l, s_acc, red_m, red_l, red_acc);
  }
};

}  // namespace
}  // namespace butler
