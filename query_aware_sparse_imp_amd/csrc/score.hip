// Importance scores of every cached token.
//
// RAW (TokenButler model card, Method): score(t) = (sum of the group's Q_imp) . K_imp[t].
//   Decode rows: the K_imp stream is read with 16-byte loads, DP/8 lanes per token (4 at
//   d' = 32, so one wave instruction covers 16 consecutive 64-byte rows), two batches of
//   8 rows in flight per thread; products and sums run in float64, where every partial
//   sum of bf16 products is exact, and the result is rounded once to float32 -- the
//   score is the exactly rounded dot product whatever the reduction order.  Multi-row
//   calls (prefill chunks): the same exact contraction on the matrix cores in float64
//   (score_rows_mfma_kernel, described with it below).
//
// Selection heads: B*Hkv score rows, where "Hkv" counts selection heads -- each the sum of
// Hq/Hkv consecutive query heads -- and kvdiv consecutive selection heads read one physical
// KV head (cache row bg / kvdiv).  kvdiv = 1 is selection per KV head; with one query head
// per selection head, every query head ranks the tokens on its own.
//
// Single-row calls can also add each score's first radix digit (the top 11 bits of the
// order-preserving key that the selection uses) into a per-row global histogram, counted
// in LDS per workgroup and flushed with atomics, so the selection that follows starts from
// it instead of reading every score once more.  With selection-cache flags, the rows of a
// kept (b, KV head) are skipped.
//
// SOFTVOTE (TokenSelect README, highlights): per-head logits z_h(t) = scale * q_h . k_t,
//   a softmax over t for every head, summed over the heads of the GQA group.
//   Pass 1 streams the keys once (bf16, D = 128: matrix cores, 16 key rows x the group's
//   heads per MFMA; otherwise D/8 lanes per key row), writes the base-2 logits of the R
//   heads and a per-block (max, sum of exp2) pair per head.  Pass 2 merges the block
//   pairs (every block computes the same deterministic merge) and turns the stored
//   logits into the summed probabilities.

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr int kRawThreads = 256;
#ifndef BUTLER_SCORE_UNROLL
#define BUTLER_SCORE_UNROLL 8
#endif
#ifndef BUTLER_SCORE_ROW_WG
#define BUTLER_SCORE_ROW_WG 64
#endif
constexpr int kRawUnroll = BUTLER_SCORE_UNROLL;
constexpr int kRawRowWg = BUTLER_SCORE_ROW_WG;

// Raw bytes of one 16-byte piece of every token of a batch.
template <int U>
struct RawBatch {
  uint4 v[U];
};

__device__ __forceinline__ bf16_t round_to(double v, bf16_t*) { return d2bf(v); }
__device__ __forceinline__ float round_to(double v, float*) { return (float)v; }

// DA > 0: the decode step's key row L - 1 (D = DA) is projected, K_imp[L-1] =
// K[L-1] . W_K, by one extra workgroup per row (the first in x) -- with the summation order
// of project_keys_kernel, so the row is the one butler_project_keys writes -- stored to
// kimp_w and scored from LDS, while the other workgroups stream tokens [t_begin, L - 1).
// Rows of kept (b, KV head) still get their K_imp row.
template <typename T, int DP, int DA>
__global__ __launch_bounds__(kRawThreads) void score_raw_kernel(
    const T* __restrict__ q_imp, const T* __restrict__ kimp, float* __restrict__ scores,
    int Hq, int Hkv, int G, int slot, int Lq, int L, int L_cap, int q_pos0, int causal,
    int tpb, uint32_t* __restrict__ radix_hist, const int32_t* __restrict__ keep,
    const T* __restrict__ k_cache, const T* __restrict__ w_k, T* kimp_w, int kvdiv,
    int t_begin, int t_end) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPT = DP / EPL;           // lanes per token
  constexpr int TPI = kRawThreads / LPT;  // tokens per block-wide step
  constexpr int U = kRawUnroll;
  const int bg = blockIdx.z, i = blockIdx.y;
  // the appended token L - 1 has the first workgroup of the row (dispatched early)
  const bool proj = DA > 0 && blockIdx.x == 0;
  const bool skip = keep && keep[bg];
  if (skip && !proj) return;   // the cached selection stands (single-row calls)
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int R = Hq / Hkv;
  const int part = threadIdx.x % LPT, sub = threadIdx.x / LPT;
  const int L_r = causal ? min(q_pos0 + i + 1, L) : L;
  const int t_stream = DA > 0 ? L - 1 : t_end;   // the streaming workgroups' end
  const int t0 = t_begin + ((int)blockIdx.x - (DA > 0 ? 1 : 0)) * tpb;   // tokens [t0, t1)
  const int t1 = min(t0 + tpb, t_stream);
  const int tv = min(t1, L_r);
  const int bk = bg / kvdiv;   // physical KV head
  const T* kb = kimp + (size_t)bk * L_cap * DP + part * EPL;
  float* srow = scores + ((size_t)bg * Lq + i) * L;
  // batch loads at clamped addresses: no control flow around them
  auto load_batch = [&](RawBatch<U>& rb, int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tu = min(t + u * TPI, max(tv - 1, 0));
      rb.v[u] = *reinterpret_cast<const uint4*>(kb + (size_t)tu * DP);
    }
  };
  __shared__ double qbar[DP];
  __shared__ uint32_t hist[2048];
  // The group's summed query: its R <= 8 values (element threadIdx.x % DP of each head)
  // are loaded together at clamped addresses -- no load behind a branch, which would make
  // the compiler wait for every load in flight -- and summed in head order into LDS.
  // Loads complete in issue order, so they are issued before the K_imp batches.
  auto load_query = [&](float (&qh)[8]) {
    const int d = threadIdx.x % DP;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      qh[r] = load_elem(q_imp + ((((size_t)b * Hq + g * R + min(r, R - 1)) * G + slot) * Lq + i) *
                                    DP + d);
  };
  auto sum_query = [&](const float (&qh)[8]) {
    if (threadIdx.x < DP) {
      double a = 0.0;
#pragma unroll
      for (int r = 0; r < 8; ++r) a += (r < R) ? (double)qh[r] : 0.0;
      qbar[threadIdx.x] = a;
    }
  };
  // score of one token from its d' values kf (this lane's EPL of them), summed over the
  // token's LPT lanes: the same arithmetic in the streaming and the appended-token paths
  auto dot = [&](const float* kf, const double* qv) {
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = fma(qv[e], (double)kf[e], acc);
    return quad_sum_d<LPT>(acc);
  };
  if constexpr (DA > 0) {
    if (proj) {
      constexpr int DW = DA;
      // W_K of the projection in its storage type: bf16 fits in the histogram's LDS, which
      // this workgroup does not use, so the kernel's LDS stays that of the streaming ones
      static_assert(sizeof(T) != 2 || DW * DP * 2 <= 2048 * 4, "W_K fits the histogram's LDS");
      constexpr int WSH = sizeof(T) == 2 ? 1 : DW * DP;
      __shared__ __align__(16) T wsh_own[WSH];
      T* wsh = sizeof(T) == 2 ? reinterpret_cast<T*>(hist) : wsh_own;
      __shared__ float ksh[DW];                       // key row L - 1, as float
      __shared__ __align__(16) T knew[DP];            // its K_imp row, storage type
      // W_K and the key row in 16-byte pieces, requested before anything else
      constexpr int NPIECE = DW * DP / EPL;
      constexpr int PER = (NPIECE + kRawThreads - 1) / kRawThreads;
      // (the pieces go straight to LDS: a register array holding them would be placed in
      // LDS by the compiler, doubling the kernel's LDS)
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int pc = threadIdx.x + u * kRawThreads;
        if (pc < NPIECE)
          *reinterpret_cast<uint4*>(wsh + pc * EPL) = *reinterpret_cast<const uint4*>(w_k + pc * EPL);
      }
      float kv[EPL], qh[8];
      const T* krow = k_cache + ((size_t)bk * L_cap + (L - 1)) * DW;
      if (threadIdx.x < DW / EPL) Vec16<T>::load(krow + threadIdx.x * EPL, kv);
      load_query(qh);
      sum_query(qh);
      if (threadIdx.x < DW / EPL) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) ksh[threadIdx.x * EPL + e] = kv[e];
      }
      __syncthreads();
      // four lanes per output j, lane r keeping the chain of chunks c = r (mod 4): the
      // four float64 partial sums of project_keys_kernel, combined in its order
      if (threadIdx.x < 4 * DP) {
        const int j = threadIdx.x >> 2, r = threadIdx.x & 3;
        double acc = 0.0;
#pragma unroll
        for (int c = r; c < DW / EPL; c += 4) {
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc = fma((double)ksh[c * EPL + e], (double)load_elem(wsh + (c * EPL + e) * DP + j),
                      acc);
        }
        const int lo = __double2loint(acc), hi = __double2hiint(acc);
        const double a1 = __hiloint2double(__shfl_xor(hi, 1), __shfl_xor(lo, 1));
        const double s01 = (r & 1) ? a1 + acc : acc + a1;   // (acc0 + acc1), (acc2 + acc3)
        const int lo2 = __double2loint(s01), hi2 = __double2hiint(s01);
        const double s23 = __hiloint2double(__shfl_xor(hi2, 2), __shfl_xor(lo2, 2));
        const double tot = (r & 2) ? s23 + s01 : s01 + s23;
        if (r == 0) {
          const T rv = round_to(tot, (T*)nullptr);
          // the first selection head of a KV head stores the row (the others compute the same)
          if (bg == bk * kvdiv) kimp_w[((size_t)bk * L_cap + (L - 1)) * DP + j] = rv;
          knew[j] = rv;
        }
      }
      __syncthreads();
      if (skip || L - 1 < t_begin) return;
      if (threadIdx.x < LPT) {
        double qv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[e] = qbar[part * EPL + e];
        Raw16 r16;
        r16.v = reinterpret_cast<const uint4*>(knew)[part];
        float kf[EPL];
        unpack16<T>(r16, kf);
        const double acc = dot(kf, qv);
        if (part == 0) {
          const float sc = (L - 1 < L_r) ? (float)acc : neg_inf();
          srow[L - 1] = sc;
          if (radix_hist && L - 1 < L_r)
            atomicAdd(&radix_hist[((size_t)bg * Lq + i) * 2048 + (score_key(sc) >> 21)], 1u);
        }
      }
      return;
    }
  }
  RawBatch<U> ba, bb;
  const int t = t0 + sub;
  constexpr int STEP = TPI * U;   // tokens of one batch
  // batches of this workgroup: the same count for every lane
  const int nb = t1 > t0 ? (t1 - t0 + STEP - 1) / STEP : 0;
  // the query values first, then the first two batches of K_imp rows, all in flight while
  // the group query is summed.  Every batch load is unconditional (past the end it reads
  // the last token again, and consume() stores nothing for it), so the compiler counts
  // the loads in flight exactly and each wait is for one batch only.
  float qh[8];
  load_query(qh);
  load_batch(ba, t);
  load_batch(bb, t + STEP);
  if (radix_hist)
    for (int j = threadIdx.x; j < 2048; j += kRawThreads) hist[j] = 0u;
  sum_query(qh);
  __syncthreads();
  double qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qbar[part * EPL + e];
  // The U tokens of a batch run as U independent chains -- each token's own sum in the
  // order dot() takes (element e = 0, 1, ... then the lanes) -- interleaved so that the
  // float64 latencies overlap; the stores and histogram counts come after all of them.
  auto consume = [&](const RawBatch<U>& rb, int tb) {
    double acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = fma(qv[e], (double)elem16<T>(rb.v[u], e), acc[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = quad_sum_d<LPT>(acc[u]);
    if (part == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tu = tb + u * TPI;
        if (tu < t1) {
          const float sc = (tu < L_r) ? (float)acc[u] : neg_inf();
          srow[tu] = sc;
          if (radix_hist && tu < L_r) atomicAdd(&hist[score_key(sc) >> 21], 1u);
        }
      }
    }
  };
  // two batches in flight: the one after next is requested as soon as one is consumed
  // (the last pair's requests may read past the end: the last token again, unused)
  for (int pr = 0; pr < nb / 2; ++pr) {
    const int tb = t + 2 * pr * STEP;
    consume(ba, tb);
    load_batch(ba, tb + 2 * STEP);
    consume(bb, tb + STEP);
    load_batch(bb, tb + 3 * STEP);
  }
  if (nb & 1) consume(ba, t + (nb - 1) * STEP);
  if (radix_hist) {
    __syncthreads();
    uint32_t* gh = radix_hist + ((size_t)bg * Lq + i) * 2048;
    for (int j = threadIdx.x; j < 2048; j += kRawThreads)
      if (hist[j]) atomicAdd(&gh[j], hist[j]);
  }
}

// ---------------------------------------------------------------------------
// soft voting
// ---------------------------------------------------------------------------

constexpr int kSvThreads = 256;
constexpr int kSvTokensPerBlock = 256;

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  if (m2 == neg_inf()) return;
  if (m == neg_inf()) { m = m2; l = l2; return; }
  const float mn = fmaxf(m, m2);
  l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
  m = mn;
}

template <typename T, int D, int R>
__global__ __launch_bounds__(kSvThreads) void softvote_logits_kernel(
    const T* __restrict__ q, const T* __restrict__ k, float* __restrict__ logits,
    float2* __restrict__ part, int Hq, int Hkv, int L, int L_cap, float scale_log2,
    int nblk, const int32_t* __restrict__ keep, int kvdiv) {
  if (keep && keep[blockIdx.y]) return;
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  constexpr int TPW = 64 / LPR;
  constexpr int ITERS = 64 / TPW;
  const int bg = blockIdx.y, blk = blockIdx.x;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int sub = lane / LPR, pe = lane % LPR;
  float qr[R][EPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float tmp[EPL];
    Vec16<T>::load(q + ((size_t)b * Hq + g * R + r) * D + pe * EPL, tmp);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[r][e] = tmp[e] * scale_log2;
  }
  float m[R], l[R];
#pragma unroll
  for (int r = 0; r < R; ++r) { m[r] = neg_inf(); l[r] = 0.f; }
  const int tbase = blk * kSvTokensPerBlock + wid * 64 + sub;
  const T* kb = k + (size_t)(bg / kvdiv) * L_cap * D + pe * EPL;
  float* zb = logits + (size_t)bg * R * L;
#pragma unroll 4
  for (int it = 0; it < ITERS; ++it) {
    const int t = tbase + it * TPW;
    float kv[EPL];
    if (t < L) {
      Vec16<T>::load(kb + (size_t)t * D, kv);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) kv[e] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a = fmaf(qr[r][e], kv[e], a);
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) a += __shfl_xor(a, o, 64);
      if (t < L) {
        if (pe == 0) zb[(size_t)r * L + t] = a;
        merge_ml(m[r], l[r], a, 1.f);
      }
    }
  }
  // lane groups of the wave -> one pair per head
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m[r], o, 64);
      const float l2 = __shfl_xor(l[r], o, 64);
      merge_ml(m[r], l[r], m2, l2);
    }
  }
  __shared__ float sm[4][R], sl[4][R];
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) { sm[wid][r] = m[r]; sl[wid][r] = l[r]; }
  }
  __syncthreads();
  if (threadIdx.x < R) {
    const int r = threadIdx.x;
    float mm = sm[0][r], ll = sl[0][r];
    for (int w = 1; w < 4; ++w) merge_ml(mm, ll, sm[w][r], sl[w][r]);
    part[((size_t)bg * nblk + blk) * R + r] = make_float2(mm, ll);
  }
}


// bf16, D = 128: logits on the matrix cores.  v_mfma_f32_16x16x32_bf16 with 16 key rows as
// A and the group's R query heads as the B columns (columns >= R are zero); lane
// (quad, pe) then holds the logits of tokens 4*quad + r of the tile for head pe.  A wave
// takes 64 tokens (4 tiles), all 16 of its 16-byte key loads issued first.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8s_t;
typedef __attribute__((ext_vector_type(4))) float f32x4s_t;

template <int R>
__global__ __launch_bounds__(kSvThreads) void softvote_logits_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, float* __restrict__ logits,
    float2* __restrict__ part, int Hq, int Hkv, int L, int L_cap, float scale_log2, int nblk,
    const int32_t* __restrict__ keep, int kvdiv) {
  if (keep && keep[blockIdx.y]) return;
  constexpr int D = 128;
  const int bg = blockIdx.y, blk = blockIdx.x;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int quad = lane >> 4, pe = lane & 15;
  const int tw = blk * kSvTokensPerBlock + wid * 64;
  const bf16_t* kb = k + (size_t)(bg / kvdiv) * L_cap * D + 8 * quad;
  uint4 kr[4][4];
#pragma unroll
  for (int tile = 0; tile < 4; ++tile) {
    const int t = min(tw + tile * 16 + pe, L - 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      kr[tile][kk] = *reinterpret_cast<const uint4*>(kb + (size_t)t * D + kk * 32);
  }
  bf16x8s_t qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (pe < R)
      raw = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + g * R + pe) * D + kk * 32 + 8 * quad);
    qf[kk] = __builtin_bit_cast(bf16x8s_t, raw);
  }
  float z[4][4];
  float mloc = neg_inf();
#pragma unroll
  for (int tile = 0; tile < 4; ++tile) {
    f32x4s_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8s_t, kr[tile][kk]),
                                                   qf[kk], c, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tw + tile * 16 + 4 * quad + r;
      z[tile][r] = (t < L) ? c[r] * scale_log2 : neg_inf();
      mloc = fmaxf(mloc, z[tile][r]);
    }
  }
  float* zb = logits + ((size_t)bg * R + min(pe, R - 1)) * L;
  float lloc = 0.f;
#pragma unroll
  for (int tile = 0; tile < 4; ++tile)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tw + tile * 16 + 4 * quad + r;
      if (pe < R && t < L) zb[t] = z[tile][r];
      lloc += (z[tile][r] == neg_inf()) ? 0.f : fast_exp2(z[tile][r] - mloc);
    }
  // the four quads of a head, then the waves
  float m = mloc, l = lloc;
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    const float m2 = __shfl_xor(m, o, 64), l2 = __shfl_xor(l, o, 64);
    merge_ml(m, l, m2, l2);
  }
  __shared__ float sm[kSvThreads / 64][16], sl[kSvThreads / 64][16];
  if (quad == 0) {
    sm[wid][pe] = m;
    sl[wid][pe] = l;
  }
  __syncthreads();
  if (threadIdx.x < R) {
    const int r = threadIdx.x;
    float mm = sm[0][r], ll = sl[0][r];
    for (int w = 1; w < kSvThreads / 64; ++w) merge_ml(mm, ll, sm[w][r], sl[w][r]);
    part[((size_t)bg * nblk + blk) * R + r] = make_float2(mm, ll);
  }
}

// Combine: 8 tokens per thread (2048 per workgroup), so the row's (max, sum) merge and the
// histogram's set-up and flush are shared by more tokens; the block's logits are requested
// first, at clamped addresses, all in flight together with the (max, sum) pairs.
constexpr int kCbTpt = 8;
constexpr int kCbTokens = kSvThreads * kCbTpt;

template <int R>
__global__ __launch_bounds__(kSvThreads) void softvote_combine_kernel(
    const float* __restrict__ logits, const float2* __restrict__ part,
    float* __restrict__ scores, int L, int nblk, uint32_t* __restrict__ radix_hist,
    const int32_t* __restrict__ keep) {
  const int bg = blockIdx.y, blk = blockIdx.x;
  if (keep && keep[bg]) return;
  const float* zb = logits + (size_t)bg * R * L;
  const int t0 = blk * kCbTokens + threadIdx.x;
  float z[kCbTpt][R];
#pragma unroll
  for (int j = 0; j < kCbTpt; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) z[j][r] = zb[(size_t)r * L + min(t0 + kSvThreads * j, L - 1)];
  __shared__ float Ms[R], Ls[R];
  __shared__ uint32_t hist[2048];
  if (radix_hist)
    for (int j = threadIdx.x; j < 2048; j += kSvThreads) hist[j] = 0u;
  // the row's per-block (max, sum) pairs of every head: thread j merges blocks j, j+256,
  // ... in order, then a butterfly over the wave and the waves in order (deterministic)
  {
    float mm[R], ll[R];
#pragma unroll
    for (int r = 0; r < R; ++r) { mm[r] = neg_inf(); ll[r] = 0.f; }
    for (int j = threadIdx.x; j < nblk; j += kSvThreads) {
      float2 p[R];
#pragma unroll
      for (int r = 0; r < R; ++r) p[r] = part[((size_t)bg * nblk + j) * R + r];
#pragma unroll
      for (int r = 0; r < R; ++r) merge_ml(mm[r], ll[r], p[r].x, p[r].y);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(mm[r], o, 64), l2 = __shfl_xor(ll[r], o, 64);
        merge_ml(mm[r], ll[r], m2, l2);
      }
    }
    __shared__ float wm[kSvThreads / 64][R], wl[kSvThreads / 64][R];
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) { wm[threadIdx.x >> 6][r] = mm[r]; wl[threadIdx.x >> 6][r] = ll[r]; }
    }
    __syncthreads();
    if (threadIdx.x < R) {
      const int r = threadIdx.x;
      float m0 = wm[0][r], l0 = wl[0][r];
      for (int w = 1; w < kSvThreads / 64; ++w) merge_ml(m0, l0, wm[w][r], wl[w][r]);
      Ms[r] = m0;
      Ls[r] = l0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kCbTpt; ++j) {
    const int t = t0 + kSvThreads * j;
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) s += fast_exp2(z[j][r] - Ms[r]) / Ls[r];
    if (t < L) {
      scores[(size_t)bg * L + t] = s;
      if (radix_hist) atomicAdd(&hist[score_key(s) >> 21], 1u);
    }
  }
  if (radix_hist) {
    __syncthreads();
    uint32_t* gh = radix_hist + (size_t)bg * 2048;
    for (int j = threadIdx.x; j < 2048; j += kSvThreads)
      if (hist[j]) atomicAdd(&gh[j], hist[j]);
  }
}


// ---------------------------------------------------------------------------
// multi-row raw scores (prefill chunks) on the matrix cores, still exact
// ---------------------------------------------------------------------------
// S[i][t] = qbar[i] . K_imp[t] for a block of query rows against every token is a dense
// contraction over d'.  v_mfma_f64_16x16x4f64 keeps it exact: the operands are exact in
// float64 (qbar is a float64 sum of R bf16 values, K_imp is bf16), every product and
// partial sum is exact, so the accumulation order does not matter and the one rounding
// to float32 gives the same bits as the decode kernel and the oracle.
// Layout of the f64 MFMA (checked on the device): A lane l = A[l%16][l/16], B lane l =
// B[l/16][l%16], accumulator r of lane l = C[4r + l/16][l%16].  The d' index is permuted
// so that lane group g4 = l/16 feeds d' = KG*g4 + s at step s (KG = d'/4): each lane then
// reads KG consecutive K_imp elements of its token with one load.
// A workgroup holds 64 query rows (qbar in VGPRs, 16 x 16 tiles of 4 x 4 per wave) and
// its 4 waves sweep 1024 tokens, 64 per wave step, each step's K_imp rows requested
// before the previous step's products; tiles past every row's causal end are written as
// -inf without arithmetic.

constexpr int kCsThreads = 256;
constexpr int kCsRows = 64;
constexpr int kCsTokBlk = 1024;

typedef __attribute__((ext_vector_type(4))) double f64x4_t;

template <int DP, int R>   // R: query heads per KV head (1, 2, 4 or 8)
__global__ __launch_bounds__(kCsThreads, 2) void score_rows_mfma_kernel(
    const bf16_t* __restrict__ q_imp, const bf16_t* __restrict__ kimp, float* __restrict__ scores,
    int Hq, int Hkv, int G, int slot, int Lq, int L, int L_cap, int q_pos0, int causal,
    int kvdiv) {
  constexpr int KG = DP / 4;   // d' values per lane group
  const int bg = blockIdx.z, i0 = blockIdx.y * kCsRows;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int ql = lane & 15, g4 = lane >> 4;
  // qbar[qb][s] = sum over the group's heads of Q_imp[row i0 + 16qb + ql][KG*g4 + s]
  double qa[4][KG];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int i = min(i0 + 16 * qb + ql, Lq - 1);
    float hv[R][KG];
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const bf16_t* src = q_imp + ((((long long)b * Hq + g * R + h) * G + slot) * Lq + i) * DP + KG * g4;
      if constexpr (KG == 8) {
        Vec16<bf16_t>::load(src, hv[h]);
      } else {
        const uint2 raw = *reinterpret_cast<const uint2*>(src);
        hv[h][0] = bf2f((bf16_t)(raw.x & 0xffffu));
        hv[h][1] = bf2f((bf16_t)(raw.x >> 16));
        hv[h][2] = bf2f((bf16_t)(raw.y & 0xffffu));
        hv[h][3] = bf2f((bf16_t)(raw.y >> 16));
      }
    }
#pragma unroll
    for (int e = 0; e < KG; ++e) {
      double a = 0.0;
#pragma unroll
      for (int h = 0; h < R; ++h) a += (double)hv[h][e];
      qa[qb][e] = a;
    }
  }
  const bf16_t* kb = kimp + (long long)(bg / kvdiv) * L_cap * DP + KG * g4;
  float* srow0 = scores + ((long long)bg * Lq) * L;
  const int i_last = min(i0 + kCsRows, Lq) - 1;
  const int t_vis = causal ? min(L, q_pos0 + i_last + 1) : L;   // tokens any row sees
  // the wave's K_imp rows of a 64-token step, at clamped addresses
  auto load_k = [&](float (&kv)[4][KG], int t0) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const bf16_t* src = kb + (long long)min(t0 + 16 * tb + ql, L - 1) * DP;
      if constexpr (KG == 8) {
        Vec16<bf16_t>::load(src, kv[tb]);
      } else {
        const uint2 raw = *reinterpret_cast<const uint2*>(src);
        kv[tb][0] = bf2f((bf16_t)(raw.x & 0xffffu));
        kv[tb][1] = bf2f((bf16_t)(raw.x >> 16));
        kv[tb][2] = bf2f((bf16_t)(raw.y & 0xffffu));
        kv[tb][3] = bf2f((bf16_t)(raw.y >> 16));
      }
    }
  };
  constexpr int kSteps = kCsTokBlk / (64 * 4);
  const int tw = blockIdx.x * kCsTokBlk + wid * 64;   // this wave's first token
  float kv[4][KG];
  load_k(kv, tw);
  for (int it = 0; it < kSteps; ++it) {
    const int t0 = tw + it * 256;
    if (t0 >= L) break;
    // the next step's rows are requested before this step's products and stores
    float kn[4][KG];
    load_k(kn, min(t0 + 256, L - 1));
    const bool live = t0 < t_vis;
    // one 16-row block at a time (4 accumulator tiles live, not 16: two waves per SIMD),
    // its four token tiles as independent chains; accumulator r of tile tb: row
    // i0 + 16qb + 4r + g4, token t0 + 16tb + ql
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      f64x4_t acc[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[tb] = f64x4_t{0.0, 0.0, 0.0, 0.0};
      if (live) {
#pragma unroll
        for (int s8 = 0; s8 < KG; ++s8)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
            acc[tb] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[qb][s8], (double)kv[tb][s8],
                                                           acc[tb], 0, 0, 0);
      }
      // The block's 16 rows as one buffer range: a store of a row past Lq or of a token
      // past L gets an offset beyond the range and is dropped by the hardware, so no
      // store sits behind a branch; the causal mask is a select.
      const int ib = i0 + 16 * qb;
      if (ib < Lq) {
        const int nrows = min(16, Lq - ib);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(srow0 + (long long)ib * L), (short)0, nrows * L * 4, 0x00020000);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ir = 4 * r + g4;
          const int lim = causal ? min(L, q_pos0 + ib + ir + 1) : L;
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            const int t = t0 + 16 * tb + ql;
            const float v = (t < lim) ? (float)acc[tb][r] : neg_inf();
            const int off = (t < L) ? (ir * L + t) * 4 : 0x7fffffff;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int e = 0; e < KG; ++e) kv[tb][e] = kn[tb][e];
  }
}

template <int DP>
hipError_t rows_t(hipStream_t s, const void* q_imp, const void* kimp, float* scores, int B,
                  int Hq, int Hkv, int G, int slot, int Lq, int L, int L_cap, int q_pos0,
                  int causal, int kvdiv) {
  dim3 grid((L + kCsTokBlk - 1) / kCsTokBlk, (Lq + kCsRows - 1) / kCsRows, B * Hkv);
#define BUTLER_ROWS(R)                                                                    \
  hipLaunchKernelGGL((score_rows_mfma_kernel<DP, R>), grid, dim3(kCsThreads), 0, s,       \
                     (const bf16_t*)q_imp, (const bf16_t*)kimp, scores, Hq, Hkv, G, slot, Lq, \
                     L, L_cap, q_pos0, causal, kvdiv)
  switch (Hq / Hkv) {
    case 1: BUTLER_ROWS(1); break;
    case 2: BUTLER_ROWS(2); break;
    case 4: BUTLER_ROWS(4); break;
    case 8: BUTLER_ROWS(8); break;
    default: return hipErrorInvalidValue;
  }
#undef BUTLER_ROWS
  return hipGetLastError();
}

template <typename T, int DP, int DA = 0>
hipError_t raw_t(hipStream_t s, const void* q_imp, const void* kimp, float* scores, int B,
                 int Hq, int Hkv, int G, int slot, int Lq, int L, int L_cap, int q_pos0,
                 int causal, uint32_t* hist, const int32_t* keep, int kvdiv,
                 const void* k_cache = nullptr, const void* w_k = nullptr, int t_begin = 0,
                 int t_end = -1) {
  if (t_end < 0) t_end = L;
  // with the projection (DA > 0, t_end = L) the appended token gets a workgroup of its own
  const int n = (DA > 0 ? t_end - 1 : t_end) - t_begin;   // tokens streamed per row
  constexpr int LPT = DP / Vec16<T>::N;
  // a tile is what one block-wide step covers (kRawUnroll loads per thread); a workgroup
  // loops over enough tiles that a row has at most kRawRowWg workgroups -- this bounds the
  // atomics that the workgroups' histograms send to the same hot bins of a row -- or twice
  // that for rows of more than 4 kRawRowWg tiles, so that no workgroup streams more than
  // 4 tiles while the row has under 2 kRawRowWg of them (measured: 4 tiles per workgroup
  // beat 2 at 128K and 8 at 256K tokens)
  const int tile = (kRawThreads / LPT) * kRawUnroll;
  const int tiles = (n + tile - 1) / tile;
  const int row_wg = tiles > 4 * kRawRowWg ? 2 * kRawRowWg : kRawRowWg;
  const int per = (tiles + row_wg - 1) / row_wg;
  const int tpb = tile * (per > 0 ? per : 1);
  const int nstream = n > 0 ? (n + tpb - 1) / tpb : 0;   // none when only token L-1 is scored
  dim3 grid(nstream + (DA > 0 ? 1 : 0), Lq, B * Hkv);
  hipLaunchKernelGGL((score_raw_kernel<T, DP, DA>), grid, dim3(kRawThreads), 0, s,
                     (const T*)q_imp, (const T*)kimp, scores, Hq, Hkv, G, slot, Lq, L, L_cap,
                     q_pos0, causal, tpb, hist, keep, (const T*)k_cache, (const T*)w_k,
                     (T*)const_cast<void*>(kimp), kvdiv, t_begin, t_end);
  return hipGetLastError();
}

template <typename T, int D, int R>
hipError_t sv_t(hipStream_t s, const void* q, const void* k, float* scores, int B, int Hq,
                int Hkv, int L, int L_cap, float scale, void* ws, uint32_t* hist,
                const int32_t* keep, int kvdiv) {
  const int nblk = (L + kSvTokensPerBlock - 1) / kSvTokensPerBlock;
  float* logits = (float*)ws;
  float2* part = (float2*)(logits + (size_t)B * Hkv * R * L);
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(nblk, B * Hkv);
  if constexpr (std::is_same<T, bf16_t>::value && D == 128) {
    hipLaunchKernelGGL((softvote_logits_mfma_kernel<R>), grid, dim3(kSvThreads), 0, s,
                       (const bf16_t*)q, (const bf16_t*)k, logits, part, Hq, Hkv, L, L_cap,
                       scale_log2, nblk, keep, kvdiv);
  } else {
    hipLaunchKernelGGL((softvote_logits_kernel<T, D, R>), grid, dim3(kSvThreads), 0, s,
                       (const T*)q, (const T*)k, logits, part, Hq, Hkv, L, L_cap, scale_log2,
                       nblk, keep, kvdiv);
  }
  const dim3 cgrid((L + kCbTokens - 1) / kCbTokens, B * Hkv);
  hipLaunchKernelGGL((softvote_combine_kernel<R>), cgrid, dim3(kSvThreads), 0, s, logits, part,
                     scores, L, nblk, hist, keep);
  return hipGetLastError();
}

bool R_ok(int Hq, int Hkv) { return Hq % Hkv == 0 && Hq / Hkv <= 8; }

}  // namespace

hipError_t launch_score_tokens(hipStream_t s, int dtype, const void* q_imp, const void* kimp,
                               float* scores, int B, int Hq, int Hkv, int G, int slot, int L,
                               int L_cap, int dp, uint32_t* hist, const int32_t* keep,
                               int kvdiv, int t_begin, int t_end) {
#define BUTLER_ST(T, DP)                                                                     \
  if (dp == DP)                                                                            \
    return raw_t<T, DP>(s, q_imp, kimp, scores, B, Hq, Hkv, G, slot, 1, L, L_cap, 0, 0, hist, \
                        keep, kvdiv, nullptr, nullptr, t_begin, t_end);
  if (dtype == 1) {
    BUTLER_ST(bf16_t, 32) BUTLER_ST(bf16_t, 16)
  } else {
    BUTLER_ST(float, 32) BUTLER_ST(float, 16)
  }
#undef BUTLER_ST
  return hipErrorInvalidValue;
}

hipError_t launch_score_raw(hipStream_t s, int dtype, const void* q_imp, const void* kimp,
                            float* scores, int B, int Hq, int Hkv, int G, int slot, int Lq,
                            int L, int L_cap, int dp, int q_pos0, int causal, uint32_t* hist,
                            const int32_t* keep, int kvdiv) {
  if (dtype == 1 && Lq > 1 && R_ok(Hq, Hkv)) {
    // several query rows: the matrix-core kernel (it builds no first-digit histogram)
    if (dp == 32) return rows_t<32>(s, q_imp, kimp, scores, B, Hq, Hkv, G, slot, Lq, L, L_cap, q_pos0, causal, kvdiv);
    if (dp == 16) return rows_t<16>(s, q_imp, kimp, scores, B, Hq, Hkv, G, slot, Lq, L, L_cap, q_pos0, causal, kvdiv);
  }
  if (dtype == 1) {
    if (dp == 32) return raw_t<bf16_t, 32>(s, q_imp, kimp, scores, B, Hq, Hkv, G, slot, Lq, L, L_cap, q_pos0, causal, hist, keep, kvdiv);
    if (dp == 16) return raw_t<bf16_t, 16>(s, q_imp, kimp, scores, B, Hq, Hkv, G, slot, Lq, L, L_cap, q_pos0, causal, hist, keep, kvdiv);
  } else {
    if (dp == 32) return raw_t<float, 32>(s, q_imp, kimp, scores, B, Hq, Hkv, G, slot, Lq, L, L_cap, q_pos0, causal, hist, keep, kvdiv);
    if (dp == 16) return raw_t<float, 16>(s, q_imp, kimp, scores, B, Hq, Hkv, G, slot, Lq, L, L_cap, q_pos0, causal, hist, keep, kvdiv);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_project_score(hipStream_t s, int dtype, const void* q_imp,
                                const void* k_cache, const void* w_k, void* kimp,
                                float* scores, int B, int Hq, int Hkv, int G, int slot, int L,
                                int L_cap, int D, int dp, uint32_t* hist, const int32_t* keep,
                                int kvdiv, int t_begin) {
#define BUTLER_PS(T, DP, DD)                                                                 \
  if (dp == DP && D == DD)                                                                 \
    return raw_t<T, DP, DD>(s, q_imp, kimp, scores, B, Hq, Hkv, G, slot, 1, L, L_cap, 0, 0,  \
                            hist, keep, kvdiv, k_cache, w_k, t_begin, L);
  if (dtype == 1) {
    BUTLER_PS(bf16_t, 32, 128) BUTLER_PS(bf16_t, 16, 128) BUTLER_PS(bf16_t, 32, 64) BUTLER_PS(bf16_t, 16, 64)
  } else {
    BUTLER_PS(float, 32, 128) BUTLER_PS(float, 16, 128) BUTLER_PS(float, 32, 64) BUTLER_PS(float, 16, 64)
  }
#undef BUTLER_PS
  return hipErrorInvalidValue;
}

size_t softvote_workspace(int B, int Hq, int Hkv, int L) {
  const int R = Hq / Hkv;
  const size_t nblk = (L + kSvTokensPerBlock - 1) / kSvTokensPerBlock;
  return (size_t)B * Hkv * R * L * sizeof(float) + (size_t)B * Hkv * nblk * R * sizeof(float2);
}

hipError_t launch_score_softvote(hipStream_t s, int dtype, const void* q, const void* k,
                                 float* scores, int B, int Hq, int Hkv, int L, int L_cap,
                                 int D, float scale, void* ws, uint32_t* hist,
                                 const int32_t* keep, int kvdiv) {
  const int R = Hq / Hkv;
#define BUTLER_SV(T, DD, RR)                                                       \
  if (D == DD && R == RR) return sv_t<T, DD, RR>(s, q, k, scores, B, Hq, Hkv, L, L_cap, scale, ws, hist, keep, kvdiv);
  if (dtype == 1) {
    BUTLER_SV(bf16_t, 128, 1) BUTLER_SV(bf16_t, 128, 2) BUTLER_SV(bf16_t, 128, 4) BUTLER_SV(bf16_t, 128, 8)
    BUTLER_SV(bf16_t, 64, 1) BUTLER_SV(bf16_t, 64, 2) BUTLER_SV(bf16_t, 64, 4) BUTLER_SV(bf16_t, 64, 8)
  } else {
    BUTLER_SV(float, 128, 1) BUTLER_SV(float, 128, 2) BUTLER_SV(float, 128, 4) BUTLER_SV(float, 128, 8)
    BUTLER_SV(float, 64, 1) BUTLER_SV(float, 64, 2) BUTLER_SV(float, 64, 4) BUTLER_SV(float, 64, 8)
  }
#undef BUTLER_SV
  return hipErrorInvalidValue;
}

}  // namespace butler
