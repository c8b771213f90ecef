// Attention over the selected tokens only (TokenButler model card, intro and Method:
// the full KV cache is kept, each step attends to the selected subset).
//
// Decode (index lists) -- split-K flash decoding.  The selected list of one (b, KV head,
// query row) is cut into splits sized so the grid is about what stays resident.  bf16 at
// D = 128 runs on the matrix cores (attn_mfma_kernel, described with it below); the
// other shapes take the VALU kernel: a 512-thread workgroup takes 256 list positions per
// round, each wave owns 32 and D/8 lanes cover one key row, every lane issuing the loads
// of 8 rows' K and V slices before any arithmetic.  All R query heads of the GQA group
// use the same gathered rows; the base-2 online softmax and P.V run in float32.  Each
// split writes (max, sum, acc[D]) per head, and a second kernel merges the splits of
// every (row, head, 32-wide slice of D) in split order with all of its loads in one
// round trip.  (Workgroups do not hand work to each other inside a kernel: the
// device-wide release that would need writes back the XCD's L2.)
//
// Heads: "Hkv" counts selection heads (Hq/Hkv query heads share one selected set), and
// kvdiv consecutive selection heads read one physical KV head, cache row bg / kvdiv;
// kvdiv = 1 is selection per KV head.
//
// Prefill (bitmask rows) -- bf16, D = 128, R = 4: the matrix-core kernel in
// attn_prefill.hip (64 query rows per workgroup, a wave per head and 32 rows, dense causal
// tiles masked by the rows' bitmask words).  Other shapes: one workgroup per query row
// compacts the set bits of its bitmask into an LDS index list and runs the VALU wave routine
// over it.
#include <type_traits>

#include "attn_tile.h"
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kRoundTokens = 256;     // list positions per workgroup round (32 per wave)
constexpr int kMaxSplits = 512;          // splits per row (more -> several rounds per split)
constexpr int kBmChunkWords = 64;     // bitmask words compacted per prefill round

// One batch: this lane group attends to rows toks[0..UB) (-1 = no row).
template <typename T, int D, int R>
__device__ __forceinline__ void attend_batch(const T* __restrict__ kb, const T* __restrict__ vb,
                                             const int (&toks)[Geo<T, D, R>::UB],
                                             const float (&qr)[R][Geo<T, D, R>::EPL],
                                             SoftState<R, Geo<T, D, R>::EPL>& st) {
  using G = Geo<T, D, R>;
  constexpr int EPL = G::EPL, LPR = G::LPR, UB = G::UB;
  Raw16 kr[UB], vr[UB];
#pragma unroll
  for (int u = 0; u < UB; ++u) {
    if (toks[u] >= 0) {
      kr[u].load(kb + (long long)toks[u] * D);
      vr[u].load(vb + (long long)toks[u] * D);
    } else {
      kr[u].v = make_uint4(0, 0, 0, 0);
      vr[u].v = make_uint4(0, 0, 0, 0);
    }
  }
  float z[R][UB];
#pragma unroll
  for (int u = 0; u < UB; ++u) {
    float kf[EPL];
    unpack16<T>(kr[u], kf);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a = fmaf(qr[r][e], kf[e], a);
      a = group_sum<LPR>(a);
      z[r][u] = (toks[u] >= 0) ? a : neg_inf();
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float mx = st.m[r];
#pragma unroll
    for (int u = 0; u < UB; ++u) mx = fmaxf(mx, z[r][u]);
    if (mx == neg_inf()) {
#pragma unroll
      for (int u = 0; u < UB; ++u) z[r][u] = 0.f;
      continue;
    }
    const float alpha = (st.m[r] == neg_inf()) ? 0.f : fast_exp2(st.m[r] - mx);
    float lsum = st.l[r] * alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.acc[r][e] *= alpha;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const float p = (toks[u] >= 0) ? fast_exp2(z[r][u] - mx) : 0.f;
      z[r][u] = p;
      lsum += p;
    }
    st.l[r] = lsum;
    st.m[r] = mx;
  }
#pragma unroll
  for (int u = 0; u < UB; ++u) {
    float vf[EPL];
    unpack16<T>(vr[u], vf);
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) st.acc[r][e] = fmaf(z[r][u], vf[e], st.acc[r][e]);
    }
  }
}

// lo <- merge(lo, hi) for one head
template <typename T, int D, int R>
__device__ __forceinline__ void load_q(const T* q, long long head0, long long head_stride,
                                       int pe, float scale_log2,
                                       float (&qr)[R][Geo<T, D, R>::EPL]) {
  constexpr int EPL = Geo<T, D, R>::EPL;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float tmp[EPL];
    Vec16<T>::load(q + head0 + r * head_stride + pe * EPL, tmp);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[r][e] = tmp[e] * scale_log2;
  }
}

// Runs this wave's share of one round: LDS list positions [wid*32, wid*32 + 32).
template <typename T, int D, int R>
__device__ __forceinline__ void wave_round(const T* kb, const T* vb, const int* s_list,
                                           const float (&qr)[R][Geo<T, D, R>::EPL],
                                           SoftState<R, Geo<T, D, R>::EPL>& st) {
  using G = Geo<T, D, R>;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int sub = lane / G::LPR;
#pragma unroll
  for (int s0 = 0; s0 < G::STEPS; s0 += G::UB) {
    int toks[G::UB];
#pragma unroll
    for (int u = 0; u < G::UB; ++u) toks[u] = s_list[wid * 32 + (s0 + u) * G::TPW + sub];
    attend_batch<T, D, R>(kb, vb, toks, qr, st);
  }
}

template <typename T, int D, int R>
__global__ __launch_bounds__(kAttnThreads) void attn_idx_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
    float* __restrict__ part, int Hq, int Hkv, int Lq, int L_cap, int cap, float scale_log2,
    int nsplit, int rounds, int rows, int kvdiv) {
  using G = Geo<T, D, R>;
  constexpr int EPL = G::EPL;
  constexpr int PS = D + 4;  // floats per (split, head) partial: m, l, pad, pad, acc[D]
  const int row = blockIdx.x % rows, split = blockIdx.x / rows;
  const int bg = row / Lq, i = row - bg * Lq;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int lane = threadIdx.x & 63;
  const int pe = lane % G::LPR;

  __shared__ int s_list[kRoundTokens];
  __shared__ float s_m[kAttnWaves * R], s_l[kAttnWaves * R], red_m[R], red_l[R];
  __shared__ float s_acc[kAttnWaves * R * D];
  __shared__ float red_acc[R * D];

  float qr[R][EPL];
  load_q<T, D, R>(q, (((long long)b * Hq + g * R) * Lq + i) * D, (long long)Lq * D, pe,
                  scale_log2, qr);
  const int n = min(count[row], cap);
  const int p_split = split * kRoundTokens * rounds;
  SoftState<R, EPL> st;
  st.init();
  const T* kb = k + (long long)(bg / kvdiv) * L_cap * D + pe * EPL;
  const T* vb = v + (long long)(bg / kvdiv) * L_cap * D + pe * EPL;
  const int32_t* irow = idx + (long long)row * cap;
  for (int rd = 0; rd < rounds; ++rd) {
    const int p0 = p_split + rd * kRoundTokens;
    if (p0 >= n) break;
    __syncthreads();
    if (threadIdx.x < kRoundTokens) {
      const int p = p0 + threadIdx.x;
      // indices outside [0, L_cap) are clamped so a bad list never reads past the cache
      s_list[threadIdx.x] = (p < n) ? (int)min((unsigned)irow[p], (unsigned)(L_cap - 1)) : -1;
    }
    __syncthreads();
    wave_round<T, D, R>(kb, vb, s_list, qr, st);
  }
  block_reduce<T, D, R, kAttnThreads>(st, s_m, s_l, s_acc, red_m, red_l, red_acc);
  float* my = part + ((long long)row * nsplit + split) * R * PS;
  for (int j = threadIdx.x; j < R * D; j += kAttnThreads) my[(j / D) * PS + 4 + j % D] = red_acc[j];
  if (threadIdx.x < R) {
    my[threadIdx.x * PS] = red_m[threadIdx.x];
    my[threadIdx.x * PS + 1] = red_l[threadIdx.x];
  }
}

// ---------------------------------------------------------------------------
// bf16, D = 128: logits on the matrix cores
// ---------------------------------------------------------------------------
//
// A wave takes 16 selected rows at a time.  v_mfma_f32_16x16x32_bf16 computes
// S[t][h] = sum_d K[t][d] q[h][d] for the 16 rows (A operand: lane l holds 8 consecutive
// d of row l%16, so 4 loads of 16 bytes per lane bring the tile's 16 key rows) and up to
// 16 query-head columns (B operand: the group's R heads, zero beyond).  Four MFMAs cover
// D = 128.  The result leaves the logits of rows 4q..4q+3 and head h in lane 16q + h;
// the wave keeps one online softmax per head (the max taken over the four 16-lane rows).
// P.V runs on the matrix cores too: the probabilities, rounded to bf16, are already laid
// out as the B operand of v_mfma_f32_16x16x16_bf16, and V^T comes from the lanes' value
// rows (16-byte loads of 8 columns of D) by byte permutes -- eight MFMAs per tile, no
// per-head VALU loop (PvStream).  Each wave keeps a ring of tiles with all 16 row loads
// in flight; the waves merge through LDS in a fixed order.

#ifndef BUTLER_MF_THREADS
#define BUTLER_MF_THREADS 512
#endif
#ifndef BUTLER_MF_BUF
#define BUTLER_MF_BUF 2
#endif
#ifndef BUTLER_MF_STAGE
#define BUTLER_MF_STAGE 4096
#endif
#ifndef BUTLER_MF_TARGET_BLOCKS
#define BUTLER_MF_TARGET_BLOCKS 256
#endif
constexpr int kMfThreads = BUTLER_MF_THREADS;
constexpr int kMfWaves = kMfThreads / 64;
constexpr int kMfRound = kMfWaves * 16;    // list positions per block round (a tile per wave)
constexpr int kMfBuf = BUTLER_MF_BUF;      // tiles per wave in the load ring
constexpr int kMfStage = BUTLER_MF_STAGE;  // list positions staged in LDS at a time
constexpr int kMfPad = (2 * kMfBuf - 2) * kMfRound;  // ring prefetch past the stage end
constexpr int kMfTargetBlocks = BUTLER_MF_TARGET_BLOCKS;  // grid size aimed at (2 per CU)
static_assert(kMfStage % kMfThreads == 0, "stage is a whole number of block-wide loads");

template <int R>
__global__ __launch_bounds__(kMfThreads) void attn_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
    float* __restrict__ part, int Hq, int Hkv, int Lq, int L_cap, int cap, float scale_log2,
    int nsplit, int split_len, int rows, int kvdiv) {
  constexpr int D = 128;
  constexpr int PS = D + 4;
  static_assert(R <= 8, "at most 8 query heads per KV head");
  const int row = blockIdx.x % rows, split = blockIdx.x / rows;
  const int bg = row / Lq, i = row - bg * Lq;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int quad = lane >> 4, pe = lane & 15;

  __shared__ int s_list[kMfStage + kMfPad];
  __shared__ float s_m[kMfWaves * R], s_l[kMfWaves * R], red_m[R], red_l[R];
  __shared__ __align__(16) float s_acc[kMfWaves * R * D];
  __shared__ float red_acc[R * D];

  // B operand: q[h = pe][kk*32 + 8*quad .. +8], zero for columns pe >= R
  bf16x8_t qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (pe < R)
      raw = *reinterpret_cast<const uint4*>(q + (((long long)b * Hq + g * R + pe) * Lq + i) * D +
                                            kk * 32 + 8 * quad);
    qf[kk] = as_bf16x8(raw);
  }
  const int p_begin = split * split_len;
  const int32_t* irow = idx + (long long)row * cap;
  // the first stage of indices is requested together with the count: its positions are
  // clamped to the row's capacity, not to its count, so the two round trips overlap
  constexpr int U = kMfStage / kMfThreads;
  int iv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) iv[u] = irow[min(p_begin + (int)threadIdx.x + u * kMfThreads, cap - 1)];
  const int n = min(count[row], cap);
  const int p_end = min(p_begin + split_len, n);
  const bf16_t* kb = k + (long long)(bg / kvdiv) * L_cap * D;
  const bf16_t* vb = v + (long long)(bg / kvdiv) * L_cap * D;

  PvStream ms;   // online-softmax state of the wave's heads
  ms.init();

  for (int cs = p_begin; cs < p_end; cs += kMfStage) {
    const int len = min(kMfStage, p_end - cs);
    const int nr = (len + kMfRound - 1) / kMfRound;
    __syncthreads();
    if (cs != p_begin) {
#pragma unroll
      for (int u = 0; u < U; ++u) iv[u] = irow[min(cs + (int)threadIdx.x + u * kMfThreads, cap - 1)];
    }
    // indices outside [0, L_cap) are clamped so a bad list never reads past the cache;
    // positions past the stage's end then repeat its last entry (a row already loaded)
#pragma unroll
    for (int u = 0; u < U; ++u)
      s_list[threadIdx.x + u * kMfThreads] = (int)min((unsigned)iv[u], (unsigned)(L_cap - 1));
    __syncthreads();
    const int last = s_list[len - 1];
    for (int j = len + (int)threadIdx.x; j < kMfStage + kMfPad; j += kMfThreads) s_list[j] = last;
    __syncthreads();
    // a ring of kMfBuf tiles per wave: kMfBuf - 1 tiles are in flight during each compute.
    // Round rho lives in t[rho % kMfBuf]; the main loop has no branch, so every wait is for
    // exactly one tile, and the last nr % kMfBuf rounds are already loaded when it ends.
    MfTile t[kMfBuf];
    const int w0 = wid * 16;
    const int lim0 = len - w0 - 4 * quad;
#pragma unroll
    for (int b = 0; b < kMfBuf - 1; ++b) mf_load(t[b], s_list, b * kMfRound + w0, kb, vb, quad, pe);
    const int nmain = nr - nr % kMfBuf;
    for (int r = 0; r < nmain; r += kMfBuf) {
#pragma unroll
      for (int b = 0; b < kMfBuf; ++b) {
        mf_load(t[(b + kMfBuf - 1) % kMfBuf], s_list, (r + b + kMfBuf - 1) * kMfRound + w0, kb, vb,
                quad, pe);
        ms.compute(t[b], qf, lim0 - (r + b) * kMfRound, scale_log2);
      }
    }
#pragma unroll
    for (int b = 0; b < kMfBuf - 1; ++b)
      if (nmain + b < nr) ms.compute(t[b], qf, lim0 - (nmain + b) * kMfRound, scale_log2);
  }
  ms.template reduce<R, kMfThreads>(s_m, s_l, s_acc, red_m, red_l, red_acc);
  float* my = part + ((long long)row * nsplit + split) * R * PS;
  for (int j = threadIdx.x; j < R * D; j += kMfThreads) my[(j / D) * PS + 4 + j % D] = red_acc[j];
  if (threadIdx.x < R) {
    my[threadIdx.x * PS] = red_m[threadIdx.x];
    my[threadIdx.x * PS + 1] = red_l[threadIdx.x];
  }
}

// Merge of the splits: one workgroup per (row, head, 32 columns of D).  Thread
// (group gs, column c) loads the column of splits gs, gs + 8, ... up front; the weights
// exp2(m_s - M) and the normaliser come from one wave over the (m, l) pairs.
constexpr int kMergeThreads = 256;
constexpr int kMergeGroups = kMergeThreads / 32;

template <int D, int R, int PER>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(
    const float* __restrict__ part, float* __restrict__ out, int Hq, int Hkv, int Lq,
    int nsplit) {
  constexpr int PS = D + 4;
  constexpr int NSL = D / 32;
  const int slice = blockIdx.x % NSL;
  const int r = (blockIdx.x / NSL) % R;
  const int row = blockIdx.x / (NSL * R);
  const int bg = row / Lq, i = row - bg * Lq;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int c = threadIdx.x & 31, gs = threadIdx.x >> 5;
  const float* base = part + (long long)row * nsplit * R * PS + (long long)r * PS;
  __shared__ float s_red[kMergeThreads / 64];
  __shared__ float s_part[kMergeGroups][32];
  // every load of the slice at once (addresses clamped, values masked afterwards)
  float av[PER], mv[PER], lv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int s = min(gs + j * kMergeGroups, nsplit - 1);
    const float* ps = base + (long long)s * R * PS;
    av[j] = ps[4 + slice * 32 + c];
    mv[j] = ps[0];
    lv[j] = ps[1];
  }
  float M = neg_inf();
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (gs + j * kMergeGroups < nsplit) M = fmaxf(M, mv[j]);
  // block max (max is exact, any order)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = M;
  __syncthreads();
  M = s_red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, s_red[w]);
  float a = 0.f, lsum = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (gs + j * kMergeGroups < nsplit && mv[j] != neg_inf()) {
      const float wgt = fast_exp2(mv[j] - M);
      a = fmaf(wgt, av[j], a);
      lsum = fmaf(wgt, lv[j], lsum);
    }
  }
  __shared__ float s_l[kMergeGroups];
  s_part[gs][c] = a;
  if (c == 0) s_l[gs] = lsum;
  __syncthreads();
  if (gs == 0) {
    float t = 0.f, L = 0.f;
#pragma unroll
    for (int j = 0; j < kMergeGroups; ++j) { t += s_part[j][c]; L += s_l[j]; }
    out[(((long long)b * Hq + g * R + r) * Lq + i) * D + slice * 32 + c] = (L > 0.f) ? t / L : 0.f;
  }
}

// Bitmask rows: one workgroup per (b, KV head, query row).
template <typename T, int D, int R>
__global__ __launch_bounds__(kAttnThreads) void attn_bitmask_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const uint32_t* __restrict__ bitmask, float* __restrict__ out, int Hq, int Hkv, int Lq,
    int L, int L_cap, int q_pos0, float scale_log2, int kvdiv) {
  using G = Geo<T, D, R>;
  constexpr int EPL = G::EPL;
  const int row = blockIdx.x;
  const int bg = row / Lq, i = row - bg * Lq;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int pe = lane % G::LPR;
  const int nwords = (L + 31) / 32;
  const int L_r = min(q_pos0 + i + 1, L);
  const int nwords_act = (L_r + 31) / 32;
  __shared__ int s_list[kBmChunkWords * 32 + kRoundTokens];
  __shared__ int s_cnt;
  __shared__ float s_m[kAttnWaves * R], s_l[kAttnWaves * R], red_m[R], red_l[R];
  __shared__ float s_acc[kAttnWaves * R * D];
  __shared__ float red_acc[R * D];

  float qr[R][EPL];
  load_q<T, D, R>(q, (((long long)b * Hq + g * R) * Lq + i) * D, (long long)Lq * D, pe,
                  scale_log2, qr);
  SoftState<R, EPL> st;
  st.init();
  const T* kb = k + (long long)(bg / kvdiv) * L_cap * D + pe * EPL;
  const T* vb = v + (long long)(bg / kvdiv) * L_cap * D + pe * EPL;
  const uint32_t* brow = bitmask + (long long)row * nwords;
  for (int w0 = 0; w0 < nwords_act; w0 += kBmChunkWords) {
    __syncthreads();
    if (wid == 0) {
      const int w = w0 + lane;
      uint32_t bits = 0;
      if (lane < kBmChunkWords && w < nwords_act) {
        bits = brow[w];
        const int lim = L_r - w * 32;  // tokens after the row's own position never count
        if (lim < 32) bits &= (1u << lim) - 1u;
      }
      const int c = __popc(bits);
      int pos = wave_inclusive_sum(c) - c;
      for (uint32_t e = bits; e; e &= e - 1) s_list[pos++] = w * 32 + (__ffs(e) - 1);
      if (lane == 63) s_cnt = pos;
    }
    __syncthreads();
    const int cnt = s_cnt;
    for (int p0 = 0; p0 < cnt; p0 += kRoundTokens) {
      // pad the tail of the list with "no row" entries
      __syncthreads();
      if (threadIdx.x < kRoundTokens && p0 + threadIdx.x >= cnt) s_list[p0 + threadIdx.x] = -1;
      __syncthreads();
      wave_round<T, D, R>(kb, vb, s_list + p0, qr, st);
    }
  }
  block_reduce<T, D, R, kAttnThreads>(st, s_m, s_l, s_acc, red_m, red_l, red_acc);
  for (int j = threadIdx.x; j < R * D; j += kAttnThreads) {
    const int r = j / D, d = j - r * D;
    out[(((long long)b * Hq + g * R + r) * Lq + i) * D + d] =
        (red_l[r] > 0.f) ? red_acc[j] / red_l[r] : 0.f;
  }
}

struct SplitPlan {
  int nsplit, rounds;
};

// The matrix-core kernel sizes its splits so the grid is about what stays resident: a
// split of split_len list positions (a multiple of the 64-position block round).
struct MfPlan {
  int nsplit, split_len;
};

MfPlan plan_mfma(long long rows, int cap) {
  long long per_row = kMfTargetBlocks / rows;
  if (per_row < 1) per_row = 1;
  long long len = (cap + per_row - 1) / per_row;
  len = (len + kMfRound - 1) / kMfRound * kMfRound;
  if (len < kMfRound) len = kMfRound;
  long long ns = (cap + len - 1) / len;
  while (ns > kMaxSplits) {
    len += kMfRound;
    ns = (cap + len - 1) / len;
  }
  return {(int)ns, (int)len};
}

SplitPlan plan_for(int cap) {
  const int raw = (cap + kRoundTokens - 1) / kRoundTokens;
  const int rounds = (raw + kMaxSplits - 1) / kMaxSplits;
  const int per = kRoundTokens * rounds;
  return {(cap + per - 1) / per, rounds};
}

// splits per thread of the merge: the smallest power of two >= nsplit / 8
template <int D, int R>
hipError_t merge_t(hipStream_t s, const float* part, float* out, long long rows, int Hq, int Hkv,
                   int Lq, int nsplit) {
  const dim3 mgrid((unsigned)(rows * R * (D / 32)));
  const int per = (nsplit + kMergeGroups - 1) / kMergeGroups;
  if (per <= 4)
    hipLaunchKernelGGL((attn_merge_kernel<D, R, 4>), mgrid, dim3(kMergeThreads), 0, s, part, out, Hq, Hkv, Lq, nsplit);
  else if (per <= 8)
    hipLaunchKernelGGL((attn_merge_kernel<D, R, 8>), mgrid, dim3(kMergeThreads), 0, s, part, out, Hq, Hkv, Lq, nsplit);
  else if (per <= 16)
    hipLaunchKernelGGL((attn_merge_kernel<D, R, 16>), mgrid, dim3(kMergeThreads), 0, s, part, out, Hq, Hkv, Lq, nsplit);
  else if (per <= 32)
    hipLaunchKernelGGL((attn_merge_kernel<D, R, 32>), mgrid, dim3(kMergeThreads), 0, s, part, out, Hq, Hkv, Lq, nsplit);
  else if (per <= 64)
    hipLaunchKernelGGL((attn_merge_kernel<D, R, 64>), mgrid, dim3(kMergeThreads), 0, s, part, out, Hq, Hkv, Lq, nsplit);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int D, int R>
hipError_t idx_t(hipStream_t s, const void* q, const void* k, const void* v,
                 const int32_t* idx, const int32_t* count, float* out, int B, int Hq, int Hkv,
                 int Lq, int L_cap, int cap, float scale, void* ws, int kvdiv) {
  const long long rows = (long long)B * Hkv * Lq;
  float* part = (float*)ws;
  int nsplit;
  if constexpr (std::is_same<T, bf16_t>::value && D == 128) {
    const MfPlan sp = plan_mfma(rows, cap);
    nsplit = sp.nsplit;
    hipLaunchKernelGGL((attn_mfma_kernel<R>), dim3((unsigned)(sp.nsplit * rows)),
                       dim3(kMfThreads), 0, s, (const bf16_t*)q, (const bf16_t*)k,
                       (const bf16_t*)v, idx, count, part, Hq, Hkv, Lq, L_cap, cap,
                       scale * 1.4426950408889634f, sp.nsplit, sp.split_len, (int)rows, kvdiv);
  } else {
    const SplitPlan sp = plan_for(cap);
    nsplit = sp.nsplit;
    hipLaunchKernelGGL((attn_idx_kernel<T, D, R>), dim3((unsigned)(sp.nsplit * rows)),
                       dim3(kAttnThreads), 0, s, (const T*)q, (const T*)k, (const T*)v, idx,
                       count, part, Hq, Hkv, Lq, L_cap, cap, scale * 1.4426950408889634f,
                       sp.nsplit, sp.rounds, (int)rows, kvdiv);
  }
  return merge_t<D, R>(s, part, out, rows, Hq, Hkv, Lq, nsplit);
}


template <typename T, int D, int R>
hipError_t bm_t(hipStream_t s, const void* q, const void* k, const void* v,
                const uint32_t* bitmask, float* out, int B, int Hq, int Hkv, int Lq, int L,
                int L_cap, int q_pos0, float scale, int kvdiv) {
  const long long rows = (long long)B * Hkv * Lq;
  if constexpr (std::is_same<T, bf16_t>::value && D == 128 && R == 4) {
    if (Lq >= 32 && kvdiv == 1) {
      // 64 query rows per workgroup: each staged K/V tile serves eight waves
      return launch_prefill_mfma(s, q, k, v, bitmask, out, B, Hq, Hkv, Lq, L, L_cap, q_pos0,
                                 scale);
    }
  }
  hipLaunchKernelGGL((attn_bitmask_kernel<T, D, R>), dim3((unsigned)rows), dim3(kAttnThreads),
                     0, s, (const T*)q, (const T*)k, (const T*)v, bitmask, out, Hq, Hkv, Lq,
                     L, L_cap, q_pos0, scale * 1.4426950408889634f, kvdiv);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace(int dtype, int B, int Hq, int Hkv, int D, int Lq, int L, int cap) {
  (void)L;
  const long long rows = (long long)B * Hkv * Lq;
  const int R = Hq / Hkv;
  const int nsplit = (dtype == 1 && D == 128) ? plan_mfma(rows, cap).nsplit : plan_for(cap).nsplit;
  return (size_t)rows * nsplit * R * (D + 4) * sizeof(float);
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
                           int cap, float scale, void* ws, int kvdiv) {
  BUTLER_ATTN_DISPATCH(idx_t, s, q, k, v, idx, count, out, B, Hq, Hkv, Lq, L_cap, cap, scale, ws,
                       kvdiv);
}

hipError_t launch_attn_merge(hipStream_t s, const float* part, float* out, long long rows, int Hq,
                             int Hkv, int Lq, int D, int nsplit) {
  const int R = Hq / Hkv;
#define BUTLER_MG(DD, RR) \
  if (D == DD && R == RR) return merge_t<DD, RR>(s, part, out, rows, Hq, Hkv, Lq, nsplit);
  BUTLER_MG(128, 1) BUTLER_MG(128, 2) BUTLER_MG(128, 4) BUTLER_MG(128, 8)
  BUTLER_MG(64, 1) BUTLER_MG(64, 2) BUTLER_MG(64, 4) BUTLER_MG(64, 8)
#undef BUTLER_MG
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bitmask(hipStream_t s, int dtype, const void* q, const void* k,
                               const void* v, const uint32_t* bitmask, float* out, int B,
                               int Hq, int Hkv, int D, int Lq, int L, int L_cap, int q_pos0,
                               float scale, void* ws, int kvdiv) {
  (void)ws;
  BUTLER_ATTN_DISPATCH(bm_t, s, q, k, v, bitmask, out, B, Hq, Hkv, Lq, L, L_cap, q_pos0, scale,
                       kvdiv);
}

}  // namespace butler
