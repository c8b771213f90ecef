// Fixed-budget top-x + sink + window selection (TokenButler model card, Method and
// Memory requirements).
//
// Scores become order-preserving uint32 keys (score_key: NaN ranks as -inf, -0 as +0).
// The x-th largest key tau is found exactly by a most-significant-digit radix select
// over digits of 11, 11 and 10 bits: a pass histograms the next digit of the keys that
// share the prefix found so far, and a scan from the top bin finds the bin that holds the
// x-th largest key.  After the third digit tau is exact, together with the number of keys
// equal to tau that the budget still takes; the lowest-index ones are taken.  The emit
// walks the row in index order, so the index list comes out ascending.
//
// Workgroups never wait on one another inside a kernel (a device-wide release on this
// GPU writes back the XCD's L2, far too slow for a per-workgroup handshake); every
// hand-off between workgroups goes through a kernel boundary.  The first radix digit can
// come from the scorer (an optional per-row histogram of the top 11 key bits, see
// butler_score), which saves one pass over the scores.  Two schedules:
//
// Decode rows longer than 4096 tokens: kernels over chunks of 256 threads x 8 or 16 keys
// (4 to 32 in the pass fused with attention, by row length)
//   0  (only without the scorer's histogram) histogram of key bits 31..21
//   1  every chunk derives the first-digit bin b1, counts its tokens that are surely
//      selected (digit above b1, or a sink / window token) and packs the keys whose
//      digit is b1 into its own candidate region -- for scores of any spread only a
//      sliver of the row
//   2  every wave of every chunk resolves tau and the tie cut from the row's candidates
//      on its own with ballot counts, bit by bit (the same work everywhere: cheaper than
//      a kernel boundary while the candidates are few; beyond 256 candidates through the
//      second digit, and past 2048 candidates of one second digit the whole workgroup
//      runs radix passes), derives its output offset from the per-chunk counts
//      and emits its bitmask words and indices through 64-token ballot words; the chunk-0
//      workgroup writes the row count and clears the histogram.
//
// Other rows (short decode rows; calls with several query rows of more than 8192 tokens --
//   those up to 8192 take one wave per row, in select_rows.hip): one workgroup per row, 64 to
//   1024 threads sized to the row, holds the row's keys in VGPRs (16 to 64 per thread,
//   strided so that a wave's ballot covers 64 consecutive tokens), builds the digit
//   histograms in LDS (the first from the scorer's histogram when given), and emits
//   through 64-token ballot words with two block-wide scans over the words (tie ranks,
//   then output positions).
//
// Single-row calls with selection-cache flags skip the selection of kept (b, KV heads) in
// every kernel, so the workspace state stays as it was; one workgroup of the row only
// re-takes the recent window at the current length in the kept list (and bitmask).
#include "attn_tile.h"
#include "common.h"
#include "kernels.h"
#include "select_rule.h"

#include <type_traits>

namespace butler {
namespace {

// Among hist[0..nbins), scanned from the top bin down, the bin that holds the need-th
// largest key, and the rank left inside it.  All NT threads call it.
template <int NT>
__device__ void find_bin_from_top(const uint32_t* hist, int nbins, int need, int* tmp,
                                  int* out_bin, int* out_need) {
  const int per = nbins / NT;
  const int hi = nbins - threadIdx.x * per;  // this thread covers bins [hi - per, hi)
  int local = 0;
  for (int j = 1; j <= per; ++j) local += (int)hist[hi - j];
  int total;
  int above = block_exclusive_sum<NT>(local, total, tmp);
  if (above < need && need <= above + local) {
    for (int j = 1; j <= per; ++j) {
      const int c = (int)hist[hi - j];
      if (above + c >= need) {
        *out_bin = hi - j;
        *out_need = need - above;
        break;
      }
      above += c;
    }
  }
  __syncthreads();
}

// Same from the bottom: the bin holding the need-th smallest value.
template <int NT>
__device__ void find_bin_from_bottom(const uint32_t* hist, int nbins, int need, int* tmp,
                                     int* out_bin, int* out_need) {
  const int per = nbins / NT;
  const int lo = threadIdx.x * per;
  int local = 0;
  for (int j = 0; j < per; ++j) local += (int)hist[lo + j];
  int total;
  int below = block_exclusive_sum<NT>(local, total, tmp);
  if (below < need && need <= below + local) {
    for (int j = 0; j < per; ++j) {
      const int c = (int)hist[lo + j];
      if (below + c >= need) {
        *out_bin = lo + j;
        *out_need = need - below;
        break;
      }
      below += c;
    }
  }
  __syncthreads();
}

// A row the selection cache keeps (keep != 0): its previous selection stands, but the
// recent window is re-taken at the current length L, so tokens appended since the
// selection was made are attended.  The list becomes its entries below
// w_lo = max(0, L - n_window) followed by w_lo .. L-1 (at most cap entries), and the
// bitmask gains the window's bits.  NT threads of one workgroup; the entries are counted
// before any is overwritten.
template <int NT>
__device__ void refresh_kept_row(long long row, int L, int n_window, int cap,
                                 int32_t* __restrict__ idx, uint32_t* __restrict__ bitmask,
                                 int32_t* __restrict__ count, int* tmp) {
  const int w_lo = max(0, L - n_window);
  if (idx) {
    int32_t* irow = idx + row * (long long)cap;
    const int n_old = min(max((int)count[row], 0), cap);
    int below = 0;
    for (int j = threadIdx.x; j < n_old; j += NT) below += (irow[j] < w_lo) ? 1 : 0;
    int p;
    block_exclusive_sum<NT>(below, p, tmp);   // p: the entries kept below the window
    for (int j = threadIdx.x; j < L - w_lo && p + j < cap; j += NT) irow[p + j] = w_lo + j;
    if (threadIdx.x == 0) count[row] = min(p + (L - w_lo), cap);
  }
  if (bitmask) {
    const int nwords = (L + 31) / 32;
    uint32_t* brow = bitmask + row * (long long)nwords;
    int bits = 0;
    for (int wd = threadIdx.x; wd < nwords; wd += NT) {
      uint32_t v = brow[wd];
      if (32 * wd + 32 > w_lo) {
        const int lo = max(w_lo - 32 * wd, 0), hi = min(L - 32 * wd, 32);   // bits [lo, hi)
        v |= (hi >= 32 ? 0xffffffffu : ((1u << hi) - 1u)) & ~((1u << lo) - 1u);
        brow[wd] = v;
      }
      bits += __popc(v);
    }
    int total;
    block_exclusive_sum<NT>(bits, total, tmp);
    if (!idx && threadIdx.x == 0) count[row] = total;   // without a list: the row's bits
  }
}

// ---------------------------------------------------------------------------
// one workgroup per row, keys in VGPRs
// ---------------------------------------------------------------------------

// In-place exclusive scan of a[0..n) (LDS) by NT threads; returns the total.
template <int NT>
__device__ __forceinline__ int block_scan_array(int* a, int n, int* tmp) {
  const int per = (n + NT - 1) / NT;
  const int lo = threadIdx.x * per;
  int local = 0;
  for (int j = 0; j < per; ++j)
    if (lo + j < n) local += a[lo + j];
  int total;
  int run = block_exclusive_sum<NT>(local, total, tmp);
  for (int j = 0; j < per; ++j) {
    if (lo + j < n) {
      const int v = a[lo + j];
      a[lo + j] = run;
      run += v;
    }
  }
  __syncthreads();
  return total;
}

// Thread tid owns tokens tid + NT*j (j < KPT): for a fixed j the 64 lanes of a wave hold
// 64 consecutive tokens, so a ballot is one 64-token word of the row in index order
// (word j*NW + wave).
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void select_row_kernel(
    const float* __restrict__ scores, int num, int den, int n_sink, int n_window,
    int32_t* __restrict__ idx, uint32_t* __restrict__ bitmask, int32_t* __restrict__ count,
    int Lq, int L, int cap, int q_pos0, int causal, uint32_t* __restrict__ ghist,
    const int32_t* __restrict__ keep, int fo) {
  constexpr int NW = NT / 64;
  constexpr int MAXW = NT * KPT / 64;
  const long long row = blockIdx.x;
  __shared__ int tmp[NW];
  if (keep && keep[row]) {   // single-row calls: the cached selection stands, window refreshed
    refresh_kept_row<NT>(row, L, n_window, cap, idx, bitmask, count, tmp);
    return;
  }
  const int i = (int)(row % Lq);
  const int L_r = causal ? min(q_pos0 + i + 1, L) : L;
  int k;
  const int mode = row_mode(L_r, num, den, n_sink, n_window, fo, k);
  const int w_lo = max(0, L_r - n_window);
  const float* s = scores + row * (long long)L;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;

  __shared__ uint32_t hist[2048];
  __shared__ int sh_bin, sh_need;
  __shared__ int wtie[MAXW], wcnt[MAXW];
  __shared__ uint64_t wsel[MAXW];

  // all loads at once, from clamped addresses, before any key is formed (a conversion
  // next to each load would make the compiler wait for each load in turn)
  float raw[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) raw[j] = s[min((int)threadIdx.x + NT * j, L_r - 1)];
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    key[j] = rank_key(raw[j], (int)threadIdx.x + NT * j, n_sink, w_lo, fo);
  auto valid = [&](int j) { return (int)threadIdx.x + NT * j < L_r; };

  uint32_t tau = (mode == kModeAll) ? 0u : 0xffffffffu;
  int need = 0;
  if (ghist && mode != kModeNormal) {
    // the scorer's histogram is not needed, but it must be left zero-filled
    uint32_t* gh = ghist + row * 2048;
    for (int j = threadIdx.x; j < 2048; j += NT) gh[j] = 0u;
  }
  if (mode == kModeNormal) {
    uint32_t prefix = 0, pmask = 0;
    need = k;
    const int shifts[3] = {21, 10, 0};
    const int bins[3] = {2048, 2048, 1024};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int sh = shifts[p], nb = bins[p];
      if (p == 0 && ghist) {
        uint32_t* gh = ghist + row * 2048;
        for (int j = threadIdx.x; j < 2048; j += NT) { hist[j] = gh[j]; gh[j] = 0u; }
        __syncthreads();
      } else {
        for (int j = threadIdx.x; j < nb; j += NT) hist[j] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KPT; ++j)
          if (valid(j) && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> sh) & (nb - 1)], 1u);
        __syncthreads();
      }
      find_bin_from_top<NT>(hist, nb, need, tmp, &sh_bin, &sh_need);
      prefix |= (uint32_t)sh_bin << sh;
      pmask |= (uint32_t)(nb - 1) << sh;
      need = sh_need;
      __syncthreads();
    }
    tau = prefix;
  }

  // ---- emit in index order -------------------------------------------------------
  // rank of every key equal to tau among the row's equal keys, in index order
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint64_t e = __ballot(valid(j) && key[j] == tau);
    if (lane == 0) wtie[j * NW + wid] = __popcll(e);
  }
  __syncthreads();
  block_scan_array<NT>(wtie, MAXW, tmp);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int t = (int)threadIdx.x + NT * j;
    const bool v = valid(j);
    const bool eq = v && key[j] == tau;
    const uint64_t e = __ballot(eq);
    const int rank = wtie[j * NW + wid] + __popcll(e & lt);
    bool sel = v && (t < n_sink || t >= w_lo || key[j] > tau);
    if (eq) sel = sel || mode == kModeAll || (mode == kModeNormal && rank < need);
    const uint64_t b = __ballot(sel);
    if (lane == 0) { wsel[j * NW + wid] = b; wcnt[j * NW + wid] = __popcll(b); }
  }
  __syncthreads();
  const int total = block_scan_array<NT>(wcnt, MAXW, tmp);
  if (idx) {
    int32_t* irow = idx + row * (long long)cap;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int w = j * NW + wid;
      const uint64_t b = wsel[w];
      if ((b >> lane) & 1ull) {
        const int pos = wcnt[w] + __popcll(b & lt);
        if (pos < cap) irow[pos] = (int)threadIdx.x + NT * j;
      }
    }
  }
  if (bitmask) {
    const int nwords = (L + 31) / 32;
    uint32_t* brow = bitmask + row * (long long)nwords;
    for (int j = threadIdx.x; j < nwords; j += NT) {
      const int w = j >> 1;
      brow[j] = (w < MAXW) ? (uint32_t)(wsel[w] >> (32 * (j & 1))) : 0u;
    }
  }
  if (threadIdx.x == 0) count[row] = total;
}

// ---------------------------------------------------------------------------
// decode rows longer than 4096 tokens: two (or three) kernels over token chunks
// ---------------------------------------------------------------------------

constexpr int kMbThreads = 256;
constexpr int kMbWaves = kMbThreads / 64;
constexpr int kFinStage = 2048;   // second-digit candidates gathered in LDS

// Block-wide sums of three ints over the kMbThreads threads; every thread gets the totals.
__device__ __forceinline__ int3 block_sum3(int a, int b, int c, int3* tmp) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
    c += __shfl_xor(c, o);
  }
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = make_int3(a, b, c);
  __syncthreads();
  int3 r = make_int3(0, 0, 0);
#pragma unroll
  for (int w = 0; w < kMbThreads / 64; ++w) {
    r.x += tmp[w].x;
    r.y += tmp[w].y;
    r.z += tmp[w].z;
  }
  __syncthreads();
  return r;
}

#ifndef BUTLER_SEL_KPT_LO
#define BUTLER_SEL_KPT_LO 8
#endif
#ifndef BUTLER_SEL_KPT_HI
#define BUTLER_SEL_KPT_HI 16
#endif
#ifndef BUTLER_SEL_KPT_SPLIT
#define BUTLER_SEL_KPT_SPLIT 131072
#endif

// Keys per thread of the chunk kernels: a chunk is kMbThreads * kpt tokens.  Longer rows
// take longer chunks, so the per-workgroup fixed work (the first-digit search, the
// candidate resolution) is shared by more tokens.
int kpt_for(int L) { return L <= BUTLER_SEL_KPT_SPLIT ? BUTLER_SEL_KPT_LO : BUTLER_SEL_KPT_HI; }

struct RowState {
  uint32_t b1;     // first-digit bin of the x-th largest key
  int need;        // rank of the x-th largest key inside that bin (1-based)
  uint32_t epoch;  // this call's number: which second-digit histogram is live
  int nb1;         // keys of the row in bin b1: the candidates
};

// Rows with more candidates than this sort each chunk's candidates by their coarse second
// digit (key bits 20..15), so that the finishing pass reads only the coarse bin of tau.
constexpr int kMbFew = 256;

struct MbWs {
  uint32_t* hist1;               // [rows][2048]   first-digit counts, zero between calls
  RowState* state;               // [rows]
  int* defcnt;                   // [rows][nchunk] tokens of the chunk that are surely selected
  int* ncand;                    // [rows][nchunk] candidates the chunk appended
  uint32_t* epoch;               // [rows]         calls made so far (never reset)
  uint32_t* hist2;               // [2][rows][64]  coarse second-digit (key bits 20..15)
                                 //                counts of the candidates of rows with many;
                                 //                buffer epoch % 2 is filled, the other is zero
  uint32_t* ctab;                // [rows][nchunk][64]  rows with many candidates: per chunk
                                 //                and coarse bin c, the candidates in bins above
                                 //                c (bits 0..15: where bin c starts in the
                                 //                sorted region) and how many of them are not
                                 //                sink / window tokens (bits 16..31)
  uint2* cand;                   // [rows][nchunk][chunk tokens]  each chunk's candidates,
                                 //                (key, index | sink/window flag << 31), packed
                                 //                from the start of the chunk's own region
                                 //                (by descending coarse bin in rows with many)
};

// Chunks of a row the finishing pass can index (L <= 8M tokens at 4096 tokens per chunk).
constexpr int kMbMaxChunks = 2048;

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

long long nchunk_k(int L, int kpt) {
  const int chunk = kMbThreads * kpt;
  return (L + chunk - 1) / chunk;
}

long long nchunk_for(int L) { return nchunk_k(L, kpt_for(L)); }

// The workspace starts with the state that lives from one call to the next (the
// first-digit histogram, the call counters, the coarse histograms, the row states): its
// layout depends only on the number of rows, so one buffer sized for the longest row
// serves calls of any length.  The per-chunk arrays behind it are rewritten by every call.
size_t mb_state_bytes(long long rows) {
  return al256(rows * 2048 * 4) + al256(rows * 4) + al256(2 * rows * 64 * 4) +
         al256(rows * sizeof(RowState));
}

size_t mb_bytes_k(long long rows, int L, int kpt) {
  const long long nchunk = nchunk_k(L, kpt);
  return mb_state_bytes(rows) + 2 * al256(rows * nchunk * 4) +
         al256((size_t)rows * nchunk * 64 * 4) +
         al256((size_t)rows * nchunk * kMbThreads * kpt * sizeof(uint2));
}

size_t mb_bytes(long long rows, int L) { return mb_bytes_k(rows, L, kpt_for(L)); }

MbWs carve_k(void* ws, long long rows, int L, int kpt) {
  const long long nchunk = nchunk_k(L, kpt);
  char* p = (char*)ws;
  MbWs w;
  w.hist1 = (uint32_t*)p;                 p += al256(rows * 2048 * sizeof(uint32_t));
  w.epoch = (uint32_t*)p;                 p += al256(rows * 4);
  w.hist2 = (uint32_t*)p;                 p += al256(2 * rows * 64 * 4);
  w.state = (RowState*)p;                 p += al256(rows * sizeof(RowState));
  w.defcnt = (int*)p;                     p += al256(rows * nchunk * sizeof(int));
  w.ncand = (int*)p;                      p += al256(rows * nchunk * sizeof(int));
  w.ctab = (uint32_t*)p;                  p += al256((size_t)rows * nchunk * 64 * 4);
  w.cand = (uint2*)p;
  return w;
}

MbWs carve(void* ws, long long rows, int L) { return carve_k(ws, rows, L, kpt_for(L)); }

// The KPT keys of tokens t0 .. t0+KPT-1 (all requested at once); returns how many exist.
template <int KPT>
__device__ __forceinline__ int load_keys(const float* s, int t0, int L, uint32_t (&key)[KPT]) {
  const int nv = max(0, min(KPT, L - t0));
  if (nv == KPT && ((((uintptr_t)(s + t0)) & 15u) == 0)) {
    float4 a[KPT / 4];
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) a[q] = *reinterpret_cast<const float4*>(s + t0 + 4 * q);
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) {
      key[4 * q] = score_key(a[q].x);
      key[4 * q + 1] = score_key(a[q].y);
      key[4 * q + 2] = score_key(a[q].z);
      key[4 * q + 3] = score_key(a[q].w);
    }
  } else {
    float f[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) f[j] = s[min(t0 + j, L - 1)];
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = score_key(f[j]);
  }
  return nv;
}

// first-digit histogram, when the scorer did not produce it
template <int KPT>
__global__ __launch_bounds__(kMbThreads) void mb_hist1_kernel(const float* __restrict__ scores,
                                                              int num, int den, int n_sink,
                                                              int n_window, int fo, int L,
                                                              int rows,
                                                              uint32_t* __restrict__ ghist,
                                                              const int32_t* __restrict__ keep) {
  const int row = blockIdx.x % rows, chunk = blockIdx.x / rows;
  if (keep && keep[row]) return;
  int k;
  if (row_mode(L, num, den, n_sink, n_window, fo, k) != kModeNormal) return;
  __shared__ uint32_t h[2048];
  for (int j = threadIdx.x; j < 2048; j += kMbThreads) h[j] = 0u;
  __syncthreads();
  uint32_t key[KPT];
  const int t0 = (chunk * kMbThreads + threadIdx.x) * KPT;
  const int nv = load_keys<KPT>(scores + (long long)row * L, t0, L, key);
  const int w_lo = max(0, L - n_window);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (fo && (t0 + j < n_sink || t0 + j >= w_lo)) key[j] = 0u;   // forced: below every score
    if (j < nv) atomicAdd(&h[key[j] >> 21], 1u);
  }
  __syncthreads();
  uint32_t* gh = ghist + (long long)row * 2048;
  for (int j = threadIdx.x; j < 2048; j += kMbThreads)
    if (h[j]) atomicAdd(&gh[j], h[j]);
}

// ---- wave-level pieces: every wave works on its own, no barrier ----

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int ballot_count(bool p) { return __popcll(__ballot(p)); }

// The bin of a 2048-bin histogram (global, 16-byte aligned) that holds the need-th largest
// key, and the rank left inside it.  Lane l sums bins [2048 - 32(l+1), 2048 - 32l), the
// lanes scan from the top, and the lane whose range holds the rank walks its 32 bins.
__device__ __forceinline__ void wave_find_top(const uint32_t* __restrict__ gh, int need,
                                              uint32_t& bin, int& rest, int& count) {
  const int lane = threadIdx.x & 63;
  const int lo = 2048 - 32 * (lane + 1);
  uint32_t c[32];
  const uint4* p = reinterpret_cast<const uint4*>(gh + lo);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 v = p[q];
    c[4 * q] = v.x;
    c[4 * q + 1] = v.y;
    c[4 * q + 2] = v.z;
    c[4 * q + 3] = v.w;
  }
  int local = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) local += (int)c[i];
  const int incl = wave_inclusive_sum(local);
  const int excl = incl - local;
  const unsigned long long m = __ballot(excl < need && need <= incl);
  const int src = m ? (int)__ffsll((unsigned long long)m) - 1 : 0;
  int above = excl, b = lo, r = 1, cnt = 0;
  bool found = false;
#pragma unroll
  for (int i = 31; i >= 0; --i) {
    if (!found && above + (int)c[i] >= need) {
      b = lo + i;
      r = need - above;
      cnt = (int)c[i];
      found = true;
    }
    if (!found) above += (int)c[i];
  }
  bin = (uint32_t)__shfl(b, src);
  rest = __shfl(r, src);
  count = __shfl(cnt, src);
}

// The same over a 64-bin histogram: the bin c holding the need-th largest key, how many
// keys lie in the bins above it, and how many in it.
__device__ __forceinline__ void wave_find_top64(const uint32_t* __restrict__ gh, int need,
                                                uint32_t& bin, int& above, int& count) {
  const int lane = threadIdx.x & 63;
  const int v = (int)gh[63 - lane];
  const int incl = wave_inclusive_sum(v);
  const unsigned long long m = __ballot(incl - v < need && need <= incl);
  const int src = m ? (int)__ffsll((unsigned long long)m) - 1 : 0;
  bin = (uint32_t)(63 - src);
  above = __shfl(incl - v, src);
  count = __shfl(v, src);
}

// One wave resolves, from n <= 64*Q candidates (all share the key bits above top_bit,
// given in prefix, and the need-th largest of them is the x-th largest key of the row;
// load(j) gives candidate j, called by all 64 lanes at once), tau bit by bit from
// top_bit down -- a ballot count of the candidates that carry the trial bit -- then, when
// the budget splits the keys equal to tau, the tie cut bit by bit over their indices
// (lowest indices first), and the counts of the selected candidates that are not sink /
// window tokens: all of them, and those before index c_lo.
template <int Q, typename Load>
__device__ void wave_resolve(const Load& load, int n, uint32_t prefix, int top_bit, int need,
                             int c_lo, uint32_t& tau, int& tie_cut, int& sel_all,
                             int& sel_before) {
  const int lane = threadIdx.x & 63;
  uint32_t ck[Q], ci[Q];
  bool cv[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    cv[q] = lane + 64 * q < n;
    const uint2 e = load(min(lane + 64 * q, n - 1));
    ck[q] = e.x;
    ci[q] = e.y;
  }
  uint32_t P = prefix;
  int kk = need;
  for (int bit = top_bit; bit >= 0; --bit) {
    const uint32_t hi = 0xffffffffu << (bit + 1);
    int c1 = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q)
      c1 += ballot_count(cv[q] && (ck[q] & hi) == P && ((ck[q] >> bit) & 1u));
    if (c1 >= kk) P |= 1u << bit;
    else kk -= c1;
  }
  tau = P;
  int ties = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) ties += ballot_count(cv[q] && ck[q] == tau);
  if (kk >= ties) {
    tie_cut = 0x7fffffff;
  } else {
    uint32_t I = 0u;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t hi = (0x7fffffffu << (bit + 1)) & 0x7fffffffu;
      int c0 = 0;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const uint32_t t = ci[q] & 0x7fffffffu;
        c0 += ballot_count(cv[q] && ck[q] == tau && (t & hi) == I && !((t >> bit) & 1u));
      }
      if (c0 < kk) {
        kk -= c0;
        I |= 1u << bit;
      }
    }
    tie_cut = (int)I;
  }
  sel_all = 0;
  sel_before = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int t = (int)(ci[q] & 0x7fffffffu);
    const bool s = cv[q] && !(ci[q] >> 31) && (ck[q] > tau || (ck[q] == tau && t <= tie_cut));
    sel_all += ballot_count(s);
    sel_before += ballot_count(s && t < c_lo);
  }
}

// Candidate j (0 <= j < n) of a row whose chunks packed their candidates into regions of
// ch entries, taken from each region in turn: cp (LDS) holds the exclusive prefix of the
// counts taken, so j lies in the last chunk whose prefix is <= j (chunks that give none
// repeat the prefix).
struct CandRow {
  const uint2* base;   // the row's first region
  const int* cp;       // [nchunk] exclusive prefix of the counts taken from each region
  const int* off;      // [nchunk] where they start in the region (null: at its start)
  int nchunk, ch;
  __device__ __forceinline__ uint2 operator()(int j) const {
    int lo = 0, hi = nchunk - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cp[mid] <= j) lo = mid;
      else hi = mid - 1;
    }
    return base[(long long)lo * ch + min((off ? off[lo] : 0) + (j - cp[lo]), ch - 1)];
  }
};

// The same for rows with many candidates, by the whole workgroup: radix passes over bits
// 20..10 and 9..0 of the candidates (LDS histograms, read from the chunk regions), the tie
// quota, the index radix of the ties, then the two counts.
__device__ void block_resolve(const CandRow at, int n, uint32_t b1, int need, int c_lo,
                              uint32_t* h, int* tmp, int3* tmp3, int* sh, uint32_t& tau,
                              int& tie_cut, int& sel_all, int& sel_before) {
  uint32_t prefix = b1 << 21, pmask = 0xffe00000u;
  const int shifts[2] = {10, 0};
  const int bins[2] = {2048, 1024};
  for (int p = 0; p < 2; ++p) {
    for (int j = threadIdx.x; j < 2048; j += kMbThreads) h[j] = 0u;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += kMbThreads) {
      const uint32_t kk = at(j).x;
      if ((kk & pmask) == prefix) atomicAdd(&h[(kk >> shifts[p]) & (uint32_t)(bins[p] - 1)], 1u);
    }
    __syncthreads();
    find_bin_from_top<kMbThreads>(h, bins[p], need, tmp, &sh[0], &sh[1]);
    prefix |= (uint32_t)sh[0] << shifts[p];
    pmask |= (uint32_t)(bins[p] - 1) << shifts[p];
    need = sh[1];
  }
  tau = prefix;
  int mine = 0;
  for (int j = threadIdx.x; j < n; j += kMbThreads) mine += (at(j).x == tau) ? 1 : 0;
  int ties;
  block_exclusive_sum<kMbThreads>(mine, ties, tmp);
  if (need >= ties) {
    tie_cut = 0x7fffffff;
  } else {
    // the need-th smallest index among the keys equal to tau: bits 30..20, 19..10, 9..0
    uint32_t pre = 0u, pm = 0u;
    int nd = need;
    const int ish[3] = {20, 10, 0};
    const uint32_t iw[3] = {2048u, 1024u, 1024u};
    for (int p = 0; p < 3; ++p) {
      for (int j = threadIdx.x; j < 2048; j += kMbThreads) h[j] = 0u;
      __syncthreads();
      for (int j = threadIdx.x; j < n; j += kMbThreads) {
        const uint2 c = at(j);
        const uint32_t t = c.y & 0x7fffffffu;
        if (c.x == tau && (t & pm) == pre) atomicAdd(&h[(t >> ish[p]) & (iw[p] - 1u)], 1u);
      }
      __syncthreads();
      find_bin_from_bottom<kMbThreads>(h, 2048, nd, tmp, &sh[0], &sh[1]);
      pre |= (uint32_t)sh[0] << ish[p];
      pm |= (iw[p] - 1u) << ish[p];
      nd = sh[1];
    }
    tie_cut = (int)pre;
  }
  int sa = 0, sb = 0;
  for (int j = threadIdx.x; j < n; j += kMbThreads) {
    const uint2 c = at(j);
    if (c.y & 0x80000000u) continue;  // sink / window tokens are counted as sure
    const int t = (int)c.y;
    if (c.x > tau || (c.x == tau && t <= tie_cut)) {
      ++sa;
      sb += (t < c_lo) ? 1 : 0;
    }
  }
  const int3 ss = block_sum3(sa, sb, 0, tmp3);
  sel_all = ss.x;
  sel_before = ss.y;
}

// Chunk pass.  Thread i of the workgroup holds tokens c_lo + i + 256 j (j < KPT), so a
// wave's ballot covers 64 consecutive tokens.  Every wave derives the first-digit bin b1
// from the row's histogram on its own, counts its tokens that are surely selected (digit
// above b1, or sink / window) and packs the keys whose first digit is b1 into the chunk's
// own candidate region: no position is taken from a shared counter (64 workgroups of a
// row serialised on one such atomic).  In rows with few candidates they go in wave order;
// in rows with many, sorted by descending coarse second digit, with the chunk's table of
// where each coarse bin starts and its counts added to the row's coarse histogram.
template <int KPT>
__global__ __launch_bounds__(kMbThreads) void mb_cand_kernel(const float* __restrict__ scores,
                                                             int num, int den, int n_sink,
                                                             int n_window, int L, int rows,
                                                             const uint32_t* __restrict__ ghist,
                                                             MbWs w,
                                                             const int32_t* __restrict__ keep,
                                                             int fo) {
  const int row = blockIdx.x % rows, chunk = blockIdx.x / rows;
  if (keep && keep[row]) return;
  const int nchunk = gridDim.x / rows;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int k;
  const int mode = row_mode(L, num, den, n_sink, n_window, fo, k);
  const int c_lo = chunk * kMbThreads * KPT;
  const float* srow = scores + (long long)row * L;
  float f[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) f[j] = srow[min(c_lo + (int)threadIdx.x + kMbThreads * j, L - 1)];
  uint32_t b1 = 0u;
  int need = 0, nb1 = 0;
  const uint32_t epoch = w.epoch[row];
  if (mode == kModeNormal) {
    wave_find_top(ghist + (long long)row * 2048, k, b1, need, nb1);
    if (chunk == 0 && threadIdx.x == 0) w.state[row] = RowState{b1, need, epoch, nb1};
  }
  const bool sorted = nb1 > kMbFew;   // the same for every workgroup of the row
  __shared__ int s_hc[64], s_hn[64], s_base[64];
  if (sorted && threadIdx.x < 64) {
    s_hc[threadIdx.x] = 0;
    s_hn[threadIdx.x] = 0;
  }
  const int w_lo = max(0, L - n_window);
  int ndef = 0, ncw = 0;
  unsigned long long cm[KPT];
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int t = c_lo + (int)threadIdx.x + kMbThreads * j;
    key[j] = rank_key(f[j], t, n_sink, w_lo, fo);
    const bool valid = t < L;
    const bool forced = t < n_sink || t >= w_lo;
    bool def, cand;
    if (mode == kModeNormal) {
      const uint32_t top = key[j] >> 21;
      def = valid && (forced || top > b1);
      cand = valid && top == b1;
    } else {
      def = valid && (forced || mode == kModeAll);
      cand = false;
    }
    ndef += def ? 1 : 0;
    cm[j] = __ballot(cand);
    ncw += __popcll(cm[j]);
  }
  ndef = wave_sum_i(ndef);
  // one atomic per workgroup (same-address atomics serialise): the waves' counts meet in LDS
  __shared__ int s_n[kMbWaves], s_d[kMbWaves];
  if (lane == 0) {
    s_n[wid] = ncw;
    s_d[wid] = ndef;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int tn = 0, td = 0;
#pragma unroll
    for (int v = 0; v < kMbWaves; ++v) {
      tn += s_n[v];
      td += s_d[v];
    }
    const long long e = (long long)row * nchunk + chunk;
    w.defcnt[e] = td;
    w.ncand[e] = tn;
  }
  uint2* crow = w.cand + ((long long)row * nchunk + chunk) * (kMbThreads * KPT);
  if (!sorted) {
    if (ncw) {
      int pos = 0;
#pragma unroll
      for (int v = 0; v < kMbWaves; ++v) pos += (v < wid) ? s_n[v] : 0;
      const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        if ((cm[j] >> lane) & 1ull) {
          const int t = c_lo + (int)threadIdx.x + kMbThreads * j;
          const uint32_t flag = (t < n_sink || t >= w_lo) ? 0x80000000u : 0u;
          crow[pos + __popcll(cm[j] & lt)] = make_uint2(key[j], (uint32_t)t | flag);
        }
        pos += __popcll(cm[j]);
      }
    }
    return;
  }
  // many candidates in the row: a counting sort by coarse bin (the order inside a bin is
  // immaterial, the finishing pass uses only the keys and indices)
  int slot[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    slot[j] = 0;
    if ((cm[j] >> lane) & 1ull) {
      const int t = c_lo + (int)threadIdx.x + kMbThreads * j;
      const int cb = (int)((key[j] >> 15) & 63u);
      slot[j] = atomicAdd(&s_hc[cb], 1);
      if (!(t < n_sink || t >= w_lo)) atomicAdd(&s_hn[cb], 1);
    }
  }
  __syncthreads();
  if (wid == 0) {
    // lane l takes bin 63 - l: the exclusive scan counts the candidates in the bins above
    const int cb = 63 - lane;
    const int hc = s_hc[cb], hn = s_hn[cb];
    const int ac = wave_inclusive_sum(hc) - hc, an = wave_inclusive_sum(hn) - hn;
    w.ctab[((long long)row * nchunk + chunk) * 64 + cb] = (uint32_t)ac | ((uint32_t)an << 16);
    s_base[cb] = ac;
    if (hc) atomicAdd(&w.hist2[((long long)(epoch & 1u) * rows + row) * 64 + cb], (uint32_t)hc);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if ((cm[j] >> lane) & 1ull) {
      const int t = c_lo + (int)threadIdx.x + kMbThreads * j;
      const uint32_t flag = (t < n_sink || t >= w_lo) ? 0x80000000u : 0u;
      crow[s_base[(key[j] >> 15) & 63u] + slot[j]] = make_uint2(key[j], (uint32_t)t | flag);
    }
  }
}

// Finishing pass, one workgroup per chunk, tokens held as in the chunk pass.  Every wave
// sums the row's per-chunk counts; the workgroup indexes the chunks' candidate regions
// (a prefix of their counts in LDS) and, while they are few, gathers the candidates into
// LDS, where every wave resolves tau and the tie cut on its own (the whole workgroup only
// for a flood of equal keys): the 64-token ballot words of the chunk are
// prefix-summed once through LDS, and each wave writes its words' indices coalesced and
// their bitmask words.  The chunk-0 workgroup writes the row count and clears the row's
// histogram (nothing in this kernel reads it).
// Attention operands of the fused finishing pass (R > 0): bf16, D = 128, one query row.
struct MbAttn {
  const bf16_t* q;      // [B, Hq, 1, 128]
  const bf16_t* k;      // [B, Hkv, L_cap, 128]
  const bf16_t* v;
  float* part;          // [rows][nchunk][R][128 + 4]: (max, sum, -, -, acc[128]) per head
  int Hq, Hkv, L_cap;   // Hkv: selection heads; kvdiv of them share a cache row
  float scale_log2;
  int kvdiv;
};

#ifndef BUTLER_SA_RING
#define BUTLER_SA_RING 2
#endif
constexpr int kMaRound = kMbWaves * 16;   // list positions per workgroup round (a tile per wave)
constexpr int kMaRing = BUTLER_SA_RING;   // tiles per wave in the load ring
constexpr int kMaPad = (kMaRing + 1) * kMaRound;   // ring prefetch past the list end

template <int KPT, int R>
__global__ __launch_bounds__(kMbThreads) void mb_finish_kernel(
    const float* __restrict__ scores, int num, int den, int n_sink, int n_window, int L,
    int rows, int cap, int32_t* __restrict__ idx, uint32_t* __restrict__ bitmask,
    int32_t* __restrict__ count, uint32_t* __restrict__ ghist, MbWs w,
    const int32_t* __restrict__ keep, MbAttn at, int fo) {
  constexpr int NWD = kMbWaves * KPT;   // 64-token words per chunk
  static_assert(NWD <= 128, "two words per lane in the prefix scan");
  const int row = blockIdx.x % rows, chunk = blockIdx.x / rows;
  if (R == 0 && keep && keep[row]) {   // the cached selection stands, window refreshed
    __shared__ int ktmp[kMbWaves];
    if (chunk == 0) refresh_kept_row<kMbThreads>(row, L, n_window, cap, idx, bitmask, count, ktmp);
    return;
  }
  const int nchunk = gridDim.x / rows;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // fused attention: the group's query heads as the MFMA B operand, requested first
  bf16x8_t qf[4];
  if constexpr (R > 0) {
    const int b = row / at.Hkv, g = row - b * at.Hkv;
    const int quad = lane >> 4, pe = lane & 15;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (pe < R)
        raw = *reinterpret_cast<const uint4*>(at.q + ((long long)b * at.Hq + g * R + pe) * 128 +
                                              kk * 32 + 8 * quad);
      qf[kk] = as_bf16x8(raw);
    }
  }
  int k;
  const int mode = row_mode(L, num, den, n_sink, n_window, fo, k);
  __shared__ uint32_t h[2048];
  __shared__ int tmp[kMbWaves];
  __shared__ int3 tmp3[kMbWaves];
  __shared__ int sh[2];
  __shared__ int s_wc[NWD];
  __shared__ uint2 s_c[kFinStage];
  const int c_lo = chunk * kMbThreads * KPT;
  const float* srow = scores + (long long)row * L;
  float f[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) f[j] = srow[min(c_lo + (int)threadIdx.x + kMbThreads * j, L - 1)];
  // the row's state is requested with the per-wave counts
  RowState st = {0u, 0};
  if (mode == kModeNormal) st = w.state[row];
  const long long e0 = (long long)row * nchunk;
  int n = 0, def_all = 0, def_before = 0;
  for (int e = lane; e < nchunk; e += 64) {
    const int d = w.defcnt[e0 + e];
    def_all += d;
    def_before += (e < chunk) ? d : 0;
    n += w.ncand[e0 + e];
  }
  // with at most 64 chunks lane e holds chunk e's candidate count, and nc_incl its
  // inclusive prefix over the chunks
  const int nc_lane = n;
  const int nc_incl = wave_inclusive_sum(nc_lane);
  n = __shfl(nc_incl, 63);
  def_all = wave_sum_i(def_all);
  def_before = wave_sum_i(def_before);
  const uint32_t epoch = w.epoch[row];   // not advanced before this kernel ends
  if (chunk == 0) {
    // clear the first-digit histogram and the coarse second-digit one the next call fills
    uint32_t* gh = ghist + (long long)row * 2048;
    for (int j = threadIdx.x; j < 2048; j += kMbThreads) gh[j] = 0u;
    if (threadIdx.x < 64) w.hist2[((long long)((epoch + 1u) & 1u) * rows + row) * 64 + threadIdx.x] = 0u;
  }
  uint32_t tau = (mode == kModeAll) ? 0u : 0xffffffffu;
  int tie_cut = -1;
  int sel_all = 0, sel_before = 0;   // selected candidates that are not sink / window
  if (mode == kModeNormal && n > 0) {   // uniform over the workgroup: n is the row's total
    constexpr int CH = kMbThreads * KPT;
    const uint2* rb = w.cand + (long long)row * nchunk * CH;
    __shared__ int s_cp[kMbMaxChunks];
    const auto lds = [&](int j) { return s_c[j]; };
#define BUTLER_RESOLVE(QQ, LOAD, NN, PRE, BIT, NEED, SA, SB) \
  wave_resolve<QQ>(LOAD, NN, PRE, BIT, NEED, c_lo, tau, tie_cut, SA, SB)
    bool done = false;
    if (n <= kMbFew && nchunk <= 64) {
      // few candidates in few chunks: every wave reads them from the regions itself; the
      // chunk of candidate j is the number of chunks whose inclusive count is <= j
      const auto direct = [&](int j) {
        int e = 0;
#pragma unroll
        for (int sft = 32; sft > 0; sft >>= 1) e += (__shfl(nc_incl, e + sft - 1) <= j) ? sft : 0;
        return rb[(long long)e * CH + min(j - __shfl(nc_incl - nc_lane, e), CH - 1)];
      };
      const uint32_t pre = st.b1 << 21;
      if (n <= 64) BUTLER_RESOLVE(1, direct, n, pre, 20, st.need, sel_all, sel_before);
      else if (n <= 128) BUTLER_RESOLVE(2, direct, n, pre, 20, st.need, sel_all, sel_before);
      else BUTLER_RESOLVE(4, direct, n, pre, 20, st.need, sel_all, sel_before);
      done = true;
    } else if (n > kMbFew && st.nb1 > kMbFew) {
      // many candidates, sorted by coarse bin in every chunk: the coarse bin cb of tau from
      // the row's coarse histogram; the candidates above cb are counted from the chunk
      // tables, and only the ones inside cb are gathered and resolved
      uint32_t cb;
      int above, m;
      wave_find_top64(w.hist2 + ((long long)(st.epoch & 1u) * rows + row) * 64, st.need, cb,
                      above, m);
      if (m <= kFinStage) {
        int* s_st = reinterpret_cast<int*>(h);   // where cb starts in each chunk's region
        int nf_all = 0, nf_before = 0;
        for (int e = threadIdx.x; e < nchunk; e += kMbThreads) {
          const uint32_t* te = w.ctab + (e0 + e) * 64;
          const uint32_t v = te[cb];
          const int end = cb ? (int)(te[cb - 1] & 0xffffu) : w.ncand[e0 + e];
          s_st[e] = (int)(v & 0xffffu);
          s_cp[e] = end - (int)(v & 0xffffu);
          nf_all += (int)(v >> 16);
          nf_before += (e < chunk) ? (int)(v >> 16) : 0;
        }
        const int3 nf = block_sum3(nf_all, nf_before, 0, tmp3);
        block_scan_array<kMbThreads>(s_cp, nchunk, tmp);
        const CandRow part{rb, s_cp, s_st, nchunk, CH};
        for (int j0 = 0; j0 < m; j0 += 2 * kMbThreads) {
          uint2 g[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) g[u] = part(min(j0 + (int)threadIdx.x + kMbThreads * u, m - 1));
#pragma unroll
          for (int u = 0; u < 2; ++u)
            if (j0 + (int)threadIdx.x + kMbThreads * u < m) s_c[j0 + threadIdx.x + kMbThreads * u] = g[u];
        }
        __syncthreads();
        int s2a = 0, s2b = 0;
        const uint32_t pre = (st.b1 << 21) | (cb << 15);
        const int need2 = st.need - above;
        if (m <= 64) BUTLER_RESOLVE(1, lds, m, pre, 14, need2, s2a, s2b);
        else if (m <= 256) BUTLER_RESOLVE(4, lds, m, pre, 14, need2, s2a, s2b);
        else if (m <= 1024) BUTLER_RESOLVE(16, lds, m, pre, 14, need2, s2a, s2b);
        else BUTLER_RESOLVE(32, lds, m, pre, 14, need2, s2a, s2b);
        sel_all = nf.x + s2a;
        sel_before = nf.y + s2b;
        done = true;
      }
    }
    if (!done) {
      // the rest (few candidates over many chunks, or a flood of keys in one coarse bin):
      // the chunks' counts prefix-summed in LDS index every candidate of the row
      for (int e = threadIdx.x; e < nchunk; e += kMbThreads) s_cp[e] = w.ncand[e0 + e];
      __syncthreads();
      block_scan_array<kMbThreads>(s_cp, nchunk, tmp);
      const CandRow crow{rb, s_cp, nullptr, nchunk, CH};
      if (n <= kMbFew) {
        if ((int)threadIdx.x < n) s_c[threadIdx.x] = crow((int)threadIdx.x);
        __syncthreads();
        const uint32_t pre = st.b1 << 21;
        if (n <= 64) BUTLER_RESOLVE(1, lds, n, pre, 20, st.need, sel_all, sel_before);
        else if (n <= 128) BUTLER_RESOLVE(2, lds, n, pre, 20, st.need, sel_all, sel_before);
        else BUTLER_RESOLVE(4, lds, n, pre, 20, st.need, sel_all, sel_before);
      } else {
        block_resolve(crow, n, st.b1, st.need, c_lo, h, tmp, tmp3, sh, tau, tie_cut, sel_all,
                      sel_before);
      }
    }
#undef BUTLER_RESOLVE
  }
  if (chunk == 0 && threadIdx.x == 0) w.epoch[row] = epoch + 1u;
  if (chunk == 0 && threadIdx.x == 0) count[row] = def_all + sel_all;
  const int w_lo = max(0, L - n_window);
  unsigned long long sm[KPT];
  int my = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int t = c_lo + (int)threadIdx.x + kMbThreads * j;
    const uint32_t key = rank_key(f[j], t, n_sink, w_lo, fo);
    bool s = t < n_sink || t >= w_lo || mode == kModeAll;
    if (mode == kModeNormal) s = s || key > tau || (key == tau && t <= tie_cut);
    sm[j] = __ballot(s && t < L);
    if (lane == j) my = __popcll(sm[j]);
  }
  // word u = j * waves + wave covers tokens c_lo + 256 j + 64 wave .. +63
  if (lane < KPT) s_wc[lane * kMbWaves + wid] = my;
  __syncthreads();
  const int v0 = (2 * lane < NWD) ? s_wc[2 * lane] : 0;
  const int v1 = (2 * lane + 1 < NWD) ? s_wc[2 * lane + 1] : 0;
  const int ex = wave_inclusive_sum(v0 + v1) - (v0 + v1);
  const int out0 = def_before + sel_before;
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int nwords = (L + 31) / 32;
  // the chunk's selected tokens, ascending, for the fused attention
  __shared__ int s_list[(R > 0) ? kMbThreads * KPT + kMaPad : 1];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int u = j * kMbWaves + wid;
    const int pe = __shfl(ex, u >> 1), pv = __shfl(v0, u >> 1);
    const int pref = pe + ((u & 1) ? pv : 0);
    const int t = c_lo + (int)threadIdx.x + kMbThreads * j;
    if ((sm[j] >> lane) & 1ull) {
      const int lpos = pref + __popcll(sm[j] & lt);
      if (idx) {
        const int pos = out0 + lpos;
        if (pos < cap) idx[(long long)row * cap + pos] = t;
      }
      if constexpr (R > 0) s_list[lpos] = t;
    }
    if (bitmask && lane < 2) {
      const int wd = (c_lo + kMbThreads * j + 64 * wid) / 32 + lane;
      if (wd < nwords) bitmask[(long long)row * nwords + wd] = (uint32_t)(sm[j] >> (32 * lane));
    }
  }
  if constexpr (R > 0) {
    // attention over the chunk's selected tokens: a ring of two 16-token tiles per wave;
    // list positions past the end repeat the last selected token and are masked out
    const int nsel = __shfl(ex + v0 + v1, 63);   // the chunk's count (inclusive scan total)
    __syncthreads();
    const int last = nsel > 0 ? s_list[nsel - 1] : 0;
    for (int j = nsel + (int)threadIdx.x; j < kMbThreads * KPT + kMaPad; j += kMbThreads)
      s_list[j] = last;
    __syncthreads();
    const int quad = lane >> 4, pe = lane & 15;
    const bf16_t* kb = at.k + (long long)(row / at.kvdiv) * at.L_cap * 128;
    const bf16_t* vb = at.v + (long long)(row / at.kvdiv) * at.L_cap * 128;
    PvStream ms;   // online-softmax state of the wave's heads
    ms.init();
    const int nr = (nsel + kMaRound - 1) / kMaRound;
    const int w0 = wid * 16;
    const int lim0 = nsel - w0 - 4 * quad;
    // round rho lives in t[rho % kMaRing]; kMaRing - 1 tiles are in flight during each
    // compute, and the main loop has no branch, so every wait is for exactly one tile.
    // The last round loaded is nr + kMaRing - 2: inside the padded list.
    MfTile t[kMaRing];
#pragma unroll
    for (int b = 0; b < kMaRing - 1; ++b) mf_load(t[b], s_list, b * kMaRound + w0, kb, vb, quad, pe);
    const int nmain = nr - nr % kMaRing;
    for (int r = 0; r < nmain; r += kMaRing) {
#pragma unroll
      for (int b = 0; b < kMaRing; ++b) {
        mf_load(t[(b + kMaRing - 1) % kMaRing], s_list, (r + b + kMaRing - 1) * kMaRound + w0,
                kb, vb, quad, pe);
        ms.compute(t[b], qf, lim0 - (r + b) * kMaRound, at.scale_log2);
      }
    }
#pragma unroll
    for (int b = 0; b < kMaRing - 1; ++b)
      if (nmain + b < nr) ms.compute(t[b], qf, lim0 - (nmain + b) * kMaRound, at.scale_log2);
    __shared__ float s_m[kMbWaves * (R > 0 ? R : 1)], s_l[kMbWaves * (R > 0 ? R : 1)];
    __shared__ float red_m[R > 0 ? R : 1], red_l[R > 0 ? R : 1];
    __shared__ __align__(16) float s_acc[kMbWaves * (R > 0 ? R : 1) * 128];
    __shared__ float red_acc[(R > 0 ? R : 1) * 128];
    ms.template reduce<R, kMbThreads>(s_m, s_l, s_acc, red_m, red_l, red_acc);
    constexpr int PS = 128 + 4;
    float* my = at.part + ((long long)row * nchunk + chunk) * R * PS;
    for (int j = threadIdx.x; j < R * 128; j += kMbThreads) my[(j / 128) * PS + 4 + j % 128] = red_acc[j];
    if (threadIdx.x < R) {
      my[threadIdx.x * PS] = red_m[threadIdx.x];
      my[threadIdx.x * PS + 1] = red_l[threadIdx.x];
    }
  }
}



#ifndef BUTLER_SEL_CHUNKED_ABOVE
#define BUTLER_SEL_CHUNKED_ABOVE 4096
#endif
bool use_chunked(int Lq, int L, int causal) {
  return !causal && Lq == 1 && L > BUTLER_SEL_CHUNKED_ABOVE;
}

// Fused finishing pass + attention: chunks small enough that a short row still spreads
// over the chip, few enough that the merge takes every chunk's partial at once.
#ifndef BUTLER_SA_KPT_SHORT
#define BUTLER_SA_KPT_SHORT 4    // rows up to 64K tokens
#endif
#ifndef BUTLER_SA_KPT_MID
#define BUTLER_SA_KPT_MID 16     // rows up to 512K tokens
#endif
int kpt_attend(int L) {
  return L <= 65536 ? BUTLER_SA_KPT_SHORT : L <= 524288 ? BUTLER_SA_KPT_MID : L <= 2097152 ? 16 : 32;
}
constexpr int kMaMaxChunks = 512;

}  // namespace

bool select_attend_fusable(int dtype, int D, int Hq, int Hkv, int L) {
  const int R = Hq / Hkv;
  return dtype == 1 && D == 128 && (R == 1 || R == 2 || R == 4 || R == 8) &&
         use_chunked(1, L, 0) && nchunk_k(L, kpt_attend(L)) <= kMaMaxChunks;
}

size_t select_attend_workspace(int rows, int Hq, int Hkv, int L) {
  const int kpt = kpt_attend(L);
  return mb_bytes_k(rows, L, kpt) +
         al256((size_t)rows * nchunk_k(L, kpt) * (Hq / Hkv) * (128 + 4) * sizeof(float));
}

hipError_t launch_select_attend(hipStream_t s, const float* scores, int num, int den,
                                int n_sink, int n_window, int fo, int32_t* idx, int32_t* count, int B,
                                int Hq, int Hkv, int L, int cap, uint32_t* hist, const void* q,
                                const void* k, const void* v, float* out, int L_cap,
                                float scale, void* ws, int kvdiv) {
  const long long rows = (long long)B * Hkv;
  const int kpt = kpt_attend(L);
  const int nchunk = (int)nchunk_k(L, kpt);
  if (nchunk > kMaMaxChunks) return hipErrorInvalidValue;
  const MbWs w = carve_k(ws, rows, L, kpt);
  float* part = (float*)((char*)ws + mb_bytes_k(rows, L, kpt));
  const MbAttn at{(const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, part, Hq, Hkv, L_cap,
                  scale * 1.4426950408889634f, kvdiv};
  const dim3 grid((unsigned)(rows * nchunk));
  uint32_t* gh = hist ? hist : w.hist1;
  const int R = Hq / Hkv;
  auto run = [&](auto kpt_c, auto r_c) {
    constexpr int KPT = decltype(kpt_c)::value;
    constexpr int RR = decltype(r_c)::value;
    if (!hist)
      hipLaunchKernelGGL(mb_hist1_kernel<KPT>, grid, dim3(kMbThreads), 0, s, scores, num, den,
                         n_sink, n_window, fo, L, (int)rows, gh, (const int32_t*)nullptr);
    hipLaunchKernelGGL(mb_cand_kernel<KPT>, grid, dim3(kMbThreads), 0, s, scores, num, den,
                       n_sink, n_window, L, (int)rows, (const uint32_t*)gh, w,
                       (const int32_t*)nullptr, fo);
    hipLaunchKernelGGL((mb_finish_kernel<KPT, RR>), grid, dim3(kMbThreads), 0, s, scores, num,
                       den, n_sink, n_window, L, (int)rows, cap, idx, (uint32_t*)nullptr, count,
                       gh, w, (const int32_t*)nullptr, at, fo);
  };
  auto by_r = [&](auto kpt_c) {
    switch (R) {
      case 1: run(kpt_c, std::integral_constant<int, 1>()); break;
      case 2: run(kpt_c, std::integral_constant<int, 2>()); break;
      case 4: run(kpt_c, std::integral_constant<int, 4>()); break;
      default: run(kpt_c, std::integral_constant<int, 8>()); break;
    }
  };
  switch (kpt) {
    case 4: by_r(std::integral_constant<int, 4>()); break;
    case 8: by_r(std::integral_constant<int, 8>()); break;
    case 16: by_r(std::integral_constant<int, 16>()); break;
    default: by_r(std::integral_constant<int, 32>()); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_merge(s, part, out, rows, Hq, Hkv, 1, 128, nchunk);
}

size_t select_workspace(int rows, int L, int Lq, int causal) {
  return use_chunked(Lq, L, causal) ? mb_bytes(rows, L) : 0;
}

size_t select_state_bytes(int rows) { return mb_state_bytes(rows); }

hipError_t launch_select(hipStream_t s, const float* scores, int num, int den, int n_sink,
                         int n_window, int fo, int32_t* idx, uint32_t* bitmask, int32_t* count,
                         int B, int Hkv, int Lq, int L, int cap, int q_pos0, int causal,
                         uint32_t* hist, const int32_t* keep, void* ws) {
  const long long rows = (long long)B * Hkv * Lq;
  if (use_chunked(Lq, L, causal)) {
    const MbWs w = carve(ws, rows, L);
    const int nchunk = (int)nchunk_for(L);
    if (nchunk > kMbMaxChunks) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(rows * nchunk));
    uint32_t* gh = hist ? hist : w.hist1;
    auto run = [&](auto kpt_c) {
      constexpr int KPT = decltype(kpt_c)::value;
      if (!hist)
        hipLaunchKernelGGL(mb_hist1_kernel<KPT>, grid, dim3(kMbThreads), 0, s, scores, num, den,
                           n_sink, n_window, fo, L, (int)rows, gh, keep);
      hipLaunchKernelGGL(mb_cand_kernel<KPT>, grid, dim3(kMbThreads), 0, s, scores, num, den,
                         n_sink, n_window, L, (int)rows, (const uint32_t*)gh, w, keep, fo);
      hipLaunchKernelGGL((mb_finish_kernel<KPT, 0>), grid, dim3(kMbThreads), 0, s, scores, num,
                         den, n_sink, n_window, L, (int)rows, cap, idx, bitmask, count, gh, w, keep,
                         MbAttn{}, fo);
    };
    switch (kpt_for(L)) {
      case 8: run(std::integral_constant<int, 8>()); break;
      case 16: run(std::integral_constant<int, 16>()); break;
      default: run(std::integral_constant<int, 32>()); break;
    }
    return hipGetLastError();
  }
  // one workgroup per row, sized to the row: 64 to 1024 threads, and keys per thread in
  // steps that keep the slots past the row's end (idle work) to a quarter or less
#define BUTLER_SR(NT, KPT)                                                                 \
  hipLaunchKernelGGL((select_row_kernel<NT, KPT>), dim3((unsigned)rows), dim3(NT), 0, s,   \
                     scores, num, den, n_sink, n_window, idx, bitmask, count, Lq, L, cap,   \
                     q_pos0, causal, hist, keep, fo)
  if (L <= 256) BUTLER_SR(64, 4);
  else if (L <= 512) BUTLER_SR(64, 8);
  else if (L <= 768) BUTLER_SR(64, 12);
  else if (L <= 1024) BUTLER_SR(64, 16);
  else if (L <= 1536) BUTLER_SR(128, 12);
  else if (L <= 2048) BUTLER_SR(128, 16);
  else if (L <= 3072) BUTLER_SR(256, 12);
  else if (L <= 4096) BUTLER_SR(256, 16);
  // 512 threads: x 16 measured faster than 256 x 32 and 1024 x 8
  else if (L <= 5120) BUTLER_SR(512, 10);
  else if (L <= 6144) BUTLER_SR(512, 12);
  else if (L <= 7168) BUTLER_SR(512, 14);
  else if (L <= 8192) BUTLER_SR(512, 16);
  else if (L <= 16384) BUTLER_SR(512, 32);
  else if (L <= 32768) BUTLER_SR(1024, 32);
  else BUTLER_SR(1024, 64);
#undef BUTLER_SR
  return hipGetLastError();
}

}  // namespace butler
