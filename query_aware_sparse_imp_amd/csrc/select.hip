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
// Decode rows longer than 4096 tokens: kernels over 2048-token chunks
//   0  (only without the scorer's histogram) histogram of key bits 31..21
//   1  every chunk derives the first-digit bin b1, counts its tokens that are surely
//      selected (digit above b1, or a sink / window token) and appends the keys whose
//      digit is b1 to the row's candidate ring -- for scores of any spread only a sliver
//      of the row
//   2  every chunk resolves tau and the tie cut from the row's candidates (the same work
//      in every workgroup of the row: cheaper than a kernel boundary while the candidates
//      are few), derives its output offset from the per-chunk counts and emits its
//      bitmask words and indices; the chunk-0 workgroup writes the row count and clears
//      the histogram.
//
// Other rows (short decode rows, every causal prefill row): one workgroup per row holds
//   the row's keys in VGPRs (up to 64 per thread, strided so that a wave's ballot covers
//   64 consecutive tokens), builds the digit histograms in LDS (the first from the
//   scorer's histogram when given), and emits through 64-token ballot words with two
//   block-wide scans over the words (tie ranks, then output positions).
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

enum { kModeNormal = 0, kModeNone = 1, kModeAll = 2 };

__device__ __forceinline__ int row_mode(int L_r, int num, int den, int& k) {
  const long long x = (long long)L_r * num / den;
  k = (int)min<long long>(x, (long long)L_r);
  return k <= 0 ? kModeNone : (k >= L_r ? kModeAll : kModeNormal);
}

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
    int Lq, int L, int cap, int q_pos0, int causal, uint32_t* __restrict__ ghist) {
  constexpr int NW = NT / 64;
  constexpr int MAXW = NT * KPT / 64;
  const long long row = blockIdx.x;
  const int i = (int)(row % Lq);
  const int L_r = causal ? min(q_pos0 + i + 1, L) : L;
  int k;
  const int mode = row_mode(L_r, num, den, k);
  const float* s = scores + row * (long long)L;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;

  __shared__ uint32_t hist[2048];
  __shared__ int tmp[NW];
  __shared__ int sh_bin, sh_need;
  __shared__ int wtie[MAXW], wcnt[MAXW];
  __shared__ uint64_t wsel[MAXW];

  // all loads at once, from clamped addresses (no control flow around them)
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = score_key(s[min((int)threadIdx.x + NT * j, L_r - 1)]);
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
  const int w_lo = max(0, L_r - n_window);
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
// decode rows longer than 4096 tokens: three (or four) kernels over 2048-token chunks
// ---------------------------------------------------------------------------

constexpr int kMbThreads = 256;
constexpr int kMbChunk = 2048;           // tokens per workgroup, 8 per thread
constexpr int kMbMaxChunks = 4096;       // rows of up to 8M tokens
constexpr int kFinStage = 2048;          // candidates staged in LDS (more: read from memory)

struct RowState {
  uint32_t b1;  // first-digit bin of the x-th largest key
  int need;     // rank of the x-th largest key inside that bin (1-based)
};

struct MbWs {
  uint32_t* hist1;               // [rows][2048]   first-digit counts, zero between calls
  unsigned long long* ccount;    // [rows]         running candidate counter (never reset)
  RowState* state;               // [rows]
  int* defcnt;                   // [rows][nchunk] tokens of the chunk that are surely selected
  int* ncand;                    // [rows][nchunk] candidates the chunk appended
  uint2* cand;                   // [rows][L]      ring of (key, index | sink/window flag << 31)
};

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

size_t mb_bytes(long long rows, int L) {
  const long long nchunk = (L + kMbChunk - 1) / kMbChunk;
  return al256(rows * 2048 * 4) + al256(rows * 8) + al256(rows * sizeof(RowState)) +
         2 * al256(rows * nchunk * 4) + al256((size_t)rows * L * sizeof(uint2));
}

MbWs carve(void* ws, long long rows, int L) {
  const long long nchunk = (L + kMbChunk - 1) / kMbChunk;
  char* p = (char*)ws;
  MbWs w;
  w.hist1 = (uint32_t*)p;                 p += al256(rows * 2048 * sizeof(uint32_t));
  w.ccount = (unsigned long long*)p;      p += al256(rows * 8);
  w.state = (RowState*)p;                 p += al256(rows * sizeof(RowState));
  w.defcnt = (int*)p;                     p += al256(rows * nchunk * sizeof(int));
  w.ncand = (int*)p;                      p += al256(rows * nchunk * sizeof(int));
  w.cand = (uint2*)p;
  return w;
}

// The 8 keys of tokens t0 .. t0+7; returns how many exist (t < L).
__device__ __forceinline__ int load_keys8(const float* s, int t0, int L, uint32_t (&key)[8]) {
  const int nv = max(0, min(8, L - t0));
  if (nv == 8 && ((((uintptr_t)(s + t0)) & 15u) == 0)) {
    const float4 a = *reinterpret_cast<const float4*>(s + t0);
    const float4 b = *reinterpret_cast<const float4*>(s + t0 + 4);
    key[0] = score_key(a.x); key[1] = score_key(a.y); key[2] = score_key(a.z);
    key[3] = score_key(a.w); key[4] = score_key(b.x); key[5] = score_key(b.y);
    key[6] = score_key(b.z); key[7] = score_key(b.w);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) key[j] = score_key(s[min(t0 + j, L - 1)]);
  }
  return nv;
}

// first-digit histogram, when the scorer did not produce it
__global__ __launch_bounds__(kMbThreads) void mb_hist1_kernel(const float* __restrict__ scores,
                                                              int num, int den, int L, int rows,
                                                              uint32_t* __restrict__ ghist) {
  const int row = blockIdx.x % rows, chunk = blockIdx.x / rows;
  int k;
  if (row_mode(L, num, den, k) != kModeNormal) return;
  __shared__ uint32_t h[2048];
  for (int j = threadIdx.x; j < 2048; j += kMbThreads) h[j] = 0u;
  __syncthreads();
  uint32_t key[8];
  const int nv = load_keys8(scores + (long long)row * L, chunk * kMbChunk + threadIdx.x * 8, L, key);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < nv) atomicAdd(&h[key[j] >> 21], 1u);
  __syncthreads();
  uint32_t* gh = ghist + (long long)row * 2048;
  for (int j = threadIdx.x; j < 2048; j += kMbThreads)
    if (h[j]) atomicAdd(&gh[j], h[j]);
}

// Chunk pass: every workgroup derives the first-digit bin b1 from the row's histogram,
// counts its tokens that are surely selected (digit above b1, or sink / window) and
// appends the keys whose first digit is b1 to the row's candidate ring.
__global__ __launch_bounds__(kMbThreads) void mb_cand_kernel(const float* __restrict__ scores,
                                                             int num, int den, int n_sink,
                                                             int n_window, int L, int rows,
                                                             const uint32_t* __restrict__ ghist,
                                                             MbWs w) {
  const int row = blockIdx.x % rows, chunk = blockIdx.x / rows;
  const int nchunk = gridDim.x / rows;
  int k;
  const int mode = row_mode(L, num, den, k);
  __shared__ uint32_t h[2048];
  __shared__ int tmp[kMbThreads / 64];
  __shared__ int sh_bin, sh_need, sh_start;
  const int t0 = chunk * kMbChunk + threadIdx.x * 8;
  uint32_t key[8];
  const int nv = load_keys8(scores + (long long)row * L, t0, L, key);
  uint32_t b1 = 0;
  if (mode == kModeNormal) {
    const uint32_t* gh = ghist + (long long)row * 2048;
    for (int j = threadIdx.x; j < 2048; j += kMbThreads) h[j] = gh[j];
    __syncthreads();
    find_bin_from_top<kMbThreads>(h, 2048, k, tmp, &sh_bin, &sh_need);
    b1 = (uint32_t)sh_bin;
    if (chunk == 0 && threadIdx.x == 0) w.state[row] = RowState{b1, sh_need};
  }
  const int w_lo = max(0, L - n_window);
  int ndef = 0, ncand = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= nv) continue;
    const int t = t0 + j;
    const bool forced = t < n_sink || t >= w_lo;
    if (mode == kModeNormal) {
      const uint32_t top = key[j] >> 21;
      ndef += (forced || top > b1) ? 1 : 0;
      ncand += (top == b1) ? 1 : 0;
    } else {
      ndef += (forced || mode == kModeAll) ? 1 : 0;
    }
  }
  int tot_def, tot_cand;
  block_exclusive_sum<kMbThreads>(ndef, tot_def, tmp);
  const int cpos = block_exclusive_sum<kMbThreads>(ncand, tot_cand, tmp);
  if (threadIdx.x == 0) {
    w.defcnt[(long long)row * nchunk + chunk] = tot_def;
    w.ncand[(long long)row * nchunk + chunk] = tot_cand;
    sh_start = tot_cand ? (int)(atomicAdd(&w.ccount[row], (unsigned long long)tot_cand) %
                                (unsigned long long)L)
                        : 0;
  }
  __syncthreads();
  if (ncand) {
    uint2* crow = w.cand + (long long)row * L;
    int pos = sh_start + cpos;
    if (pos >= L) pos -= L;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= nv || (key[j] >> 21) != b1) continue;
      const int t = t0 + j;
      const uint32_t flag = (t < n_sink || t >= w_lo) ? 0x80000000u : 0u;
      crow[pos] = make_uint2(key[j], (uint32_t)t | flag);
      if (++pos == L) pos = 0;
    }
  }
}

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

// Whether candidate c comes before (key kj, index ij) in (key desc, index asc) order.
__device__ __forceinline__ int precedes(uint2 c, uint32_t kj, uint32_t ij) {
  const uint32_t ii = c.y & 0x7fffffffu;
  return (c.x > kj || (c.x == kj && ii < ij)) ? 1 : 0;
}

// Finishing pass, one workgroup per chunk: every workgroup of a row resolves the same tau
// and tie cut from the row's candidates (a rank count when they are few, else the radix
// over bits 20..0 and the index radix of the ties), sums the sure and the selected
// candidate counts of the chunks before its own into its output offset, and emits its
// tokens.  The chunk-0 workgroup writes the row count and clears the row's histogram
// (nothing in this kernel reads it).
__global__ __launch_bounds__(kMbThreads) void mb_finish_kernel(
    const float* __restrict__ scores, int num, int den, int n_sink, int n_window, int L,
    int rows, int cap, int32_t* __restrict__ idx, uint32_t* __restrict__ bitmask,
    int32_t* __restrict__ count, uint32_t* __restrict__ ghist, MbWs w) {
  const int row = blockIdx.x % rows, chunk = blockIdx.x / rows;
  const int nchunk = gridDim.x / rows;
  int k;
  const int mode = row_mode(L, num, den, k);
  __shared__ uint32_t h[2048];
  __shared__ uint2 s_c[kFinStage];
  __shared__ int tmp[kMbThreads / 64];
  __shared__ int3 tmp3[kMbThreads / 64];
  __shared__ int sh_bin, sh_need, sh_tie;
  __shared__ uint32_t sh_tau;
  __shared__ uint8_t bytes[kMbThreads];
  const int w_lo = max(0, L - n_window);
  const int c_lo = chunk * kMbChunk;
  const int t0 = c_lo + threadIdx.x * 8;
  uint32_t key[8];
  const int nv = load_keys8(scores + (long long)row * L, t0, L, key);
  // the row's state and candidate counter are requested with the per-chunk counts
  RowState st = {0u, 0};
  unsigned long long end = 0ull;
  if (mode == kModeNormal) {
    st = w.state[row];
    end = w.ccount[row];
  }
  int n_loc = 0, def_all = 0, def_before = 0;
  for (int c = threadIdx.x; c < nchunk; c += kMbThreads) {
    const int d = w.defcnt[(long long)row * nchunk + c];
    def_all += d;
    def_before += (c < chunk) ? d : 0;
    n_loc += w.ncand[(long long)row * nchunk + c];
  }
  const int3 sums = block_sum3(n_loc, def_all, def_before, tmp3);
  const int n = sums.x;
  def_all = sums.y;
  def_before = sums.z;
  int tot;
  if (chunk == 0) {
    uint32_t* gh = ghist + (long long)row * 2048;
    for (int j = threadIdx.x; j < 2048; j += kMbThreads) gh[j] = 0u;
  }
  uint32_t tau = (mode == kModeAll) ? 0u : 0xffffffffu;
  int tie_cut = -1;
  int sel_all = 0, sel_before = 0;   // selected candidates that are not sink / window
  if (mode == kModeNormal && n > 0) {
    const int base = (int)((end - (unsigned long long)n) % (unsigned long long)L);
    const uint2* crow = w.cand + (long long)row * L;
    auto at = [&](int j) {
      const int p = base + j;
      return crow[p >= L ? p - L : p];
    };
    const bool staged = n <= kFinStage;
    if (staged) {
      for (int j = threadIdx.x; j < n; j += kMbThreads) s_c[j] = at(j);
    }
    __syncthreads();
    auto ckey = [&](int j) { return staged ? s_c[j].x : at(j).x; };
    auto cid = [&](int j) { return staged ? s_c[j].y : at(j).y; };
    if (n <= kMbThreads) {
      // rank of each candidate in (key desc, index asc) order; the one of rank need-1 is
      // the last token the budget takes
      if ((int)threadIdx.x < n) {
        const uint2 me = s_c[threadIdx.x];
        const uint32_t kj = me.x, ij = me.y & 0x7fffffffu;
        int rank = 0, i = 0;
        for (; i + 4 <= n; i += 4) {
          const uint2 c0 = s_c[i], c1 = s_c[i + 1], c2 = s_c[i + 2], c3 = s_c[i + 3];
          rank += precedes(c0, kj, ij) + precedes(c1, kj, ij) + precedes(c2, kj, ij) +
                  precedes(c3, kj, ij);
        }
        for (; i < n; ++i) rank += precedes(s_c[i], kj, ij);
        if (rank == st.need - 1) {
          sh_tau = kj;
          sh_tie = (int)ij;
        }
      }
      __syncthreads();
      tau = sh_tau;
      tie_cut = sh_tie;
    } else {
      // bits 20..10, then 9..0, over the candidates (all have first digit b1)
      uint32_t prefix = st.b1 << 21, pmask = 0xffe00000u;
      int need = st.need;
      const int shifts[2] = {10, 0};
      const int bins[2] = {2048, 1024};
      for (int p = 0; p < 2; ++p) {
        for (int j = threadIdx.x; j < 2048; j += kMbThreads) h[j] = 0u;
        __syncthreads();
        for (int j = threadIdx.x; j < n; j += kMbThreads) {
          const uint32_t kk = ckey(j);
          if ((kk & pmask) == prefix) atomicAdd(&h[(kk >> shifts[p]) & (uint32_t)(bins[p] - 1)], 1u);
        }
        __syncthreads();
        find_bin_from_top<kMbThreads>(h, bins[p], need, tmp, &sh_bin, &sh_need);
        prefix |= (uint32_t)sh_bin << shifts[p];
        pmask |= (uint32_t)(bins[p] - 1) << shifts[p];
        need = sh_need;
      }
      tau = prefix;
      int mine = 0;
      for (int j = threadIdx.x; j < n; j += kMbThreads) mine += (ckey(j) == tau) ? 1 : 0;
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
            const uint32_t t = cid(j) & 0x7fffffffu;
            if (ckey(j) == tau && (t & pm) == pre) atomicAdd(&h[(t >> ish[p]) & (iw[p] - 1u)], 1u);
          }
          __syncthreads();
          find_bin_from_bottom<kMbThreads>(h, 2048, nd, tmp, &sh_bin, &sh_need);
          pre |= (uint32_t)sh_bin << ish[p];
          pm |= (iw[p] - 1u) << ish[p];
          nd = sh_need;
        }
        tie_cut = (int)pre;
      }
    }
    for (int j = threadIdx.x; j < n; j += kMbThreads) {
      const uint32_t id = cid(j);
      if (id & 0x80000000u) continue;  // sink / window tokens are counted as sure
      const uint32_t kk = ckey(j);
      const int t = (int)id;
      if (kk > tau || (kk == tau && t <= tie_cut)) {
        ++sel_all;
        sel_before += (t < c_lo) ? 1 : 0;
      }
    }
    const int3 ss = block_sum3(sel_all, sel_before, 0, tmp3);
    sel_all = ss.x;
    sel_before = ss.y;
  }
  if (chunk == 0 && threadIdx.x == 0) count[row] = def_all + sel_all;
  uint32_t sel = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= nv) continue;
    const int t = t0 + j;
    bool s = t < n_sink || t >= w_lo;
    if (mode == kModeAll) s = true;
    else if (mode == kModeNormal) s = s || key[j] > tau || (key[j] == tau && t <= tie_cut);
    sel |= (uint32_t)s << j;
  }
  const int ex = block_exclusive_sum<kMbThreads>(__popc(sel), tot, tmp);
  if (idx) {
    int pos = def_before + sel_before + ex;
    int32_t* irow = idx + (long long)row * cap;
    for (uint32_t e = sel; e; e &= e - 1) {
      if (pos < cap) irow[pos] = t0 + (__ffs(e) - 1);
      ++pos;
    }
  }
  if (bitmask) {
    bytes[threadIdx.x] = (uint8_t)sel;
    __syncthreads();
    const int nwords = (L + 31) / 32;
    const int wd = chunk * (kMbChunk / 32) + threadIdx.x;
    if (threadIdx.x < kMbChunk / 32 && wd < nwords) {
      const int b0 = threadIdx.x * 4;
      bitmask[(long long)row * nwords + wd] = (uint32_t)bytes[b0] | ((uint32_t)bytes[b0 + 1] << 8) |
                                              ((uint32_t)bytes[b0 + 2] << 16) |
                                              ((uint32_t)bytes[b0 + 3] << 24);
    }
  }
}

bool use_chunked(int Lq, int L, int causal) {
  return !causal && Lq == 1 && L > 4096;
}

}  // namespace

size_t select_workspace(int rows, int L, int Lq, int causal) {
  return use_chunked(Lq, L, causal) ? mb_bytes(rows, L) : 0;
}

hipError_t launch_select(hipStream_t s, const float* scores, int num, int den, int n_sink,
                         int n_window, int32_t* idx, uint32_t* bitmask, int32_t* count,
                         int B, int Hkv, int Lq, int L, int cap, int q_pos0, int causal,
                         uint32_t* hist, void* ws) {
  const long long rows = (long long)B * Hkv * Lq;
  if (use_chunked(Lq, L, causal)) {
    const MbWs w = carve(ws, rows, L);
    const int nchunk = (L + kMbChunk - 1) / kMbChunk;
    const dim3 grid((unsigned)(rows * nchunk));
    uint32_t* gh = hist;
    if (!gh) {
      gh = w.hist1;
      hipLaunchKernelGGL(mb_hist1_kernel, grid, dim3(kMbThreads), 0, s, scores, num, den, L,
                         (int)rows, gh);
    }
    hipLaunchKernelGGL(mb_cand_kernel, grid, dim3(kMbThreads), 0, s, scores, num, den, n_sink,
                       n_window, L, (int)rows, (const uint32_t*)gh, w);
    hipLaunchKernelGGL(mb_finish_kernel, grid, dim3(kMbThreads), 0, s, scores, num, den, n_sink,
                       n_window, L, (int)rows, cap, idx, bitmask, count, gh, w);
    return hipGetLastError();
  }
  // one workgroup per row; the widest rows get 1024 threads x 64 keys
  if (L <= 4096) {
    hipLaunchKernelGGL((select_row_kernel<256, 16>), dim3((unsigned)rows), dim3(256), 0, s,
                       scores, num, den, n_sink, n_window, idx, bitmask, count, Lq, L, cap,
                       q_pos0, causal, hist);
  } else if (L <= 16384) {
    hipLaunchKernelGGL((select_row_kernel<512, 32>), dim3((unsigned)rows), dim3(512), 0, s,
                       scores, num, den, n_sink, n_window, idx, bitmask, count, Lq, L, cap,
                       q_pos0, causal, hist);
  } else if (L <= 32768) {
    hipLaunchKernelGGL((select_row_kernel<1024, 32>), dim3((unsigned)rows), dim3(1024), 0, s,
                       scores, num, den, n_sink, n_window, idx, bitmask, count, Lq, L, cap,
                       q_pos0, causal, hist);
  } else {
    hipLaunchKernelGGL((select_row_kernel<1024, 64>), dim3((unsigned)rows), dim3(1024), 0, s,
                       scores, num, den, n_sink, n_window, idx, bitmask, count, Lq, L, cap,
                       q_pos0, causal, hist);
  }
  return hipGetLastError();
}

}  // namespace butler
