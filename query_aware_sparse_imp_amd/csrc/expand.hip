// Neighbour fetching for the prediction interval (TokenButler arXiv abstract: the
// predictor runs once per interval and the selection is widened with token neighbours
// in between).  Per (b, KV head) row, the reused index list S becomes
//   S' = { u : |u - t| <= width for some t in S } U [L - n_window, L),   0 <= u < L,
// the window taken at the current length, so tokens appended since the selection was
// made are attended.  A row's output is split by 32-token words into C chunks of at most
// 1024 words, one workgroup per (row, chunk), so a few long rows still spread over the
// chip.  A workgroup walks the row up to the end of its chunk in segments of 2^18 tokens:
//   1. the members of S that fall in the segment (plus one guard word on each side) are
//      set as single bits in an LDS bitmask.  S is read in coalesced rounds of 4096
//      entries, four consecutive ones per thread, and a thread ORs bits into a register
//      while they fall in one word, so a sorted S costs about one LDS atomic per thread
//      and round;
//   2. each word is dilated by `width` (< 32) from itself and its two neighbours as two
//      64-bit funnels (shifts 0..width, ORed by doubling) and the window and the row end
//      are applied.  Words before the chunk are only counted; the chunk's words are kept
//      in LDS;
//   3. the count before the chunk (a block sum) plus a block scan over the chunk's words
//      give every word its output position; the thread of a word writes its tokens.
// Every workgroup reads all of S: the redundant reads hit L2, and they buy the output
// offset without any hand-off between workgroups.  S need not be sorted or free of
// repeats; entries outside [0, L) are ignored.
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr int kExThreads = 1024;
constexpr int kExSegWords = 8192;                         // 2^18 tokens per segment
constexpr int kExChunkWords = kExThreads;                 // at most one word per thread
constexpr int kExTargetBlocks = 512;
constexpr int kExMaxLen = 8388608;

// OR of x << d for d = 0..w (w < 64), by doubling the covered shift range
__device__ __forceinline__ uint64_t spread_up(uint64_t x, int w) {
  for (int covered = 1; covered <= w;) {
    const int s = min(covered, w + 1 - covered);
    x |= x << s;
    covered += s;
  }
  return x;
}

__device__ __forceinline__ uint64_t spread_down(uint64_t x, int w) {
  for (int covered = 1; covered <= w;) {
    const int s = min(covered, w + 1 - covered);
    x |= x >> s;
    covered += s;
  }
  return x;
}

// grid (rows, C); chunk c covers words [c * cwords, (c + 1) * cwords) of the row
__global__ __launch_bounds__(kExThreads) void expand_neighbors_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, int L, int cap_in, int cap_out, int width, int n_window,
    int cwords) {
  __shared__ uint32_t bm[kExSegWords + 2];   // bm[k] holds tokens seg0 - 32 + 32k ...
  __shared__ uint32_t chw[kExChunkWords];    // the chunk's dilated words
  __shared__ int tmp[kExThreads / 64];
  const long long row = blockIdx.x;
  const int n = max(0, min(count[row], cap_in));
  const int32_t* irow = idx + row * (long long)cap_in;
  int32_t* orow = idx_out + row * (long long)cap_out;
  const int wlo = max(0, L - n_window);
  const int row_words = (L + 31) / 32;
  const int cw0 = (int)blockIdx.y * cwords, cw1 = min(cw0 + cwords, row_words);
  int before = 0;                            // this thread's share of the count before cw0
  for (int seg0 = 0; seg0 < L && (seg0 >> 5) < cw1; seg0 += kExSegWords * 32) {
    const int seg1 = min(L, seg0 + kExSegWords * 32);
    const int sw0 = seg0 >> 5;
    const int nwords = min((seg1 - seg0 + 31) / 32, cw1 - sw0);   // words used here
    for (int j = threadIdx.x; j < nwords + 2; j += kExThreads) bm[j] = 0u;
    __syncthreads();
    // 1. single bits of S over the used words and their guards
    const int lo_tok = seg0 - 32, hi_tok = seg0 + 32 * (nwords + 1);
    for (int e = 4 * (int)threadIdx.x; e < n; e += 4 * kExThreads) {
      int tv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) tv[u] = irow[min(e + u, n - 1)];
      int cw = -1;
      uint32_t cb = 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = tv[u];
        if (e + u >= n || t < 0 || t >= L || t < lo_tok || t >= hi_tok) continue;
        const int wd = (t - lo_tok) >> 5;
        if (wd != cw) {
          if (cw >= 0) atomicOr(&bm[cw], cb);
          cw = wd;
          cb = 0u;
        }
        cb |= 1u << ((t - lo_tok) & 31);
      }
      if (cw >= 0) atomicOr(&bm[cw], cb);
    }
    __syncthreads();
    // 2. dilation, window and row end; count before the chunk, keep the chunk's words
    for (int j = threadIdx.x; j < nwords; j += kExThreads) {
      const uint32_t p = bm[j], cur = bm[j + 1], nx = bm[j + 2];
      const uint64_t up = spread_up(((uint64_t)cur << 32) | p, width);
      const uint64_t dn = spread_down(((uint64_t)nx << 32) | cur, width);
      uint32_t r = (uint32_t)(up >> 32) | (uint32_t)dn;
      const int t0 = seg0 + 32 * j;                       // first token of the word
      if (wlo < t0 + 32) r |= (wlo <= t0) ? 0xffffffffu : (0xffffffffu << (wlo - t0));
      if (seg1 < t0 + 32) r &= (1u << (seg1 - t0)) - 1u;  // seg1 - t0 in [1, 31]
      const int J = sw0 + j;
      if (J < cw0) before += __popc(r);
      else chw[J - cw0] = r;
    }
    __syncthreads();   // the next segment clears bm; chw is complete after the last one
  }
  // 3. output positions and the chunk's tokens
  const int nch = max(0, cw1 - cw0);
  const uint32_t x = ((int)threadIdx.x < nch) ? chw[threadIdx.x] : 0u;
  int total_before;
  block_exclusive_sum<kExThreads>(before, total_before, tmp);
  int total;
  int pos = total_before + block_exclusive_sum<kExThreads>(__popc(x), total, tmp);
  const int tw = 32 * (cw0 + (int)threadIdx.x);
  for (uint32_t e = x; e; e &= e - 1) {
    if (pos < cap_out) orow[pos] = tw + (__ffs(e) - 1);
    ++pos;
  }
  if (threadIdx.x == 0 && blockIdx.y == gridDim.y - 1) count_out[row] = total_before + total;
}

int expand_chunk_words(int rows, int L) {
  const int row_words = (L + 31) / 32;
  const int want_chunks = max(1, kExTargetBlocks / max(rows, 1));
  int cwords = (row_words + want_chunks - 1) / want_chunks;
  cwords = ((cwords + 63) / 64) * 64;                      // whole waves
  return min(max(cwords, 64), kExChunkWords);
}

}  // namespace

hipError_t launch_expand_neighbors(hipStream_t s, const int32_t* idx, const int32_t* count,
                                   int32_t* idx_out, int32_t* count_out, int rows, int L,
                                   int cap_in, int cap_out, int width, int n_window) {
  const int cwords = expand_chunk_words(rows, L);
  const int chunks = ((L + 31) / 32 + cwords - 1) / cwords;
  hipLaunchKernelGGL(expand_neighbors_kernel, dim3((unsigned)rows, (unsigned)chunks),
                     dim3(kExThreads), 0, s, idx, count, idx_out, count_out, L, cap_in,
                     cap_out, width, n_window, cwords);
  return hipGetLastError();
}

int expand_max_len() { return kExMaxLen; }

}  // namespace butler
