// Fixed-budget top-x + sink + window selection (TokenButler model card, Method and
// Memory requirements).
//
// Scores become order-preserving uint32 keys (score_key).  The x-th largest key tau
// is found exactly by a most-significant-digit radix select over digits of 11, 11 and
// 10 bits: each pass histograms, in LDS, the next digit of the keys that share the
// prefix found so far, and a block-wide scan from the top bin finds the bin that holds
// the x-th largest key.  After the third pass tau is known together with the number of
// keys equal to tau that the budget still takes; those are the lowest-index ones.
// The emit pass walks the row in index order, 32 tokens (one bitmask word) per thread:
// a block scan ranks the keys equal to tau, a second one places the selected tokens,
// so the index list comes out ascending and the result does not depend on timing.
//
// One workgroup handles one row (a (b, KV head, query row) triple); rows are
// independent, so a prefill chunk launches thousands of workgroups while a decode step
// launches B * Hkv of them.
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr int kSelThreads = 512;

struct RadixState {
  uint32_t tau;  // key of the x-th largest score
  int need;      // keys equal to tau that belong to the top x (lowest indices first)
};

// Finds, among hist[0..nbins) scanned from the top bin down, the bin holding the
// need-th largest key.  Returns (bin, need - keys in higher bins) via LDS.
template <int NT>
__device__ void find_bin_from_top(const uint32_t* hist, int nbins, int need, int* tmp,
                                  int* out_bin, int* out_need) {
  const int per = nbins / NT;  // bins per thread (nbins is a multiple of NT)
  const int hi = nbins - threadIdx.x * per;  // this thread covers bins [hi-per, hi)
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

template <int NT>
__global__ __launch_bounds__(NT) void select_rows_kernel(
    const float* __restrict__ scores, int num, int den, int n_sink, int n_window,
    int32_t* __restrict__ idx, uint32_t* __restrict__ bitmask, int32_t* __restrict__ count,
    int Lq, int L, int cap, int q_pos0, int causal) {
  const long long row = blockIdx.x + (long long)blockIdx.y * gridDim.x;
  const int i = (int)(row % Lq);
  const int L_r = causal ? min(q_pos0 + i + 1, L) : L;
  const long long x = (long long)L_r * num / den;
  const int k = (int)min<long long>(x, (long long)L_r);
  const float* s = scores + row * (long long)L;

  __shared__ uint32_t hist[2048];
  __shared__ int tmp[NT / 64];
  __shared__ int sh_bin, sh_need;

  uint32_t tau;
  int need;
  if (k <= 0) {
    tau = 0xffffffffu;  // no key exceeds or equals it (NaN keys never reach 0xffffffff)
    need = 0;
  } else if (k >= L_r) {
    tau = 0u;           // every real key is above it
    need = 0;
  } else {
    uint32_t prefix = 0, pmask = 0;
    need = k;
    const int shifts[3] = {21, 10, 0};
    const int bins[3] = {2048, 2048, 1024};
    for (int p = 0; p < 3; ++p) {
      const int sh = shifts[p], nb = bins[p];
      for (int j = threadIdx.x; j < nb; j += NT) hist[j] = 0;
      __syncthreads();
      for (int t = threadIdx.x; t < L_r; t += NT) {
        const uint32_t key = score_key(s[t]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      find_bin_from_top<NT>(hist, nb, need, tmp, &sh_bin, &sh_need);
      prefix |= (uint32_t)sh_bin << sh;
      pmask |= (uint32_t)(nb - 1) << sh;
      need = sh_need;
      __syncthreads();
    }
    tau = prefix;
  }

  // ---- emit in index order, one 32-token word per thread per step ----------
  const int nwords_row = (L + 31) / 32;
  const int nwords_act = (L_r + 31) / 32;
  const int w_lo = max(0, L_r - n_window);
  int32_t* irow = idx ? idx + row * (long long)cap : nullptr;
  uint32_t* brow = bitmask ? bitmask + row * (long long)nwords_row : nullptr;
  int tie_carry = 0, pos_carry = 0;
  for (int w0 = 0; w0 < nwords_row; w0 += NT) {
    const int w = w0 + threadIdx.x;
    uint32_t gt = 0, eq = 0, forced = 0;
    if (w < nwords_act) {
      const int tb = w * 32;
      const int n = min(32, L_r - tb);
      for (int j = 0; j < n; ++j) {
        const int t = tb + j;
        const uint32_t key = score_key(s[t]);
        gt |= (uint32_t)(key > tau) << j;
        eq |= (uint32_t)(key == tau) << j;
        forced |= (uint32_t)(t < n_sink || t >= w_lo) << j;
      }
    }
    int ties_total;
    const int tie_before = block_exclusive_sum<NT>(__popc(eq), ties_total, tmp);
    uint32_t take = 0;
    int rank = tie_carry + tie_before;
    for (uint32_t e = eq; e; e &= e - 1) {
      const int j = __ffs(e) - 1;
      if (rank < need) take |= 1u << j;
      ++rank;
    }
    const uint32_t sel = gt | take | forced;
    int sel_total;
    const int pos_before = block_exclusive_sum<NT>(__popc(sel), sel_total, tmp);
    if (w < nwords_row) {
      if (brow) brow[w] = sel;
      if (irow) {
        int pos = pos_carry + pos_before;
        for (uint32_t e = sel; e; e &= e - 1) {
          if (pos < cap) irow[pos] = w * 32 + (__ffs(e) - 1);
          ++pos;
        }
      }
    }
    tie_carry += ties_total;
    pos_carry += sel_total;
  }
  if (threadIdx.x == 0) count[row] = pos_carry;
}

}  // namespace

size_t select_workspace(int rows, int L, int Lq) {
  (void)rows; (void)L; (void)Lq;
  return 0;
}

hipError_t launch_select(hipStream_t s, const float* scores, int num, int den, int n_sink,
                         int n_window, int32_t* idx, uint32_t* bitmask, int32_t* count,
                         int B, int Hkv, int Lq, int L, int cap, int q_pos0, int causal,
                         void* ws) {
  (void)ws;
  const long long rows = (long long)B * Hkv * Lq;
  unsigned gx = (unsigned)(rows < 65536 ? rows : 65536);
  unsigned gy = (unsigned)((rows + gx - 1) / gx);
  if ((long long)gx * gy != rows) {
    // rows is not a multiple of 65536: fall back to a 1-D grid when it fits
    gx = (unsigned)rows;
    gy = 1;
  }
  hipLaunchKernelGGL((select_rows_kernel<kSelThreads>), dim3(gx, gy), dim3(kSelThreads), 0, s,
                     scores, num, den, n_sink, n_window, idx, bitmask, count, Lq, L, cap,
                     q_pos0, causal);
  return hipGetLastError();
}

}  // namespace butler
