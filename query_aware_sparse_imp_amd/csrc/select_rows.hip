// Fixed-budget top-x + sink + window selection for calls with many query rows (causal
// prefill chunks, multi-query calls) of up to 8192 tokens (TokenButler model card, Method
// and Memory requirements: every query row keeps its own top fraction of the causal prefix,
// plus the sink and the recent window).
//
// One wave per row and no barrier anywhere: a workgroup is four independent rows.  The
// wave holds its row's keys in VGPRs (lane l, slot j: token l + 64 j, so a ballot over one
// slot is the 64-token word j of the row in index order), and finds the x-th largest key
// tau exactly with the same three radix digits as the other selection kernels (key bits
// 31..21, 20..10, 9..0), on a histogram of its own in LDS: 2048 counts of 16 bits packed
// two to a word (a row has at most 8192 tokens), 4 KB per wave.  A digit's bin is found
// by a wave prefix sum over 64 lanes of 32 (16) bins each, scanned from the top, and one
// lane's walk of its bins.  The emit then walks the slots in index order with running
// counts in scalar registers: the rank of every key equal to tau (only when the budget
// splits them), the output position, and the bitmask words, gathered 64 to a VGPR and
// stored as whole 256-byte lines.
//
// Compared with one workgroup per row, a row's phases wait on nothing but its own wave:
// many more rows are resident per CU (a CU holds up to 32 rows of 1024 tokens, 12 of
// 8192), so one row's score loads overlap other rows' radix passes.
#include "common.h"
#include "kernels.h"
#include "select_rule.h"

#include <type_traits>

namespace butler {
namespace {

constexpr int kSwWaves = 4;      // rows per workgroup
constexpr int kSwWords = 1024;   // 2048 bins, two 16-bit counts per word

// Orders the wave's LDS accesses of one phase before those of the next: a wave's LDS
// instructions run in issue order, so only the compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// A copy of v that the compiler cannot see through: the per-slot tests of each phase are
// then formed afresh instead of being kept live (in scalar registers, one pair per slot)
// from the phase that first formed them.
__device__ __forceinline__ int opaque_v(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ int opaque_s(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

// Exclusive prefix sum over the 64 lanes (lane 0 first).
__device__ __forceinline__ int wave_exclusive_sum(int v, int lane) {
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  return incl - v;
}

// Among the NB bins of hist (packed 16-bit counts), scanned from the top bin down, the bin
// that holds the need-th largest key (1 <= need <= the total count), the rank left inside
// it, and its count.  Lane l covers bins [NB - (l + 1) P, NB - l P), P = NB / 64.
template <int NB>
__device__ __forceinline__ void wave_find_bin(const uint32_t* hist, int need, int lane,
                                              int& bin, int& need_in, int& cnt) {
  constexpr int P = NB / 64, WPL = P / 2;
  const int base = NB / 2 - (lane + 1) * WPL;   // first word of this lane's bins
  uint32_t w[WPL];
#pragma unroll
  for (int q = 0; q < WPL / 4; ++q) {
    const uint4 v = reinterpret_cast<const uint4*>(hist + base)[q];
    w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
  }
  uint32_t sum = 0;
#pragma unroll
  for (int m = 0; m < WPL; ++m) sum += w[m];   // low halves stay below 2^16: no carry
  const int local = (int)(sum & 0xffffu) + (int)(sum >> 16);
  const int above = wave_exclusive_sum(local, lane);
  const uint64_t hit = __ballot(above < need && need <= above + local);
  const int f = __builtin_amdgcn_readfirstlane((int)__ffsll((unsigned long long)hit) - 1);
  int b_f = 0, n_f = 0, c_f = 0;
  if (lane == f) {
    int run = above;
    bool done = false;
#pragma unroll
    for (int m = WPL - 1; m >= 0; --m) {
#pragma unroll
      for (int h = 1; h >= 0; --h) {
        const int c = (int)((w[m] >> (16 * h)) & 0xffffu);
        if (!done && run + c >= need) {
          done = true;
          b_f = 2 * (base + m) + h;
          n_f = need - run;
          c_f = c;
        }
        run += c;
      }
    }
  }
  bin = __builtin_amdgcn_readlane(b_f, f);
  need_in = __builtin_amdgcn_readlane(n_f, f);
  cnt = __builtin_amdgcn_readlane(c_f, f);
}

// Histogram of digit (key >> SH) & (NB - 1) over the valid keys that share prefix under
// pmask (every valid key when ALL), then the bin of the need-th largest.
template <int KPT, int NB, int SH, bool ALL>
__device__ __forceinline__ void wave_digit(const uint32_t (&key)[KPT], uint32_t* hist,
                                           int lane, int L_r, uint32_t prefix, uint32_t pmask,
                                           int need, int& bin, int& need_in, int& cnt) {
  uint4* h4 = reinterpret_cast<uint4*>(hist);
#pragma unroll
  for (int q = 0; q < NB / 2 / 4 / 64; ++q) h4[lane + 64 * q] = make_uint4(0u, 0u, 0u, 0u);
  wave_lds_order();
  const int ln = opaque_v(lane), lr = opaque_s(L_r);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t d = (key[j] >> SH) & (NB - 1);
    const uint32_t inc = 1u << ((d & 1u) << 4);
    if constexpr (ALL) {
      // every slot adds, past the row's end nothing (no branch around the atomic)
      atomicAdd(&hist[d >> 1], ln + 64 * j < lr ? inc : 0u);
    } else {
      if (ln + 64 * j < lr && (key[j] & pmask) == prefix) atomicAdd(&hist[d >> 1], inc);
    }
  }
  wave_lds_order();
  wave_find_bin<NB>(hist, need, lane, bin, need_in, cnt);
  wave_lds_order();
}

// Waves per SIMD asked of the register allocator: the row's keys take KPT registers.
constexpr int sw_waves_per_simd(int kpt) { return kpt >= 96 ? 3 : (kpt >= 64 ? 4 : (kpt >= 48 ? 5 : 1)); }

template <int KPT>
__global__ __launch_bounds__(64 * kSwWaves, sw_waves_per_simd(KPT)) void select_wave_kernel(
    const float* __restrict__ scores, int num, int den, int n_sink, int n_window, int fo,
    int32_t* __restrict__ idx, uint32_t* __restrict__ bitmask, int32_t* __restrict__ count,
    long long rows, int Lq, int L, int cap, int q_pos0, int causal) {
  __shared__ __align__(16) uint32_t hist_all[kSwWaves][kSwWords];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const long long row = (long long)blockIdx.x * kSwWaves + wid;
  if (row >= rows) return;
  uint32_t* hist = hist_all[wid];
  const int i = (int)(row % Lq);
  const int L_r = causal ? min(q_pos0 + i + 1, L) : L;
  int k;
  const int mode = row_mode(L_r, num, den, n_sink, n_window, fo, k);
  const int w_lo = max(0, L_r - n_window);
  const float* s = scores + row * (long long)L;

  // every load at once, before any key is formed (a conversion next to each load would
  // make the compiler wait for each load in turn), through a buffer resource whose range
  // is the row's L_r scores: slots past the end read 0 (masked below) instead of needing
  // a clamped address each, and all loads share one offset register
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)s, (short)0, L_r * 4, 0x00020000);
  float raw[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    raw[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (lane + 64 * j), 0, 0));
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = rank_key(raw[j], lane + 64 * j, n_sink, w_lo, fo);

  // tau: the k-th largest key; need: how many keys equal to tau the budget takes
  uint32_t tau = 0;
  int need = 0, n_eq = 0;
  if (mode == kModeNormal) {
    int b0, b1, b2, n0, n1;
    wave_digit<KPT, 2048, 21, true>(key, hist, lane, L_r, 0u, 0u, k, b0, n0, n_eq);
    const uint32_t p0 = (uint32_t)b0 << 21;
    wave_digit<KPT, 2048, 10, false>(key, hist, lane, L_r, p0, 0xffe00000u, n0, b1, n1, n_eq);
    const uint32_t p1 = p0 | ((uint32_t)b1 << 10);
    wave_digit<KPT, 1024, 0, false>(key, hist, lane, L_r, p1, 0xfffffc00u, n1, b2, need, n_eq);
    tau = p1 | (uint32_t)b2;
  }

  // ---- emit in index order ----------------------------------------------------------
  const int nwords = (L + 31) / 32;   // <= 2 KPT: the instance covers the row stride L
  uint32_t* brow = bitmask ? bitmask + row * (long long)nwords : nullptr;
  int32_t* irow = idx ? idx + row * (long long)cap : nullptr;
  // without a tie cut a key is taken iff key >= lo: 0 takes every key, and no key reaches
  // 0xffffffff (the largest, +inf's, is 0xff800000)
  const uint32_t lo = mode == kModeAll ? 0u : (mode == kModeNormal ? tau : 0xffffffffu);
  const bool odd = lane & 1;
  const int pair = lane >> 1;
  int sel_base = 0;
  auto emit = [&](auto ties_c, auto idx_c, auto bm_c) {
    constexpr bool TIES = decltype(ties_c)::value, IDX = decltype(idx_c)::value,
                   BM = decltype(bm_c)::value;
    int tie_base = 0;
    uint32_t wordv = 0;
    const int ln = opaque_v(lane), lr = opaque_s(L_r);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      // bitwise rather than short-circuit logic: lane masks combined by scalar instructions
      const int t = ln + 64 * j;
      const bool v = t < lr;
      const bool forced = (t < n_sink) | (t >= w_lo);
      bool sel;
      if constexpr (TIES) {
        // the budget takes the need lowest-index keys equal to tau
        const bool eq = v & (key[j] == tau);
        const uint64_t e = __ballot(eq);
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(e >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)e, tie_base));
        tie_base += __popcll(e);
        sel = v & (forced | (key[j] > tau) | (eq & (rank < need)));
      } else {
        sel = v & (forced | (key[j] >= lo));
      }
      const uint64_t b = __ballot(sel);
      if constexpr (IDX) {
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)b, sel_base));
        if (sel && pos < cap) irow[pos] = t;
      }
      sel_base = opaque_s(sel_base + __popcll(b));   // counted now: b need not stay live
      if constexpr (BM) {
        // lanes 2m and 2m + 1 of group j / 32 take the two halves of word j (m = j % 32)
        const uint32_t half = odd ? (uint32_t)(b >> 32) : (uint32_t)b;
        wordv = (uint32_t)opaque_v((int)((pair == (j & 31)) ? half : wordv));   // now, not
                                                                                   // at the store
        if ((j & 31) == 31 || j == KPT - 1) {
          const int wd = 64 * (j >> 5) + lane;
          if (wd < nwords) brow[wd] = wordv;
          wordv = 0;
        }
      }
      // one slot at a time: hoisting the next slots' ballots would only raise the register
      // pressure (each ballot is a pair of scalar registers)
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  const bool ties = mode == kModeNormal && n_eq > need;
  if (ties) {
    if (irow && brow) emit(T_(), T_(), T_());
    else if (irow) emit(T_(), T_(), F_());
    else emit(T_(), F_(), T_());
  } else {
    if (irow && brow) emit(F_(), T_(), T_());
    else if (irow) emit(F_(), T_(), F_());
    else emit(F_(), F_(), T_());
  }
  if (lane == 0) count[row] = sel_base;
}

}  // namespace

bool select_rows_fits(int Lq, int L) { return Lq > 1 && L >= 1 && L <= 8192; }

hipError_t launch_select_rows(hipStream_t s, const float* scores, int num, int den, int n_sink,
                              int n_window, int fo, int32_t* idx, uint32_t* bitmask,
                              int32_t* count, int B, int Hs, int Lq, int L, int cap, int q_pos0,
                              int causal) {
  if (!select_rows_fits(Lq, L)) return hipErrorInvalidValue;
  const long long rows = (long long)B * Hs * Lq;
  const dim3 grid((unsigned)((rows + kSwWaves - 1) / kSwWaves));
  // keys per lane: the row stride rounded up to 1024 tokens
#define BUTLER_SW(KPT)                                                                     \
  hipLaunchKernelGGL((select_wave_kernel<KPT>), grid, dim3(64 * kSwWaves), 0, s, scores, num, \
                     den, n_sink, n_window, fo, idx, bitmask, count, rows, Lq, L, cap, q_pos0, \
                     causal)
  switch ((L + 1023) / 1024) {
    case 1: BUTLER_SW(16); break;
    case 2: BUTLER_SW(32); break;
    case 3: BUTLER_SW(48); break;
    case 4: BUTLER_SW(64); break;
    case 5: BUTLER_SW(80); break;
    case 6: BUTLER_SW(96); break;
    case 7: BUTLER_SW(112); break;
    default: BUTLER_SW(128); break;
  }
#undef BUTLER_SW
  return hipGetLastError();
}

}  // namespace butler
