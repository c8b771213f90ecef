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
constexpr int kSwCand = 256;     // tau's first-digit bin resolved without more radix passes

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

// Order-preserving key of a score, equal to score_key in five vector instructions: the
// max with -inf turns NaN into -inf and adding +0 turns -0 into +0 (IEEE arithmetic, with
// denormals kept), then a negative value has every bit flipped and a non-negative one its
// sign bit set.
__device__ __forceinline__ uint32_t fast_key(float f) {
  const float g = fmaxf(f, -__builtin_inff()) + 0.0f;
  const uint32_t u = __float_as_uint(g);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// A wave's radix histogram: NB counts, 32-bit (8 KB for 2048 bins), or 16-bit packed two
// to a word (PACKED: word w holds bins 2w and 2w + 1) for the short-row instances, whose
// many resident waves would not fit 8 KB each in LDS.
template <bool PACKED>
constexpr int sw_words(int nb) { return PACKED ? nb / 2 : nb; }

// Count of bin b in hist.
template <bool PACKED>
__device__ __forceinline__ int bin_count(const uint32_t* hist, int b) {
  if constexpr (PACKED)
    return (int)((hist[b >> 1] >> ((b & 1) << 4)) & 0xffffu);
  else
    return (int)hist[b];
}

// Among the NB bins of hist, scanned from the top bin down, the bin that holds the need-th
// largest key (1 <= need <= the total count), the rank left inside it, and its count.
// Lane l sums bins [NB - (l + 1) P, NB - l P), P = NB / 64; a prefix sum over the lanes
// finds the lane f whose bins hold the rank, then lane m < P takes f's bin NB - f P - 1 - m
// (from the top) and a second prefix sum finds the bin.
template <int NB, bool PACKED>
__device__ __forceinline__ void wave_find_bin(const uint32_t* hist, int need, int lane,
                                              int& bin, int& need_in, int& cnt) {
  constexpr int P = NB / 64, WPL = PACKED ? P / 2 : P;
  const int base = sw_words<PACKED>(NB) - (lane + 1) * WPL;   // first word of this lane's bins
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < WPL / 4; ++q) {
    const uint4 v = reinterpret_cast<const uint4*>(hist + base)[q];
    sum += v.x + v.y + v.z + v.w;   // packed: the low halves stay below 2^16
  }
  const int local = PACKED ? (int)(sum & 0xffffu) + (int)(sum >> 16) : (int)sum;
  const int above = wave_exclusive_sum(local, lane);
  const uint64_t hit = __ballot(above < need && need <= above + local);
  const int f = __builtin_amdgcn_readfirstlane((int)__ffsll((unsigned long long)hit) - 1);
  const int above_f = __builtin_amdgcn_readlane(above, f);
  const int b = NB - f * P - 1 - lane;   // lane m < P: f's bins from the top down
  const int c = lane < P ? bin_count<PACKED>(hist, b) : 0;
  const int run = above_f + wave_exclusive_sum(c, lane);   // keys above bin b
  const uint64_t hit2 = __ballot(lane < P && run < need && need <= run + c);
  const int g = __builtin_amdgcn_readfirstlane((int)__ffsll((unsigned long long)hit2) - 1);
  bin = __builtin_amdgcn_readlane(b, g);
  need_in = need - __builtin_amdgcn_readlane(run, g);
  cnt = __builtin_amdgcn_readlane(c, g);
}

template <int NB, bool PACKED>
__device__ __forceinline__ void wave_clear(uint32_t* hist, int lane) {
  uint4* h4 = reinterpret_cast<uint4*>(hist);
#pragma unroll
  for (int q = 0; q < sw_words<PACKED>(NB) / 4 / 64; ++q)
    h4[lane + 64 * q] = make_uint4(0u, 0u, 0u, 0u);
  wave_lds_order();
}

template <bool PACKED>
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t d) {
  if constexpr (PACKED)
    atomicAdd(&hist[d >> 1], 1u << ((d & 1u) << 4));
  else
    atomicAdd(&hist[d], 1u);
}

// First radix digit (key bits 31..21) of the row's L_r keys, then the bin of the need-th
// largest.  Slots wholly inside the row add with every lane, the one slot that holds the
// row's end with its valid lanes, and slots past the end not at all.
template <int KPT, bool PACKED>
__device__ __forceinline__ void wave_digit0(const uint32_t (&key)[KPT], uint32_t* hist,
                                            int lane, int L_r, int need, int& bin,
                                            int& need_in, int& cnt) {
  wave_clear<2048, PACKED>(hist, lane);
  const int lr = opaque_s(L_r);
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (__builtin_expect(64 * j < lr, 1)) hist_add<PACKED>(hist, key[j] >> 21);
  wave_lds_order();
  // the slot that holds the row's end added its lanes past the end (keys of 0) to bin 0
  if ((lr & 63) && lane == 0) hist[0] -= (uint32_t)(64 - (lr & 63));
  wave_lds_order();
  wave_find_bin<2048, PACKED>(hist, need, lane, bin, need_in, cnt);
  wave_lds_order();
}

// A later digit (key >> SH) & (NB - 1) over the keys that share prefix under pmask (a key
// zeroed as past the row's end or forced never does: prefix holds a first digit of 3 or
// more), then the bin of the need-th largest.
template <int KPT, int NB, int SH, bool PACKED>
__device__ __forceinline__ void wave_digit(const uint32_t (&key)[KPT], uint32_t* hist,
                                           int lane, uint32_t prefix, uint32_t pmask,
                                           int need, int& bin, int& need_in, int& cnt) {
  wave_clear<NB, PACKED>(hist, lane);
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((key[j] & pmask) == prefix) hist_add<PACKED>(hist, (key[j] >> SH) & (NB - 1));
  wave_lds_order();
  wave_find_bin<NB, PACKED>(hist, need, lane, bin, need_in, cnt);
  wave_lds_order();
}

// Waves per SIMD asked of the register allocator: the row's keys take KPT registers.
constexpr int sw_waves_per_simd(int kpt) { return kpt >= 96 ? 3 : (kpt >= 64 ? 4 : (kpt >= 48 ? 5 : 1)); }

template <int KPT>
__global__ __launch_bounds__(64 * kSwWaves, sw_waves_per_simd(KPT)) void select_wave_kernel(
    const float* __restrict__ scores, int num, int den, int n_sink, int n_window, int fo,
    int32_t* __restrict__ idx, uint32_t* __restrict__ bitmask, int32_t* __restrict__ count,
    long long rows, int Lq, int L, int cap, int q_pos0, int causal) {
  constexpr bool PACKED = KPT < 48;
  __shared__ __align__(16) uint32_t hist_all[kSwWaves][sw_words<PACKED>(2048)];
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
  // is the row's L_r scores: slots past the end read 0 instead of needing a clamped
  // address each, and all loads share one offset register
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)s, (short)0, L_r * 4, 0x00020000);
  float raw[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    raw[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (lane + 64 * j), 0, 0));
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = fast_key(raw[j]);
  // keys that do not rank become 0, below every score's key (-inf's is 0x007fffff): the
  // slots past the row's end, and the forced tokens when the budget excludes them; only
  // the slots that hold such a token are touched
  {
    const int ln = opaque_v(lane), lr = opaque_s(L_r), ns = opaque_s(n_sink), wl = opaque_s(w_lo);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (64 * j + 64 > lr || (fo && (64 * j < ns || 64 * j + 64 > wl))) {
        const int t = ln + 64 * j;
        key[j] = ((t >= lr) | (fo && ((t < ns) | (t >= wl)))) ? 0u : key[j];
      }
    }
  }

  // tau: the k-th largest key; need: how many keys equal to tau the budget takes
  uint32_t tau = 0;
  int need = 0, n_eq = 0;
  if (mode == kModeNormal) {
    int b0, b1, b2, n0, n1, c0;
    wave_digit0<KPT, PACKED>(key, hist, lane, L_r, k, b0, n0, c0);
    const uint32_t p0 = (uint32_t)b0 << 21;
    if (c0 <= kSwCand) {
      // few keys share tau's first digit: gather them into LDS, four per lane at most,
      // and find the n0-th largest of them bit by bit (21 ballot counts), no histogram
      int base = 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const bool m = (key[j] >> 21) == (uint32_t)b0;
        const uint64_t bm = __ballot(m);
        if (bm) {
          const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bm, base));
          if (m & (pos < kSwCand)) hist[pos] = key[j];   // pos < c0: the same keys were counted
          base = opaque_s(base + __popcll(bm));
        }
      }
      wave_lds_order();
      uint32_t c[kSwCand / 64];
#pragma unroll
      for (int q = 0; q < kSwCand / 64; ++q) c[q] = (lane + 64 * q < c0) ? hist[lane + 64 * q] : 0u;
      wave_lds_order();
      // the zero padding never counts: the n0-th largest candidate is a score's key (the
      // budget takes fewer keys than there are non-forced tokens), at least -inf's
      // 0x007fffff, so t > 0
      uint32_t t = p0;
#pragma unroll
      for (int bit = 20; bit >= 0; --bit) {
        const uint32_t trial = t | (1u << bit);
        int n = 0;
#pragma unroll
        for (int q = 0; q < kSwCand / 64; ++q) n += __popcll(__ballot(c[q] >= trial));
        t = n >= n0 ? trial : t;
      }
      int n_gt = 0;
#pragma unroll
      for (int q = 0; q < kSwCand / 64; ++q) {
        n_gt += __popcll(__ballot(c[q] > t));
        n_eq += __popcll(__ballot(c[q] == t));
      }
      tau = t;
      need = n0 - n_gt;
    } else {
      wave_digit<KPT, 2048, 10, PACKED>(key, hist, lane, p0, 0xffe00000u, n0, b1, n1, n_eq);
      const uint32_t p1 = p0 | ((uint32_t)b1 << 10);
      wave_digit<KPT, 1024, 0, PACKED>(key, hist, lane, p1, 0xfffffc00u, n1, b2, need, n_eq);
      tau = p1 | (uint32_t)b2;
    }
  }

  // ---- emit in index order ----------------------------------------------------------
  const int nwords = (L + 31) / 32;   // <= 2 KPT: the instance covers the row stride L
  uint32_t* brow = bitmask ? bitmask + row * (long long)nwords : nullptr;
  int32_t* irow = idx ? idx + row * (long long)cap : nullptr;
  const bool ties = mode == kModeNormal && n_eq > need;
  // without a tie cut a token is taken iff it is forced or key >= lo: lo = 1 takes every
  // score (0 is past the row's end), and no score's key reaches 0xffffffff (the largest,
  // +inf's, is 0xff800000)
  const uint32_t lo = mode == kModeAll ? 1u : (mode == kModeNormal ? tau : 0xffffffffu);
  const bool odd = lane & 1;
  const int pair = lane >> 1;
  int sel_base = 0;
  auto emit = [&](auto ties_c, auto idx_c, auto bm_c) {
    constexpr bool TIES = decltype(ties_c)::value, IDX = decltype(idx_c)::value,
                   BM = decltype(bm_c)::value;
    int tie_base = 0;
    uint32_t wordv = 0;
    const int ln = opaque_v(lane), lr = opaque_s(L_r), ns = opaque_s(n_sink),
              wl = opaque_s(w_lo);
    // slots [js, js + span) hold no forced token: one unsigned range test per slot
    const int nsr = min(ns, lr);
    const int js = (nsr + 63) >> 6, span = opaque_s(max((wl >> 6) - js, 0));
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      int rank = 0;
      if constexpr (TIES) {
        // the budget takes the need lowest-index keys equal to tau (a zeroed key never is)
        const uint64_t e = __ballot(key[j] == tau);
        rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(e >> 32),
                                         __builtin_amdgcn_mbcnt_lo((uint32_t)e, tie_base));
        tie_base += __popcll(e);
      }
      uint64_t b;
      if constexpr (TIES) {
        const int t = ln + 64 * j;
        const bool by_key = (key[j] > tau) | ((key[j] == tau) & (rank < need));
        b = __ballot((t < lr) & ((t < ns) | (t >= wl) | by_key));
      } else {
        // a ballot in each branch keeps the branch (the forced test runs only where needed)
        if ((unsigned)(j - js) >= (unsigned)span) {
          const int t = ln + 64 * j;
          b = __ballot((key[j] >= lo) | (t < nsr) | ((t >= wl) & (t < lr)));
        } else {
          b = __ballot(key[j] >= lo);
        }
      }
      if constexpr (IDX) {
        const bool sel = (b >> ln) & 1ull;
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)b, sel_base));
        if (sel && pos < cap) irow[pos] = ln + 64 * j;
      }
      sel_base = opaque_s(sel_base + __popcll(b));   // counted now: b need not stay live
      if constexpr (BM) {
        // lanes 2m and 2m + 1 of group j / 32 take the two halves of word j (m = j % 32)
        const uint32_t half = odd ? (uint32_t)(b >> 32) : (uint32_t)b;
        wordv = (uint32_t)opaque_v((int)((pair == (j & 31)) ? half : wordv));   // now, not
                                                                                   // at the store
        if ((j & 31) == 31 || j == KPT - 1) {
          const int wd = 64 * (j >> 5) + ln;
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
