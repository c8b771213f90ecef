// The fixed-budget selection rule shared by the selection kernels (TokenButler model card,
// Method and Memory requirements): how many tokens a row ranks, and the key it ranks by.
#pragma once
#include "common.h"

namespace butler {

enum { kModeNormal = 0, kModeNone = 1, kModeAll = 2 };

// x = floor(L_r * num / den) ranked over every token (fo == 0), or over the tokens that
// are neither sink nor window (fo != 0: the budget excludes the forced tokens).
__device__ __forceinline__ int row_mode(int L_r, int num, int den, int n_sink, int n_window,
                                        int fo, int& k) {
  const long long x = (long long)L_r * num / den;
  int pool = L_r;
  if (fo) {
    const int s = min(n_sink, L_r), w_lo = max(0, L_r - n_window);
    pool = L_r - (s + (L_r - max(w_lo, s)));   // tokens outside [0, s) U [w_lo, L_r)
  }
  k = (int)min<long long>(x, (long long)pool);
  return k <= 0 ? kModeNone : (k >= pool ? kModeAll : kModeNormal);
}

// Ranking key of token t: the order-preserving score key, or 0 -- below every score's key
// (NaN and -inf rank at 0x007fffff) -- for a forced token when the budget excludes them.
__device__ __forceinline__ uint32_t rank_key(float f, int t, int n_sink, int w_lo, int fo) {
  // a mask rather than a choice, so that no branch forms around the key of each slot
  const uint32_t keep = (fo && (t < n_sink || t >= w_lo)) ? 0u : 0xffffffffu;
  return score_key(f) & keep;
}

}  // namespace butler
