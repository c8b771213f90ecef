// Selection cache (TokenSelect README, highlights, Selection Cache): consecutive similar
// queries share one token selection.  One wave per (b, KV head) compares the group's
// current query -- its R heads stacked into one R*D vector -- with the reference query the
// cached selection was made for, by cosine similarity in float32.  Similar enough: the
// (b, KV head) keeps its selection (score and select skip its rows).  Otherwise the
// reference takes the current query and the selection is recomputed.
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(64) void selection_cache_kernel(const T* __restrict__ q,
                                                             T* __restrict__ q_ref,
                                                             int32_t* __restrict__ keep, int Hq,
                                                             int Hkv, float threshold) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPH = D / EPL;   // lanes per head row
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int R = Hq / Hkv;
  const int lane = threadIdx.x;
  // lane covers elements [EPL*lane .. +EPL) of head rows r = lane / LPH + j * (64 / LPH)
  float qq = 0.f, rr = 0.f, qr = 0.f;
  const int rows_per_pass = 64 / LPH;
  for (int r0 = 0; r0 < R; r0 += rows_per_pass) {
    const int r = r0 + lane / LPH;
    if (r < R) {
      const long long off = ((long long)b * Hq + g * R + r) * D + (lane % LPH) * EPL;
      float a[EPL], c[EPL];
      Vec16<T>::load(q + off, a);
      Vec16<T>::load(q_ref + off, c);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        qq = fmaf(a[e], a[e], qq);
        rr = fmaf(c[e], c[e], rr);
        qr = fmaf(a[e], c[e], qr);
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    qq += __shfl_xor(qq, o);
    rr += __shfl_xor(rr, o);
    qr += __shfl_xor(qr, o);
  }
  const float den = sqrtf(qq) * sqrtf(rr);
  const float cosv = (den > 0.f) ? qr / den : 0.f;
  const bool hit = cosv >= threshold;
  if (lane == 0) keep[bg] = hit ? 1 : 0;
  if (!hit) {
    // refresh the reference with the current query
    for (int r0 = 0; r0 < R; r0 += rows_per_pass) {
      const int r = r0 + lane / LPH;
      if (r < R) {
        const long long off = ((long long)b * Hq + g * R + r) * D + (lane % LPH) * EPL;
        *reinterpret_cast<uint4*>(q_ref + off) = *reinterpret_cast<const uint4*>(q + off);
      }
    }
  }
}

}  // namespace

hipError_t launch_selection_cache(hipStream_t s, int dtype, const void* q, void* q_ref,
                                  int32_t* keep, int B, int Hq, int Hkv, int D, float threshold) {
  const dim3 grid((unsigned)(B * Hkv));
  if (dtype == 1) {
    if (D == 128)
      hipLaunchKernelGGL((selection_cache_kernel<bf16_t, 128>), grid, dim3(64), 0, s,
                         (const bf16_t*)q, (bf16_t*)q_ref, keep, Hq, Hkv, threshold);
    else
      hipLaunchKernelGGL((selection_cache_kernel<bf16_t, 64>), grid, dim3(64), 0, s,
                         (const bf16_t*)q, (bf16_t*)q_ref, keep, Hq, Hkv, threshold);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((selection_cache_kernel<float, 128>), grid, dim3(64), 0, s,
                         (const float*)q, (float*)q_ref, keep, Hq, Hkv, threshold);
    else
      hipLaunchKernelGGL((selection_cache_kernel<float, 64>), grid, dim3(64), 0, s,
                         (const float*)q, (float*)q_ref, keep, Hq, Hkv, threshold);
  }
  return hipGetLastError();
}

}  // namespace butler
