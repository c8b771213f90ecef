// Device helpers shared by the libbutler kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define BUTLER_WAVE 64

typedef uint16_t bf16_t;

// bf16 <-> fp32.  bf16 is the upper half of an IEEE fp32; the narrowing rounds
// to nearest, ties to even, and keeps NaN a (quiet) NaN.
__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float64 -> bf16 rounded once to nearest even.  The double is first rounded to odd
// into float32 (truncate, then set the last bit when anything was dropped); a
// round-to-nearest-even from there to bf16 is then the correctly rounded result,
// because float32 keeps at least two more bits than bf16.
__device__ __forceinline__ uint16_t d2bf(double d) {
  const float t = __double2float_rz(d);
  uint32_t u = __float_as_uint(t);
  if ((double)t != d && (u & 0x7fffffffu) < 0x7f800000u) u |= 1u;
  return f2bf(__uint_as_float(u));
}

// Element loaders: 16 bytes -> 8 (bf16) or 4 (fp32) floats.
template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const bf16_t* p, float* out) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = __uint_as_float(w[j] << 16);
      out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void load_raw(const bf16_t* p, uint4& v) {
    v = *reinterpret_cast<const uint4*>(p);
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float* out) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
};

__device__ __forceinline__ float load_elem(const bf16_t* p) { return bf2f(*p); }
__device__ __forceinline__ float load_elem(const float* p) { return *p; }

// Monotone key of a score: larger key <=> larger score.  NaN ranks as -inf and
// -0 as +0, so equal scores always give equal keys.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exp2 on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive wave-wide prefix sum (wave64).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive block-wide prefix sum over NT threads; `tmp` holds NT/64 ints of
// LDS.  Returns this thread's exclusive prefix and the block total.
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int& total, int* tmp) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int inc = wave_inclusive_sum(v);
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    int w = (lane < NW) ? tmp[lane] : 0;
    w = wave_inclusive_sum(w);
    if (lane < NW) tmp[lane] = w;
  }
  __syncthreads();
  const int before = wid ? tmp[wid - 1] : 0;
  total = tmp[NW - 1];
  __syncthreads();
  return before + inc - v;
}

template <int NT>
__device__ __forceinline__ float block_sum_f(float v, float* tmp) {
  constexpr int NW = NT / 64;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += tmp[w];
  __syncthreads();
  return s;
}

__device__ __forceinline__ float neg_inf() { return __uint_as_float(0xff800000u); }

// Cross-lane moves inside a row of 16 lanes (DPP), as floats.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes (N in 1..64, a power of two).  Every
// step adds the same two partial sums in both lanes of a pair, so all lanes of a group
// end with bitwise the same total.  Within 16 lanes the steps are DPP moves (quad
// permutations, then the half-row and row mirrors); wider groups add LDS permutes.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_f<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_f<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp_f<0x140>(x);  // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// 16 raw bytes of a row.
struct Raw16 {
  uint4 v;
  __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const uint4*>(p); }
};
template <typename T> __device__ __forceinline__ void unpack16(const Raw16& r, float* out);
template <> __device__ __forceinline__ void unpack16<bf16_t>(const Raw16& r, float* out) {
  const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(w[j] << 16);
    out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
// Element e of 16 raw bytes as a float (e < 8 for bf16, e < 4 for float).
template <typename T> __device__ __forceinline__ float elem16(const uint4& v, int e);
template <> __device__ __forceinline__ float elem16<bf16_t>(const uint4& v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}
template <> __device__ __forceinline__ float elem16<float>(const uint4& v, int e) {
  return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
}
template <> __device__ __forceinline__ void unpack16<float>(const Raw16& r, float* out) {
  out[0] = __uint_as_float(r.v.x); out[1] = __uint_as_float(r.v.y);
  out[2] = __uint_as_float(r.v.z); out[3] = __uint_as_float(r.v.w);
}

// Sum of a double over aligned groups of N lanes (N in {1, 2, 4, 8}): quad-permute DPP
// moves of both 32-bit halves, then one xor-4 shuffle for N = 8; every lane of a group
// ends with the same bits.
template <int N>
__device__ __forceinline__ double quad_sum_d(double x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "group of 1, 2, 4 or 8 lanes");
  if constexpr (N >= 2) {
    const int lo = __double2loint(x), hi = __double2hiint(x);
    x += __hiloint2double(__builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false),
                          __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false));
  }
  if constexpr (N >= 4) {
    const int lo = __double2loint(x), hi = __double2hiint(x);
    x += __hiloint2double(__builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false),
                          __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false));
  }
  if constexpr (N >= 8) x += __shfl_xor(x, 4);
  return x;
}
