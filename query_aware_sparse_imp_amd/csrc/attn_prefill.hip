// Prefill attention over bitmask rows on the matrix cores (TokenButler model card, Method:
// every query row attends to its own selected subset of the causal prefix).  bf16, D = 128,
// R = 4 query heads per KV head, the rows of one selection set per KV head.
#include "attn_tile.h"
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

// ---------------------------------------------------------------------------
// Prefill on the matrix cores (bf16, D = 128, R = 4): one workgroup per (b, KV head, 64
// query rows), one wave per query head of the group and 32-row group.  Key tiles of 64
// tokens run from 0 to the block's causal end; each tile is staged in LDS once for the
// eight waves -- K as [token][d], V transposed to [d][token] (two tokens packed per 32-bit
// word) -- in two buffers each, K one tile ahead of V: a wave takes the logits of the next
// tile on the matrix cores beside the softmax of this one on the vector units (the two
// waves of a SIMD would otherwise reach each phase together), and one barrier separates
// two tiles.
//   S^T = K . Q^T        A = K rows (tokens), B = the wave's 32 queries (kept in VGPRs),
//                        as two 32-token halves (two accumulator sets)
//   O^T += V^T . P^T      A = V^T rows (d), B = P^T straight from the S^T accumulators,
//                        four 16-token K steps
// In the 32x32 accumulator layout lane l holds query l%32 and tokens 8(r/4) + 4(l/32) +
// r%4: ordered by r, that is exactly the MFMA B operand of a 16-token K step if the K
// order is permuted the same way on the V^T side (tokens {0-3, 8-11} for lanes 0-31,
// {4-7, 12-15} for lanes 32-63: two 8-byte LDS reads).  The query is the lane in both
// S^T and O^T, so the online softmax (max, rescale, sum) needs only the partner lane
// l ^ 32.  Masking comes from the row's bitmask words of the tile.  The kernel is bound by
// its vector work (the exponentials and the softmax around them), not by the matrix
// cores: the logits are masked with one bitfield extract and one bit-select each, the
// scale sits in the exponent's FMA, and the accumulators are rescaled only when some
// query's reference max moved, which it does only by more than 2^8 in probability.
// ---------------------------------------------------------------------------

typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

constexpr int kPfThreads = 256;
constexpr int kPfKS = 128 + 8;   // LDS row stride (bf16) of the K tile

// max of three floats that are finite or -inf.  fmaxf would first canonicalise each
// operand built by bit operations (one more instruction per logit); v_max3_f32 needs no
// canonical inputs for such values.
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

constexpr int kPfTok = 64;
constexpr int kPfVS = kPfTok + 4;   // LDS row stride (bf16) of the transposed V tile

__global__ __launch_bounds__(2 * kPfThreads) void attn_prefill_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const uint32_t* __restrict__ bitmask, float* __restrict__ out, int Hq, int Hkv, int Lq,
    int L, int L_cap, int q_pos0, float scale_log2) {
  constexpr int D = 128, R = 4, RG = 2;
  const int nrb = (Lq + 32 * RG - 1) / (32 * RG);
  const int rb = blockIdx.x % nrb, bg = blockIdx.x / nrb;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h = g * R + (wid & 3);
  const int i0 = rb * 32 * RG + 32 * (wid >> 2);
  const int ql = lane & 31, hi = lane >> 5;
  const int qi = min(i0 + ql, Lq - 1);
  const bool qvalid = i0 + ql < Lq;
  const int nwords = (L + 31) / 32;
  bf16x8_t qf[8];
  {
    const bf16_t* qr = q + (((long long)b * Hq + h) * Lq + qi) * D + 8 * hi;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) qf[s8] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 16 * s8));
  }
  const uint32_t* brow = bitmask + ((long long)bg * Lq + qi) * nwords;
  const bf16_t* kb = k + (long long)bg * L_cap * D;
  const bf16_t* vb = v + (long long)bg * L_cap * D;
  const int t_end = min(L, q_pos0 + min(rb * 32 * RG + 32 * RG, Lq));
  __shared__ __align__(16) bf16_t Ks[2][kPfTok * kPfKS];
  __shared__ __align__(16) bf16_t Vt[2][D * kPfVS];
  // staging roles: threads 256.. stage K (chunks c = kt + 256u: token c/16, d 8*(c%16)),
  // threads ..255 stage V token pairs tp = (tid + 256u) / 16 at d group dg = tid % 16
  const bool do_k = tid >= kPfThreads;
  const int kt = do_k ? tid - kPfThreads : tid;
  const int dg = tid & 15;
  uint4 rs[4];        // K: 4 chunks; V: 2 pairs x 2 tokens
  uint32_t wn0, wn1;  // bitmask words of the tile in flight
  // K rows of tile tk (K stagers) or V rows of tile tv (V stagers), clamped addresses
  auto gload = [&](int tk, int tv) {
    if (do_k) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = kt + kPfThreads * u;
        rs[u] = *reinterpret_cast<const uint4*>(kb + (long long)min(tk + (c >> 4), L - 1) * D + (c & 15) * 8);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tp = (tid + kPfThreads * u) >> 4;
        rs[2 * u] = *reinterpret_cast<const uint4*>(vb + (long long)min(tv + 2 * tp, L - 1) * D + dg * 8);
        rs[2 * u + 1] = *reinterpret_cast<const uint4*>(vb + (long long)min(tv + 2 * tp + 1, L - 1) * D + dg * 8);
      }
    }
  };
  auto gload_words = [&](int t0) {
    const int w0 = t0 >> 5;
    wn0 = brow[min(w0, nwords - 1)];
    const uint32_t w1 = brow[min(w0 + 1, nwords - 1)];
    wn1 = (w0 + 1 < nwords) ? w1 : 0u;   // past the last word: no tokens
  };
  // the held rows into K buffer kbuf (K stagers) or V buffer vbuf (V stagers)
  auto stage = [&](int kbuf, int vbuf) {
    if (do_k) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = kt + kPfThreads * u;
        *reinterpret_cast<uint4*>(&Ks[kbuf][(c >> 4) * kPfKS + (c & 15) * 8]) = rs[u];
      }
    } else {
      uint32_t* vw = reinterpret_cast<uint32_t*>(Vt[vbuf]);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tp = (tid + kPfThreads * u) >> 4;
        const uint32_t x0[4] = {rs[2 * u].x, rs[2 * u].y, rs[2 * u].z, rs[2 * u].w};
        const uint32_t x1[4] = {rs[2 * u + 1].x, rs[2 * u + 1].y, rs[2 * u + 1].z, rs[2 * u + 1].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vw[(8 * dg + 2 * j) * (kPfVS / 2) + tp] = (x0[j] & 0xffffu) | (x1[j] << 16);
          vw[(8 * dg + 2 * j + 1) * (kPfVS / 2) + tp] = (x0[j] >> 16) | (x1[j] & 0xffff0000u);
        }
      }
    }
  };
  // the logits S^T of the tile in K buffer kbuf: two 32-token halves
  auto logits = [&](int kbuf, f32x16_t& c0, f32x16_t& c1) {
    const bf16_t* Kc = Ks[kbuf];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      c0[r] = 0.f;
      c1[r] = 0.f;
    }
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(&Kc[ql * kPfKS + 16 * s8 + 8 * hi]);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(&Kc[(32 + ql) * kPfKS + 16 * s8 + 8 * hi]);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s8], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s8], c1, 0, 0, 0);
    }
  };
  float m = neg_inf(), msc = 0.f, l = 0.f;
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // K runs one tile ahead of V: iteration `it` takes the logits of tile it + 1 (matrix
  // cores) beside the softmax of tile it (vector units), then P.V of tile it.  Iteration it
  // reads K buffer (it+1)%2 and V buffer it%2 and refills K buffer it%2 with tile it + 2
  // and V buffer (it+1)%2 with tile it + 1: one barrier per tile.
  gload(0, 0);
  gload_words(0);
  stage(0, 0);
  gload(kPfTok, 0);
  stage(1, 0);   // V stagers store tile 0 again: the same values
  __syncthreads();
  f32x16_t s0, s1;   // logits of the current tile
  logits(0, s0, s1);
  __syncthreads();   // every wave is done with K buffer 0 before iteration 0 refills it
  int it = 0;
  for (int t0 = 0; t0 < t_end; t0 += kPfTok, ++it) {
    const uint32_t wd0 = qvalid ? wn0 : 0u, wd1 = qvalid ? wn1 : 0u;
    gload(t0 + 2 * kPfTok, t0 + kPfTok);   // past the end: clamped, never used
    gload_words(t0 + kPfTok);
    f32x16_t n0, n1;
    logits((it + 1) & 1, n0, n1);
    const f32x16_t c0 = s0, c1 = s1;
    // Raw logits of the selected tokens, -inf elsewhere: the token's bitmask bit,
    // sign-extended into a 32-bit lane mask, picks between the logit and -inf.  The
    // running max is kept raw (m) and scaled (msc); the scale goes into the exponent's FMA.
    const uint32_t w0 = wd0 >> (4 * hi), w1 = wd1 >> (4 * hi);
    float z[32], mt = neg_inf();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = 8 * (r >> 2) + (r & 3);
      const uint32_t k0 = (uint32_t)((int)(w0 << (31 - tt)) >> 31);
      const uint32_t k1 = (uint32_t)((int)(w1 << (31 - tt)) >> 31);
      z[r] = __uint_as_float((__float_as_uint(c0[r]) & k0) | (0xff800000u & ~k0));
      z[16 + r] = __uint_as_float((__float_as_uint(c1[r]) & k1) | (0xff800000u & ~k1));
    }
    {
      float ma = neg_inf(), mb = neg_inf();
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        ma = max3_f32(ma, z[r], z[16 + r]);
        mb = max3_f32(mb, z[r + 1], z[17 + r]);
      }
      mt = fmaxf(ma, mb);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // The reference max moves only when this tile's max passes it by more than 8 in the
    // base-2 exponent: below that the probabilities stay under 2^8, which the float32 sums
    // and the bf16 rounding of P hold as well as values under 1 (softmax does not depend
    // on the shift), and the accumulators keep their scale (alpha is exactly 1).
    const bool move = (m == neg_inf()) || (mt * scale_log2 > msc + 8.f);
    const float mn = move ? fmaxf(m, mt) : m;
    const float ms = (mn == neg_inf()) ? 0.f : mn * scale_log2;
    // nothing accumulated while m is -inf; an unchanged max rescales by exactly 1
    const float alpha = (m == neg_inf()) ? 0.f : fast_exp2(msc - ms);
    float pr[32], ps = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      pr[r] = fast_exp2(fmaf(z[r], scale_log2, -ms));   // exp2(-inf) = 0
      ps += pr[r];
    }
    ps += __shfl_xor(ps, 32);
    l = l * alpha + ps;
    m = mn;
    msc = ms;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    bf16x8_t pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[ks][e] = (__bf16)pr[8 * ks + e];
    const bf16_t* Vc = Vt[it & 1];
    bf16x8_t va[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bf16_t* vrow = &Vc[((j >> 2) * 32 + ql) * kPfVS + 16 * (j & 3)];
      const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(vrow + 4 * hi);
      const bf16x4_t hi4 = *reinterpret_cast<const bf16x4_t*>(vrow + 8 + 4 * hi);
      va[j] = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      o[j >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j], pb[j & 3], o[j >> 2], 0, 0, 0);
    // V^T operands read two ahead of their products (the scheduler otherwise puts each
    // read right before its MFMA and waits on it)
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int j = 0; j < 14; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    // the buffers refilled here were last read before the previous barrier
    stage(it & 1, (it + 1) & 1);
    __syncthreads();
    s0 = n0;
    s1 = n1;
  }
  if (qvalid) {
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    float* orow = out + (((long long)b * Hq + h) * Lq + i0 + ql) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 v4;
        v4.x = o[db][4 * r4] * inv;
        v4.y = o[db][4 * r4 + 1] * inv;
        v4.z = o[db][4 * r4 + 2] * inv;
        v4.w = o[db][4 * r4 + 3] * inv;
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * r4 + 4 * hi) = v4;
      }
  }
}

}  // namespace

// One workgroup per (b, KV head, 64 query rows), 512 threads.
hipError_t launch_prefill_mfma(hipStream_t s, const void* q, const void* k, const void* v,
                               const uint32_t* bitmask, float* out, int B, int Hq, int Hkv,
                               int Lq, int L, int L_cap, int q_pos0, float scale) {
  const long long blocks = (long long)B * Hkv * ((Lq + 63) / 64);
  hipLaunchKernelGGL(attn_prefill_mfma_kernel, dim3((unsigned)blocks), dim3(2 * kPfThreads), 0, s,
                     (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, bitmask, out, Hq, Hkv,
                     Lq, L, L_cap, q_pos0, scale * 1.4426950408889634f);
  return hipGetLastError();
}

}  // namespace butler
