// C ABI of libbutler (declared in include/butler.h): host-side argument checks, the
// two-phase workspace query and the kernel launches.  Every check runs before anything
// is enqueued, and none of them touches the HIP runtime, so argument errors are
// reported identically with or without a GPU.
#include <stdint.h>
#include <stdlib.h>

#include "../../include/butler.h"
#include "kernels.h"

using namespace butler;

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int from_hip(hipError_t e) { return e == hipSuccess ? BUTLER_OK : BUTLER_ERR_HIP; }

inline bool debug_sync() {
  static const bool on = [] {
    const char* v = getenv("BUTLER_DEBUG_SYNC");
    return v && v[0] == '1';
  }();
  return on;
}

inline int finish(hipStream_t s, hipError_t e) {
  if (e != hipSuccess) return BUTLER_ERR_HIP;
  if (debug_sync() && hipStreamSynchronize(s) != hipSuccess) return BUTLER_ERR_HIP;
  return BUTLER_OK;
}

// Two-phase workspace protocol.  workspace == NULL with ws_bytes != NULL is always a
// size query: *ws_bytes = need, nothing is enqueued.  workspace == NULL with
// ws_bytes == NULL is a call without workspace, allowed when need == 0.  Returns 1 when
// the call must return *rc now, 0 when it should proceed.
inline int workspace_phase(void* ws, size_t* ws_bytes, size_t need, int* rc) {
  if (ws == nullptr) {
    if (ws_bytes != nullptr) { *ws_bytes = need; *rc = BUTLER_OK; return 1; }
    if (need == 0) return 0;
    *rc = BUTLER_ERR_WORKSPACE;
    return 1;
  }
  if (ws_bytes == nullptr || *ws_bytes < need) { *rc = BUTLER_ERR_WORKSPACE; return 1; }
  if (!aligned16(ws)) { *rc = BUTLER_ERR_INVALID_ARG; return 1; }
  return 0;
}

inline bool valid_dtype(int d) { return d == BUTLER_F32 || d == BUTLER_BF16; }
inline bool pow2_group(int R) { return R == 1 || R == 2 || R == 4 || R == 8; }

// The address the GPU reads p at: p itself for device memory, the mapped address for
// pinned host memory.  False for memory HIP does not know (pageable host memory), which
// no kernel may touch.  The only validation step that calls the HIP runtime.
inline bool gpu_view(const void* p, const void** out, bool allow_host) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();   // the failed query must not surface as a launch error
    return false;
  }
  if (a.type == hipMemoryTypeDevice) { *out = p; return true; }
  if (allow_host && a.type == hipMemoryTypeHost && a.devicePointer) {
    *out = a.devicePointer;
    return true;
  }
  return false;
}

// Query heads per selected set: 0 is the KV head's whole group (Hq/Hkv), otherwise a
// divisor of it.  Gives the selection heads per batch entry (Hs) and how many of them
// share one KV head (kvdiv); false when sel_group is not such a divisor.
inline bool sel_heads(int Hq, int Hkv, int sel_group, int* Hs, int* kvdiv) {
  const int R = Hq / Hkv;
  const int gs = sel_group == 0 ? R : sel_group;
  if (gs <= 0 || R % gs) return false;
  *Hs = Hq / gs;
  *kvdiv = R / gs;
  return true;
}

}  // namespace

namespace butler {

// butler_select_attend, split so that its allocation-free variant (scratch.hip) runs the
// same checks and launches on another buffer.
int select_attend_plan(const SelectAttendArgs& a, SelectAttendPlan* plan) {
  if (!valid_dtype(a.dtype)) return BUTLER_ERR_UNSUPPORTED;
  if (a.B <= 0 || a.Hq <= 0 || a.Hkv <= 0 || a.L <= 0 || a.L_cap < a.L)
    return BUTLER_ERR_INVALID_ARG;
  if (a.budget_num < 0 || a.budget_den <= 0 || a.n_sink < 0 || a.n_window < 0)
    return BUTLER_ERR_INVALID_ARG;
  plan->fo = a.budget_excludes_forced ? 1 : 0;
  if (plan->fo && a.radix_hist) return BUTLER_ERR_INVALID_ARG;   // see butler_select_topk
  if (a.Hq % a.Hkv) return BUTLER_ERR_INVALID_ARG;
  if (!pow2_group(a.Hq / a.Hkv) || !(a.D == 64 || a.D == 128)) return BUTLER_ERR_UNSUPPORTED;
  if (!sel_heads(a.Hq, a.Hkv, a.sel_group, &plan->Hs, &plan->kvdiv)) return BUTLER_ERR_INVALID_ARG;
  if (!(a.softmax_scale > 0.f)) return BUTLER_ERR_INVALID_ARG;
  const long long rows = (long long)a.B * plan->Hs;
  if (rows > 0x7fffffffLL || a.L > 8388608) return BUTLER_ERR_UNSUPPORTED;
  {
    const long long x = (long long)a.L * a.budget_num / a.budget_den;
    long long need_cap = x + a.n_sink + a.n_window;
    if (need_cap > a.L) need_cap = a.L;
    if (a.cap < need_cap) return BUTLER_ERR_INVALID_ARG;
  }
  if (rows * ((a.cap + 255) / 256) > 0x7fffffffLL) return BUTLER_ERR_UNSUPPORTED;
  plan->rows = (int)rows;
  plan->fused = select_attend_fusable(a.dtype, a.D, a.Hq, plan->Hs, a.L);
  // unfused: the selection's workspace, then the attention's.  The selection part is at
  // least the state region, so a buffer that also serves fused calls (longer rows) keeps
  // that state when a short row takes this path.
  size_t sel_ws = select_workspace(plan->rows, a.L, 1, 0);
  if (sel_ws < select_state_bytes(plan->rows)) sel_ws = select_state_bytes(plan->rows);
  plan->sel_ws = (sel_ws + 255) / 256 * 256;
  plan->need = plan->fused
                   ? select_attend_workspace(plan->rows, a.Hq, plan->Hs, a.L)
                   : plan->sel_ws + attn_workspace(a.dtype, a.B, a.Hq, plan->Hs, a.D, 1, a.L, a.cap);
  return BUTLER_OK;
}

int select_attend_check_pointers(const SelectAttendArgs& a) {
  if (!a.scores || !a.idx || !a.count || !a.q || !a.k_cache || !a.v_cache || !a.out)
    return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(a.scores) || !aligned16(a.q) || !aligned16(a.k_cache) || !aligned16(a.v_cache) ||
      !aligned16(a.out))
    return BUTLER_ERR_INVALID_ARG;
  if (a.radix_hist && !aligned16(a.radix_hist)) return BUTLER_ERR_INVALID_ARG;
  return BUTLER_OK;
}

hipError_t select_attend_launch(hipStream_t s, const SelectAttendArgs& a,
                                const SelectAttendPlan& plan, void* ws) {
  if (plan.fused)
    return launch_select_attend(s, a.scores, a.budget_num, a.budget_den, a.n_sink, a.n_window,
                                plan.fo, a.idx, a.count, a.B, a.Hq, plan.Hs, a.L, a.cap,
                                a.radix_hist, a.q, a.k_cache, a.v_cache, a.out, a.L_cap,
                                a.softmax_scale, ws, plan.kvdiv);
  hipError_t e = launch_select(s, a.scores, a.budget_num, a.budget_den, a.n_sink, a.n_window,
                               plan.fo, a.idx, nullptr, a.count, a.B, plan.Hs, 1, a.L, a.cap, 0,
                               0, a.radix_hist, nullptr, ws);
  if (e != hipSuccess) return e;
  return launch_attn_idx(s, a.dtype, a.q, a.k_cache, a.v_cache, a.idx, a.count, a.out, a.B,
                         a.Hq, plan.Hs, a.D, 1, a.L_cap, a.cap, a.softmax_scale,
                         (char*)ws + plan.sel_ws, plan.kvdiv);
}

int finish_call(hipStream_t s, hipError_t e) { return finish(s, e); }

}  // namespace butler

extern "C" {

const char* butler_status_string(int status) {
  switch (status) {
    case BUTLER_OK: return "BUTLER_OK";
    case BUTLER_ERR_INVALID_ARG: return "BUTLER_ERR_INVALID_ARG";
    case BUTLER_ERR_UNSUPPORTED: return "BUTLER_ERR_UNSUPPORTED";
    case BUTLER_ERR_WORKSPACE: return "BUTLER_ERR_WORKSPACE";
    case BUTLER_ERR_HIP: return "BUTLER_ERR_HIP";
    default: return "BUTLER_ERR_UNKNOWN";
  }
}

int butler_abi_version(void) { return 8; }

int butler_project_keys(void* stream, int dtype, const void* k_cache, const void* w_k,
                        void* kimp, int B, int Hkv, int L_cap, int D, int dprime, int pos0,
                        int n_new) {
  if (!valid_dtype(dtype)) return BUTLER_ERR_UNSUPPORTED;
  if (!k_cache || !w_k || !kimp) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(w_k) || !aligned16(kimp)) return BUTLER_ERR_INVALID_ARG;
  if (B <= 0 || Hkv <= 0 || L_cap <= 0 || n_new <= 0 || pos0 < 0) return BUTLER_ERR_INVALID_ARG;
  if ((long long)pos0 + n_new > L_cap) return BUTLER_ERR_INVALID_ARG;
  if (!(D == 64 || D == 128) || !(dprime == 16 || dprime == 32)) return BUTLER_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  return finish(s, launch_project_keys(s, dtype, k_cache, w_k, kimp, B, Hkv, L_cap, D, dprime,
                                       pos0, n_new));
}

int butler_produce_queries(void* stream, int dtype, const void* h, const void* w1,
                           const void* w2, void* q_imp, int B, int Lq, int E, int F, int Hq,
                           int G, int dprime, float ln_eps, void* workspace,
                           size_t* ws_bytes) {
  if (dtype != BUTLER_BF16) return BUTLER_ERR_UNSUPPORTED;
  if (B <= 0 || Lq <= 0 || E <= 0 || F <= 0 || Hq <= 0 || G <= 0 || dprime <= 0)
    return BUTLER_ERR_INVALID_ARG;
  if (!(ln_eps > 0.f)) return BUTLER_ERR_INVALID_ARG;
  const long long N2 = (long long)Hq * G * dprime;
  if (E % 64 || F % 64 || N2 % 64 || N2 > (1 << 24) || dprime % 8) return BUTLER_ERR_UNSUPPORTED;
  if (E > 8192) return BUTLER_ERR_UNSUPPORTED;   // LN holds a row in registers
  if ((long long)B * Lq > (1 << 24)) return BUTLER_ERR_UNSUPPORTED;
  int rc;
  if (workspace_phase(workspace, ws_bytes, produce_workspace(B * Lq, E, F, (int)N2), &rc))
    return rc;
  if (!h || !w1 || !w2 || !q_imp) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w1) || !aligned16(w2) || !aligned16(q_imp))
    return BUTLER_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  return finish(s, launch_produce(s, h, w1, w2, q_imp, B, Lq, E, F, Hq, G, dprime, ln_eps,
                                  workspace));
}

int butler_score(void* stream, int mode, int dtype, const void* q, const void* keys,
                 float* scores, uint32_t* radix_hist, const int32_t* keep, int B, int Hq,
                 int Hkv, int sel_group, int G, int slot,
                 int Lq, int L,
                 int L_cap, int dk, int q_pos0, int causal, float softmax_scale,
                 void* workspace, size_t* ws_bytes) {
  if (!valid_dtype(dtype)) return BUTLER_ERR_UNSUPPORTED;
  if (mode != BUTLER_SCORE_RAW && mode != BUTLER_SCORE_SOFTVOTE) return BUTLER_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || L <= 0 || L_cap < L || q_pos0 < 0)
    return BUTLER_ERR_INVALID_ARG;
  if (Hq % Hkv) return BUTLER_ERR_INVALID_ARG;
  if (!pow2_group(Hq / Hkv)) return BUTLER_ERR_UNSUPPORTED;
  int Hs, kvdiv;
  if (!sel_heads(Hq, Hkv, sel_group, &Hs, &kvdiv)) return BUTLER_ERR_INVALID_ARG;
  if ((long long)B * Hs * Lq > 65535LL * 65535LL) return BUTLER_ERR_UNSUPPORTED;
  size_t need = 0;
  if (mode == BUTLER_SCORE_RAW) {
    if (G <= 0 || slot < 0 || slot >= G) return BUTLER_ERR_INVALID_ARG;
    if (!(dk == 16 || dk == 32)) return BUTLER_ERR_UNSUPPORTED;
    if (Lq > 65535 || (long long)B * Hs > 65535) return BUTLER_ERR_UNSUPPORTED;
  } else {
    if (!(dk == 64 || dk == 128)) return BUTLER_ERR_UNSUPPORTED;
    if (Lq != 1 || causal) return BUTLER_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.f)) return BUTLER_ERR_INVALID_ARG;
    need = softvote_workspace(B, Hq, Hs, L);
  }
  int rc;
  if (workspace_phase(workspace, ws_bytes, need, &rc)) return rc;
  if (!q || !keys || !scores) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(keys) || !aligned16(scores)) return BUTLER_ERR_INVALID_ARG;
  if (radix_hist && !aligned16(radix_hist)) return BUTLER_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  // the first-digit histogram and the selection-cache flags are decode-row hand-offs;
  // multi-row calls ignore them
  uint32_t* hist = (Lq > 1) ? nullptr : radix_hist;
  const int32_t* kp = (Lq > 1) ? nullptr : keep;
  if (mode == BUTLER_SCORE_RAW)
    return finish(s, launch_score_raw(s, dtype, q, keys, scores, B, Hq, Hs, G, slot, Lq, L,
                                      L_cap, dk, q_pos0, causal, hist, kp, kvdiv));
  return finish(s, launch_score_softvote(s, dtype, q, keys, scores, B, Hq, Hs, L, L_cap, dk,
                                         softmax_scale, workspace, hist, kp, kvdiv));
}

int butler_project_and_score(void* stream, int dtype, const void* q_imp, const void* k_cache,
                             const void* w_k, void* kimp, float* scores, uint32_t* radix_hist,
                             const int32_t* keep, int B, int Hq, int Hkv, int sel_group, int G,
                             int slot, int L, int L_cap, int D, int dprime) {
  if (!valid_dtype(dtype)) return BUTLER_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || L_cap < L) return BUTLER_ERR_INVALID_ARG;
  if (Hq % Hkv || G <= 0 || slot < 0 || slot >= G) return BUTLER_ERR_INVALID_ARG;
  if (!pow2_group(Hq / Hkv)) return BUTLER_ERR_UNSUPPORTED;
  int Hs, kvdiv;
  if (!sel_heads(Hq, Hkv, sel_group, &Hs, &kvdiv)) return BUTLER_ERR_INVALID_ARG;
  if (!(D == 64 || D == 128) || !(dprime == 16 || dprime == 32)) return BUTLER_ERR_UNSUPPORTED;
  if ((long long)B * Hs > 65535) return BUTLER_ERR_UNSUPPORTED;
  if (!q_imp || !k_cache || !w_k || !kimp || !scores) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(q_imp) || !aligned16(k_cache) || !aligned16(w_k) || !aligned16(kimp) ||
      !aligned16(scores))
    return BUTLER_ERR_INVALID_ARG;
  if (radix_hist && !aligned16(radix_hist)) return BUTLER_ERR_INVALID_ARG;
  if (kimp == k_cache || kimp == w_k) return BUTLER_ERR_INVALID_ARG;   // no aliasing
  hipStream_t s = (hipStream_t)stream;
  return finish(s, launch_project_score(s, dtype, q_imp, k_cache, w_k, kimp, scores, B, Hq, Hs,
                                        G, slot, L, L_cap, D, dprime, radix_hist, keep, kvdiv,
                                        0));
}

int butler_score_tokens(void* stream, int dtype, const void* q_imp, void* kimp,
                        const void* k_cache, const void* w_k, float* scores,
                        uint32_t* radix_hist, const int32_t* keep, int B, int Hq, int Hkv,
                        int sel_group, int G, int slot, int L, int L_cap, int D, int dprime,
                        int t_begin, int t_end) {
  if (!valid_dtype(dtype)) return BUTLER_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || L_cap < L) return BUTLER_ERR_INVALID_ARG;
  if (t_begin < 0 || t_end <= t_begin || t_end > L) return BUTLER_ERR_INVALID_ARG;
  if (Hq % Hkv || G <= 0 || slot < 0 || slot >= G) return BUTLER_ERR_INVALID_ARG;
  if (!pow2_group(Hq / Hkv)) return BUTLER_ERR_UNSUPPORTED;
  int Hs, kvdiv;
  if (!sel_heads(Hq, Hkv, sel_group, &Hs, &kvdiv)) return BUTLER_ERR_INVALID_ARG;
  if (!(dprime == 16 || dprime == 32)) return BUTLER_ERR_UNSUPPORTED;
  if ((long long)B * Hs > 65535) return BUTLER_ERR_UNSUPPORTED;
  const bool project = k_cache != nullptr || w_k != nullptr;
  if (project) {
    if (!k_cache || !w_k || t_end != L) return BUTLER_ERR_INVALID_ARG;
    if (!(D == 64 || D == 128)) return BUTLER_ERR_UNSUPPORTED;
    if (!aligned16(k_cache) || !aligned16(w_k)) return BUTLER_ERR_INVALID_ARG;
    if (kimp == k_cache || kimp == w_k) return BUTLER_ERR_INVALID_ARG;   // no aliasing
  }
  if (!q_imp || !kimp || !scores) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(q_imp) || !aligned16(kimp) || !aligned16(scores)) return BUTLER_ERR_INVALID_ARG;
  if (radix_hist && !aligned16(radix_hist)) return BUTLER_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (project)
    return finish(s, launch_project_score(s, dtype, q_imp, k_cache, w_k, kimp, scores, B,
                                          Hq, Hs, G, slot, L, L_cap, D, dprime, radix_hist, keep,
                                          kvdiv, t_begin));
  return finish(s, launch_score_tokens(s, dtype, q_imp, kimp, scores, B, Hq, Hs, G, slot, L,
                                       L_cap, dprime, radix_hist, keep, kvdiv, t_begin, t_end));
}

int butler_select_topk(void* stream, const float* scores, uint32_t* radix_hist,
                       const int32_t* keep, int budget_num, int budget_den, int n_sink,
                       int n_window, int budget_excludes_forced, int32_t* idx,
                       uint32_t* bitmask, int32_t* count, int B, int Hs, int Lq, int L,
                       int cap, int q_pos0, int causal, void* workspace, size_t* ws_bytes) {
  if (B <= 0 || Hs <= 0 || Lq <= 0 || L <= 0 || q_pos0 < 0) return BUTLER_ERR_INVALID_ARG;
  if (budget_num < 0 || budget_den <= 0 || n_sink < 0 || n_window < 0)
    return BUTLER_ERR_INVALID_ARG;
  const int fo = budget_excludes_forced ? 1 : 0;
  // the scorer's histogram counts every token's key; the forced tokens then rank below all
  if (fo && radix_hist && Lq == 1) return BUTLER_ERR_INVALID_ARG;
  const long long rows = (long long)B * Hs * Lq;
  if (rows > 0x7fffffffLL) return BUTLER_ERR_UNSUPPORTED;
  // one workgroup per row holds at most 64K keys; long rows use the chunked decode
  // schedule (one query row per KV head, no causal mask), up to 8M tokens
  if ((causal || Lq > 1) && L > 65536) return BUTLER_ERR_UNSUPPORTED;
  if (L > 8388608) return BUTLER_ERR_UNSUPPORTED;
  if (idx) {
    const long long x = (long long)L * budget_num / budget_den;
    long long need_cap = x + n_sink + n_window;
    if (need_cap > L) need_cap = L;
    if (cap < need_cap) return BUTLER_ERR_INVALID_ARG;
  }
  int rc;
  if (workspace_phase(workspace, ws_bytes, select_workspace((int)rows, L, Lq, causal), &rc)) return rc;
  if (!scores || !count || (!idx && !bitmask)) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(scores)) return BUTLER_ERR_INVALID_ARG;
  if (radix_hist && !aligned16(radix_hist)) return BUTLER_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* hist = (Lq > 1) ? nullptr : radix_hist;   // see butler_score
  const int32_t* kp = (Lq > 1) ? nullptr : keep;
  if (select_rows_fits(Lq, L))
    return finish(s, launch_select_rows(s, scores, budget_num, budget_den, n_sink, n_window, fo,
                                        idx, bitmask, count, B, Hs, Lq, L, cap, q_pos0, causal));
  return finish(s, launch_select(s, scores, budget_num, budget_den, n_sink, n_window, fo, idx,
                                 bitmask, count, B, Hs, Lq, L, cap, q_pos0, causal, hist, kp,
                                 workspace));
}

int butler_sparse_decode_attn(void* stream, int dtype, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* idx, const int32_t* count,
                              const uint32_t* bitmask, float* out, int B, int Hq, int Hkv,
                              int sel_group, int D, int Lq, int L, int L_cap, int cap,
                              int q_pos0, float softmax_scale, void* workspace,
                              size_t* ws_bytes) {
  if (!valid_dtype(dtype)) return BUTLER_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || L <= 0 || L_cap < L || q_pos0 < 0)
    return BUTLER_ERR_INVALID_ARG;
  if (Hq % Hkv) return BUTLER_ERR_INVALID_ARG;
  if (!pow2_group(Hq / Hkv) || !(D == 64 || D == 128)) return BUTLER_ERR_UNSUPPORTED;
  int Hs, kvdiv;
  if (!sel_heads(Hq, Hkv, sel_group, &Hs, &kvdiv)) return BUTLER_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f)) return BUTLER_ERR_INVALID_ARG;
  const bool use_idx = idx != nullptr;
  if (!use_idx && !bitmask) return BUTLER_ERR_INVALID_ARG;
  const long long rows = (long long)B * Hs * Lq;
  if (use_idx) {
    if (cap <= 0 || !count) return BUTLER_ERR_INVALID_ARG;
    if (rows * ((cap + 255) / 256) > 0x7fffffffLL) return BUTLER_ERR_UNSUPPORTED;
  } else {
    if (L > 16384 || rows > 0x7fffffffLL) return BUTLER_ERR_UNSUPPORTED;
  }
  const size_t need = use_idx ? attn_workspace(dtype, B, Hq, Hs, D, Lq, L, cap) : 0;
  int rc;
  if (workspace_phase(workspace, ws_bytes, need, &rc)) return rc;
  if (!q || !k_cache || !v_cache || !out) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return BUTLER_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (use_idx)
    return finish(s, launch_attn_idx(s, dtype, q, k_cache, v_cache, idx, count, out, B, Hq, Hs,
                                     D, Lq, L_cap, cap, softmax_scale, workspace, kvdiv));
  return finish(s, launch_attn_bitmask(s, dtype, q, k_cache, v_cache, bitmask, out, B, Hq, Hs,
                                       D, Lq, L, L_cap, q_pos0, softmax_scale, workspace, kvdiv));
}

int butler_select_attend(void* stream, int dtype, const float* scores, uint32_t* radix_hist,
                         int budget_num, int budget_den, int n_sink, int n_window,
                         int budget_excludes_forced, int32_t* idx, int32_t* count, const void* q,
                         const void* k_cache, const void* v_cache, float* out, int B, int Hq,
                         int Hkv, int sel_group, int D, int L, int L_cap, int cap,
                         float softmax_scale, void* workspace, size_t* ws_bytes) {
  SelectAttendArgs a{dtype, scores, radix_hist, budget_num, budget_den, n_sink, n_window,
                     budget_excludes_forced, idx, count, q, k_cache, v_cache, out, B, Hq, Hkv,
                     sel_group, D, L, L_cap, cap, softmax_scale};
  SelectAttendPlan plan;
  int rc = select_attend_plan(a, &plan);
  if (rc != BUTLER_OK) return rc;
  if (workspace_phase(workspace, ws_bytes, plan.need, &rc)) return rc;
  rc = select_attend_check_pointers(a);
  if (rc != BUTLER_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  return finish(s, select_attend_launch(s, a, plan, workspace));
}

int butler_selection_cache(void* stream, int dtype, const void* q, void* q_ref, int32_t* keep,
                           int B, int Hq, int Hkv, int sel_group, int D, float threshold) {
  if (!valid_dtype(dtype)) return BUTLER_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return BUTLER_ERR_INVALID_ARG;
  if (!pow2_group(Hq / Hkv) || !(D == 64 || D == 128)) return BUTLER_ERR_UNSUPPORTED;
  int Hs, kvdiv;
  if (!sel_heads(Hq, Hkv, sel_group, &Hs, &kvdiv)) return BUTLER_ERR_INVALID_ARG;
  if ((long long)B * Hs > 0x7fffffffLL) return BUTLER_ERR_UNSUPPORTED;
  if (threshold != threshold) return BUTLER_ERR_INVALID_ARG;   // NaN
  if (!q || !q_ref || !keep) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(q_ref) || !aligned16(keep)) return BUTLER_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  // the cache compares the query heads of one selection head: its group of Hq / Hs
  return finish(s, launch_selection_cache(s, dtype, q, q_ref, keep, B, Hq, Hs, D, threshold));
}

int butler_expand_neighbors(void* stream, const int32_t* idx, const int32_t* count,
                            int32_t* idx_out, int32_t* count_out, int B, int Hs, int L,
                            int cap_in, int cap_out, int width, int n_window) {
  if (B <= 0 || Hs <= 0 || L <= 0 || cap_in <= 0 || cap_out <= 0) return BUTLER_ERR_INVALID_ARG;
  if (width < 0 || width > 31 || n_window < 0) return BUTLER_ERR_INVALID_ARG;
  if (L > expand_max_len() || (long long)B * Hs > 0x7fffffffLL) return BUTLER_ERR_UNSUPPORTED;
  if (cap_out < L && (long long)cap_out < (long long)cap_in * (2 * width + 1) + n_window)
    return BUTLER_ERR_INVALID_ARG;
  if (!idx || !count || !idx_out || !count_out) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(idx) || !aligned16(count) || !aligned16(idx_out) || !aligned16(count_out))
    return BUTLER_ERR_INVALID_ARG;
  if (idx == idx_out || count == count_out) return BUTLER_ERR_INVALID_ARG;   // no aliasing
  hipStream_t s = (hipStream_t)stream;
  return finish(s, launch_expand_neighbors(s, idx, count, idx_out, count_out, B * Hs, L, cap_in,
                                           cap_out, width, n_window));
}

int butler_fetch_rows(void* stream, int dtype, const int32_t* idx, const int32_t* count,
                      const void* k_cache, const void* v_cache, void* k_sel, void* v_sel, int B,
                      int Hq, int Hkv, int sel_group, int D, int L_cap, int cap) {
  if (!valid_dtype(dtype)) return BUTLER_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || L_cap <= 0 || cap <= 0 || Hq % Hkv)
    return BUTLER_ERR_INVALID_ARG;
  if (!pow2_group(Hq / Hkv) || !(D == 64 || D == 128)) return BUTLER_ERR_UNSUPPORTED;
  int Hs, kvdiv;
  if (!sel_heads(Hq, Hkv, sel_group, &Hs, &kvdiv)) return BUTLER_ERR_INVALID_ARG;
  const long long rows = (long long)B * Hs;
  const int row_bytes = D * (dtype == BUTLER_BF16 ? 2 : 4);
  if (rows > 0x7fffffffLL || fetch_rows_blocks(rows, cap, row_bytes) > 0x7fffffffLL)
    return BUTLER_ERR_UNSUPPORTED;
  if (!idx || !count || !k_cache || !v_cache || !k_sel || !v_sel) return BUTLER_ERR_INVALID_ARG;
  if (!aligned16(idx) || !aligned16(count) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(k_sel) || !aligned16(v_sel))
    return BUTLER_ERR_INVALID_ARG;
  if (k_sel == v_sel || k_sel == k_cache || v_sel == v_cache) return BUTLER_ERR_INVALID_ARG;
  const void *kd, *vd, *ksd, *vsd, *id, *cd;
  if (!gpu_view(k_cache, &kd, true) || !gpu_view(v_cache, &vd, true)) return BUTLER_ERR_INVALID_ARG;
  if (!gpu_view(k_sel, &ksd, false) || !gpu_view(v_sel, &vsd, false) ||
      !gpu_view(idx, &id, false) || !gpu_view(count, &cd, false))
    return BUTLER_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  return finish(s, launch_fetch_rows(s, idx, count, kd, vd, k_sel, v_sel, (int)rows, kvdiv,
                                     row_bytes, L_cap, cap));
}

}  // extern "C"
