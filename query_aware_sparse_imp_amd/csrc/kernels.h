// Host-side launchers of the libbutler kernels.  Each returns a hipError_t
// from the launch; arguments are validated by the C ABI layer (api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace butler {

// Head counts: in the scoring, selection and attention launchers "Hkv" is the number of
// selection heads per batch entry (Hq/Hkv query heads share one selected set) and kvdiv
// consecutive selection heads read one physical KV head (cache row = selection row /
// kvdiv).  kvdiv = 1: one selection per KV head.

// ---- key projection -------------------------------------------------------
hipError_t launch_project_keys(hipStream_t s, int dtype, const void* k, const void* w,
                               void* kimp, int B, int Hkv, int L_cap, int D, int dp,
                               int pos0, int n_new);

// ---- producer -------------------------------------------------------------
size_t produce_workspace(int M, int E, int F, int N2);
hipError_t launch_produce(hipStream_t s, const void* h, const void* w1, const void* w2,
                          void* q_imp, int B, int Lq, int E, int F, int Hq, int G, int dp,
                          float eps, void* ws);

// ---- scoring --------------------------------------------------------------
hipError_t launch_project_score(hipStream_t s, int dtype, const void* q_imp,
                                const void* k_cache, const void* w_k, void* kimp,
                                float* scores, int B, int Hq, int Hkv, int G, int slot, int L,
                                int L_cap, int D, int dp, uint32_t* hist, const int32_t* keep,
                                int kvdiv, int t_begin);
// Raw scores of tokens [t_begin, t_end) of single decode rows of length L (row stride L).
hipError_t launch_score_tokens(hipStream_t s, int dtype, const void* q_imp, const void* kimp,
                               float* scores, int B, int Hq, int Hkv, int G, int slot, int L,
                               int L_cap, int dp, uint32_t* hist, const int32_t* keep,
                               int kvdiv, int t_begin, int t_end);
hipError_t launch_score_raw(hipStream_t s, int dtype, const void* q_imp, const void* kimp,
                            float* scores, int B, int Hq, int Hkv, int G, int slot, int Lq,
                            int L, int L_cap, int dp, int q_pos0, int causal, uint32_t* hist,
                            const int32_t* keep, int kvdiv);
size_t softvote_workspace(int B, int Hq, int Hkv, int L);
hipError_t launch_score_softvote(hipStream_t s, int dtype, const void* q, const void* k,
                                 float* scores, int B, int Hq, int Hkv, int L, int L_cap,
                                 int D, float scale, void* ws, uint32_t* hist,
                                 const int32_t* keep, int kvdiv);

// ---- selection ------------------------------------------------------------
size_t select_workspace(int rows, int L, int Lq, int causal);
// The leading part of a chunked-selection workspace that carries state from one call to
// the next; it depends only on the rows.
size_t select_state_bytes(int rows);
hipError_t launch_select(hipStream_t s, const float* scores, int num, int den, int n_sink,
                         int n_window, int fo, int32_t* idx, uint32_t* bitmask, int32_t* count,
                         int B, int Hkv, int Lq, int L, int cap, int q_pos0, int causal,
                         uint32_t* hist, const int32_t* keep, void* ws);
// Calls with several query rows per (b, head) and rows of at most 8192 tokens: one wave
// per row (no scorer histogram, no selection-cache flags).
bool select_rows_fits(int Lq, int L);
hipError_t launch_select_rows(hipStream_t s, const float* scores, int num, int den, int n_sink,
                              int n_window, int fo, int32_t* idx, uint32_t* bitmask,
                              int32_t* count, int B, int Hs, int Lq, int L, int cap, int q_pos0,
                              int causal);

// ---- attention ------------------------------------------------------------
size_t attn_workspace(int dtype, int B, int Hq, int Hkv, int D, int Lq, int L, int cap);
hipError_t launch_attn_idx(hipStream_t s, int dtype, const void* q, const void* k,
                           const void* v, const int32_t* idx, const int32_t* count,
                           float* out, int B, int Hq, int Hkv, int D, int Lq, int L_cap,
                           int cap, float scale, void* ws, int kvdiv);
hipError_t launch_attn_bitmask(hipStream_t s, int dtype, const void* q, const void* k,
                               const void* v, const uint32_t* bitmask, float* out, int B,
                               int Hq, int Hkv, int D, int Lq, int L, int L_cap, int q_pos0,
                               float scale, void* ws, int kvdiv);

// bf16, D = 128, 4 query heads per KV head, Lq >= 32, one selection set per KV head
hipError_t launch_prefill_mfma(hipStream_t s, const void* q, const void* k, const void* v,
                               const uint32_t* bitmask, float* out, int B, int Hq, int Hkv,
                               int Lq, int L, int L_cap, int q_pos0, float scale);
hipError_t launch_attn_merge(hipStream_t s, const float* part, float* out, long long rows, int Hq,
                             int Hkv, int Lq, int D, int nsplit);
bool select_attend_fusable(int dtype, int D, int Hq, int Hkv, int L);
size_t select_attend_workspace(int rows, int Hq, int Hkv, int L);
hipError_t launch_select_attend(hipStream_t s, const float* scores, int num, int den,
                                int n_sink, int n_window, int fo, int32_t* idx, int32_t* count, int B,
                                int Hq, int Hkv, int L, int cap, uint32_t* hist, const void* q,
                                const void* k, const void* v, float* out, int L_cap,
                                float scale, void* ws, int kvdiv);
// Arguments of butler_select_attend, shared with its allocation-free variant.
struct SelectAttendArgs {
  int dtype;
  const float* scores;
  uint32_t* radix_hist;
  int budget_num, budget_den, n_sink, n_window, budget_excludes_forced;
  int32_t* idx;
  int32_t* count;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  float* out;
  int B, Hq, Hkv, sel_group, D, L, L_cap, cap;
  float softmax_scale;
};
struct SelectAttendPlan {
  int fo, Hs, kvdiv, rows;
  bool fused;
  size_t sel_ws;   // unfused: where the attention's part of the workspace starts
  size_t need;     // workspace bytes
};
// Size checks (no pointer is looked at) and the workspace the call needs; a butler_status.
int select_attend_plan(const SelectAttendArgs& a, SelectAttendPlan* plan);
int select_attend_check_pointers(const SelectAttendArgs& a);
hipError_t select_attend_launch(hipStream_t s, const SelectAttendArgs& a,
                                const SelectAttendPlan& plan, void* ws);
// The status of a finished launch sequence (BUTLER_DEBUG_SYNC=1 also synchronises).
int finish_call(hipStream_t s, hipError_t e);

hipError_t launch_selection_cache(hipStream_t s, int dtype, const void* q, void* q_ref,
                                  int32_t* keep, int B, int Hq, int Hkv, int D, float threshold);

hipError_t launch_expand_neighbors(hipStream_t s, const int32_t* idx, const int32_t* count,
                                   int32_t* idx_out, int32_t* count_out, int rows, int L,
                                   int cap_in, int cap_out, int width, int n_window);
int expand_max_len();

// ---- selected-row fetch ------------------------------------------------------
long long fetch_rows_blocks(long long rows, int cap, int row_bytes);
hipError_t launch_fetch_rows(hipStream_t s, const int32_t* idx, const int32_t* count,
                             const void* k, const void* v, void* k_sel, void* v_sel, int rows,
                             int kvdiv, int row_bytes, int L_cap, int cap);

}  // namespace butler
