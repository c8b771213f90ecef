"""C ABI checks that need no GPU: the library loads, exports every function that
include/butler.h declares, answers workspace queries, and rejects bad arguments with
the documented status before anything is enqueued (no HIP call is made on these paths).
"""
import ctypes
import os
import subprocess

import pytest

import query_aware_sparse_imp_amd as qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = qa.lib
OK, INV, UNS, WSE = 0, -1, -2, -3
FAKE = 0x10000          # a 16-byte aligned non-null address; never dereferenced here
MIS = 0x10004           # misaligned


def test_every_declared_symbol_is_exported():
    names = qa.declared_symbols()
    assert {"butler_project_keys", "butler_produce_queries", "butler_score",
            "butler_select_topk", "butler_sparse_decode_attn",
            "butler_selection_cache", "butler_expand_neighbors"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", qa.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_status_strings_and_version():
    assert qa.butler_abi_version() == 8
    assert qa.butler_status_string(0) == "BUTLER_OK"
    assert qa.butler_status_string(-3) == "BUTLER_ERR_WORKSPACE"
    assert qa.butler_status_string(123) == "BUTLER_ERR_UNKNOWN"


def test_project_keys_validation():
    f = L.butler_project_keys
    assert f(None, 1, None, FAKE, FAKE, 1, 8, 100, 128, 32, 0, 1) == INV      # null
    assert f(None, 1, MIS, FAKE, FAKE, 1, 8, 100, 128, 32, 0, 1) == INV       # misaligned
    assert f(None, 1, FAKE, FAKE, FAKE, 1, 8, 100, 128, 32, 99, 2) == INV     # past L_cap
    assert f(None, 1, FAKE, FAKE, FAKE, 1, 8, 100, 96, 32, 0, 1) == UNS       # D
    assert f(None, 1, FAKE, FAKE, FAKE, 1, 8, 100, 128, 24, 0, 1) == UNS      # d'
    assert f(None, 7, FAKE, FAKE, FAKE, 1, 8, 100, 128, 32, 0, 1) == UNS      # dtype
    assert f(None, 1, FAKE, FAKE, FAKE, 0, 8, 100, 128, 32, 0, 1) == INV      # B


def _score(mode=0, dtype=1, q=FAKE, keys=FAKE, scores=FAKE, B=1, Hq=32, Hkv=8, sg=0, G=1,
           slot=0, Lq=1, Lk=1000, L_cap=1000, dk=32, q_pos0=0, causal=0, scale=0.1, ws=None,
           n=None):
    return L.butler_score(None, mode, dtype, q, keys, scores, None, None, B, Hq, Hkv, sg, G,
                          slot, Lq, Lk, L_cap, dk, q_pos0, causal, scale, ws, n)


def test_score_validation_and_workspace_query():
    assert _score(Hq=30) == INV                         # Hq % Hkv
    assert _score(Hq=24, Hkv=8) == UNS                  # group of 3
    assert _score(Lk=1001) == INV                       # L > L_cap
    assert _score(slot=1, G=1) == INV
    assert _score(dk=64) == UNS                         # raw d'
    assert _score(mode=1, dk=128, Lq=2) == UNS          # softvote decode only
    n = ctypes.c_size_t(0)
    assert _score(mode=1, dk=128, n=ctypes.byref(n)) == OK
    R, Lk = 4, 1000
    assert n.value >= 8 * R * Lk * 4
    small = ctypes.c_size_t(16)
    assert _score(mode=1, dk=128, ws=FAKE, n=ctypes.byref(small)) == WSE
    assert _score(q=None) == INV
    # sel_group: 0 or a divisor of R = 4
    assert _score(sg=3) == INV and _score(sg=8) == INV and _score(sg=-1) == INV
    # per-query-head softvote: the same logits workspace, Hs = 32 rows of one head each
    n1 = ctypes.c_size_t(0)
    assert _score(mode=1, dk=128, sg=1, n=ctypes.byref(n1)) == OK
    assert n1.value >= 32 * Lk * 4
    assert _score(B=2100, sg=1) == UNS                  # B * Hs > 65535 (raw grid)
    assert _score(B=2100, sg=0, q=None) == INV          # sizes pass, then the null q


def test_select_validation():
    f = L.butler_select_topk

    def call(*, hist=None, num=1, den=2, sink=4, fo=0, idx=FAKE, cap=1000, Lr=1000, Lq=1):
        # stream, scores, radix_hist, keep, num, den, sink, window, excludes_forced, idx,
        # bitmask, count, B, Hkv, Lq, L, cap, q_pos0, causal, ws, ws_bytes
        return f(None, FAKE, hist, None, num, den, sink, 64, fo, idx, None, FAKE, 1, 8, Lq, Lr,
                 cap, 0, 0, None, None)
    assert call(cap=567) == INV                    # cap smaller than min(L, x + sink + window)
    assert call(den=0) == INV
    assert call(sink=-1) == INV                    # negative sink
    assert call(idx=None, cap=0) == INV            # no output
    assert call(hist=FAKE, fo=1) == INV            # the scorer's histogram with forced tokens out


def test_attention_validation_and_workspace_query():
    f = L.butler_sparse_decode_attn
    n = ctypes.c_size_t(0)
    assert f(None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 32, 8, 0, 128, 1, 32768,
             32768, 16452, 0, 0.088, None, ctypes.byref(n)) == OK
    # one (max, sum, acc[D]) partial per (row, split, head): a whole number of splits >= 1
    per_split = 8 * 4 * (128 + 4) * 4
    assert n.value >= per_split and n.value % per_split == 0
    # per query head: 32 rows of one head each, the same bytes per split
    n1 = ctypes.c_size_t(0)
    assert f(None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 32, 8, 1, 128, 1, 32768,
             32768, 16452, 0, 0.088, None, ctypes.byref(n1)) == OK
    assert n1.value >= per_split and n1.value % (32 * (128 + 4) * 4) == 0
    assert f(None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 32, 8, 3, 128, 1, 32768,
             32768, 16452, 0, 0.088, None, ctypes.byref(n1)) == INV         # sel_group 3
    assert f(None, 1, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1, 32, 8, 0, 128, 1, 32768,
             32768, 16452, 0, 0.088, None, None) == INV                     # idx without count
    assert f(None, 1, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1, 32, 8, 0, 128, 4, 20000,
             20000, 0, 0, 0.088, None, None) == UNS                         # bitmask L too long
    assert f(None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 32, 8, 0, 96, 1, 100, 100,
             100, 0, 0.088, None, None) == UNS                              # D
    assert f(None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 32, 8, 0, 128, 1, 100, 100,
             100, 0, -1.0, None, None) == INV                               # scale


def test_produce_validation_and_workspace_query():
    f = L.butler_produce_queries
    n = ctypes.c_size_t(0)
    assert f(None, 1, FAKE, FAKE, FAKE, FAKE, 1, 1, 4096, 1024, 32, 4, 32, 1e-5, None,
             ctypes.byref(n)) == OK
    assert n.value >= 1024 * 2                        # one decode row: the hidden activation
    assert f(None, 1, FAKE, FAKE, FAKE, FAKE, 2, 1024, 4096, 1024, 32, 4, 32, 1e-5, None,
             ctypes.byref(n)) == OK
    assert n.value >= 2048 * (4096 + 1024) * 2        # prefill rows: x_hat and activations
    assert f(None, 0, FAKE, FAKE, FAKE, FAKE, 1, 1, 4096, 1024, 32, 4, 32, 1e-5, None,
             ctypes.byref(n)) == UNS                                        # fp32 producer
    assert f(None, 1, FAKE, FAKE, FAKE, FAKE, 1, 1, 4000, 1024, 32, 4, 32, 1e-5, None,
             ctypes.byref(n)) == UNS                                        # E % 64


def test_selection_cache_validation():
    f = L.butler_selection_cache
    assert f(None, 1, None, FAKE, FAKE, 16, 32, 8, 0, 128, 0.98) == INV      # null q
    assert f(None, 1, FAKE, FAKE, MIS, 16, 32, 8, 0, 128, 0.98) == INV       # misaligned keep
    assert f(None, 1, FAKE, FAKE, FAKE, 16, 30, 8, 0, 128, 0.98) == INV      # Hq % Hkv
    assert f(None, 1, FAKE, FAKE, FAKE, 16, 32, 8, 3, 128, 0.98) == INV      # sel_group 3
    assert f(None, 1, FAKE, FAKE, FAKE, 16, 32, 8, 0, 96, 0.98) == UNS       # D
    assert f(None, 5, FAKE, FAKE, FAKE, 16, 32, 8, 0, 128, 0.98) == UNS      # dtype
    assert f(None, 1, FAKE, FAKE, FAKE, 16, 32, 8, 0, 128, float("nan")) == INV  # threshold



def test_expand_neighbors_validation():
    f = L.butler_expand_neighbors
    A, B2, C, D = FAKE, FAKE + 256, FAKE + 512, FAKE + 768
    # idx, count, idx_out, count_out, B, Hkv, L, cap_in, cap_out, width, n_window
    assert f(None, A, B2, A, D, 1, 8, 4096, 64, 512, 1, 16) == INV        # idx_out aliases idx
    assert f(None, A, B2, C, B2, 1, 8, 4096, 64, 512, 1, 16) == INV       # count_out aliases
    assert f(None, None, B2, C, D, 1, 8, 4096, 64, 512, 1, 16) == INV     # null idx
    assert f(None, MIS, B2, C, D, 1, 8, 4096, 64, 512, 1, 16) == INV      # misaligned
    assert f(None, A, B2, C, D, 1, 8, 4096, 64, 512, 32, 16) == INV       # width > 31
    assert f(None, A, B2, C, D, 1, 8, 4096, 64, 512, -1, 16) == INV       # negative width
    assert f(None, A, B2, C, D, 1, 8, 4096, 64, 100, 1, 16) == INV        # cap_out too small
    assert f(None, A, B2, C, D, 1, 8, (1 << 23) + 1, 64, 1 << 24, 1, 16) == UNS   # L
    assert f(None, A, B2, C, D, 0, 8, 4096, 64, 512, 1, 16) == INV        # B


def test_project_and_score_validation():
    f = L.butler_project_and_score
    P = [FAKE + 256 * i for i in range(5)]      # q_imp, k_cache, w_k, kimp, scores

    def call(*, dtype=1, ptrs=P, hist=None, B=1, Hq=32, Hkv=8, sg=0, G=1, slot=0, Lr=100,
             L_cap=100, D=128, dp=32):
        return f(None, dtype, *ptrs, hist, None, B, Hq, Hkv, sg, G, slot, Lr, L_cap, D, dp)
    assert call(dtype=7) == UNS
    assert call(Lr=101) == INV                                   # L > L_cap
    assert call(slot=1) == INV                                   # slot >= G
    assert call(Hq=30) == INV                                    # Hq % Hkv
    assert call(Hq=24) == UNS                                    # R = 3
    assert call(D=96) == UNS
    assert call(dp=8) == UNS
    assert call(ptrs=[P[0], P[1], P[2], P[1], P[4]]) == INV      # kimp aliases k_cache
    assert call(ptrs=[P[0], MIS, P[2], P[3], P[4]]) == INV       # misaligned
    assert call(ptrs=[P[0], None, P[2], P[3], P[4]]) == INV
    assert call(hist=MIS) == INV
    assert call(B=9000) == UNS                                   # B * Hkv > 65535
    assert call(B=2100, sg=1) == UNS                             # B * Hs > 65535
    assert call(sg=3) == INV and call(sg=16) == INV              # not a divisor of R = 4


def test_select_attend_validation_and_workspace_query():
    f = L.butler_select_attend
    P = [FAKE + 256 * i for i in range(7)]      # scores, idx, count, q, k, v, out

    def call(*, dtype=1, num=1, den=2, ptrs=P, B=1, Hq=32, Hkv=8, sg=0, D=128, Lr=32768,
             L_cap=32768, cap=16452, scale=0.088, ws=FAKE, n=None):
        n = n if n is not None else ctypes.c_size_t(1 << 40)
        return f(None, dtype, ptrs[0], None, num, den, 4, 64, 0, ptrs[1], ptrs[2], ptrs[3],
                 ptrs[4], ptrs[5], ptrs[6], B, Hq, Hkv, sg, D, Lr, L_cap, cap, scale, ws,
                 ctypes.byref(n))
    n = ctypes.c_size_t(0)
    assert call(ws=None, n=n) == OK and n.value > 0                       # size query (fused)
    fused = n.value
    assert call(ws=None, n=n, Lr=3001, L_cap=3001, cap=1568) == OK and n.value > 0   # unfused
    assert fused >= 8 * 32 * 4 * 132 * 4                                  # one partial per chunk
    assert call(cap=16451) == INV                                        # cap too small
    assert call(den=0) == INV
    assert call(Hq=30) == INV
    assert call(D=96) == UNS
    assert call(dtype=3) == UNS
    assert call(scale=0.0) == INV
    assert call(Lr=32769) == INV                                         # L > L_cap
    assert call(ptrs=[P[0], None] + P[2:]) == INV                        # idx required
    assert call(ptrs=[P[0], P[1], P[2], MIS] + P[4:]) == INV             # misaligned q
    assert call(ws=FAKE, n=ctypes.c_size_t(16)) == WSE                   # workspace too small
    n1 = ctypes.c_size_t(0)
    assert call(ws=None, n=n1, sg=1) == OK and n1.value > fused          # 32 selection rows
    assert call(sg=3) == INV


def test_fetch_rows_validation():
    """Size and pointer checks; pointers HIP does not know (here every one of them, GPU or
    not) are rejected before any launch, so pageable host memory never reaches a kernel."""
    f = L.butler_fetch_rows
    P = [FAKE + 256 * i for i in range(6)]      # idx, count, k_cache, v_cache, k_sel, v_sel

    def call(*, dtype=1, ptrs=P, B=1, Hq=32, Hkv=8, sg=0, D=128, L_cap=32768, cap=16452):
        return f(None, dtype, *ptrs, B, Hq, Hkv, sg, D, L_cap, cap)
    assert call(dtype=4) == UNS
    assert call(D=96) == UNS
    assert call(Hq=24) == UNS                                   # R = 3
    assert call(Hq=30) == INV                                   # Hq % Hkv
    assert call(sg=3) == INV                                    # not a divisor of R
    assert call(cap=0) == INV
    assert call(B=0) == INV
    assert call(ptrs=[None] + P[1:]) == INV
    assert call(ptrs=P[:4] + [MIS, P[5]]) == INV                # misaligned k_sel
    assert call(ptrs=P[:4] + [P[4], P[4]]) == INV               # k_sel aliases v_sel
    assert call(ptrs=P[:4] + [P[2], P[5]]) == INV               # k_sel aliases k_cache
    assert call() == INV                                        # memory unknown to HIP
    assert call(sg=1) == INV


def test_select_attend_noalloc_validation_without_a_gpu():
    """The allocation-free variant checks its arguments as butler_select_attend does, and
    refuses a call whose workspace would not fit the library's fixed scratch array, before
    it touches the HIP runtime (so these run without a GPU)."""
    f = L.butler_select_attend_noalloc
    P = [FAKE + 256 * i for i in range(7)]

    def call(*, dtype=1, num=1, den=2, ptrs=P, B=1, Hq=32, Hkv=8, sg=0, D=128, Lr=32768,
             L_cap=32768, cap=16452, scale=0.088):
        return f(None, dtype, ptrs[0], None, num, den, 4, 64, 0, ptrs[1], ptrs[2], ptrs[3],
                 ptrs[4], ptrs[5], ptrs[6], B, Hq, Hkv, sg, D, Lr, L_cap, cap, scale)
    assert call(cap=16451) == INV
    assert call(D=96) == UNS
    assert call(ptrs=[P[0], None] + P[2:]) == INV
    # the workspace butler_select_attend would ask for at this shape exceeds the array
    big_L = 8388608
    n = ctypes.c_size_t(0)
    assert L.butler_select_attend(None, 1, P[0], None, 1, 16, 4, 128, 0, P[1], P[2], P[3], P[4],
                                  P[5], P[6], 2, 32, 8, 0, 128, big_L, big_L, big_L, 0.088,
                                  None, ctypes.byref(n)) == OK
    assert n.value > (64 << 20)
    assert call(B=2, num=1, den=16, Lr=big_L, L_cap=big_L, cap=big_L) == WSE


def test_score_tokens_validation():
    f = L.butler_score_tokens

    def call(*, dtype=1, q=FAKE, kimp=FAKE + 256, k=None, wk=None, scores=FAKE + 512, B=1,
             Hq=32, Hkv=8, sg=0, G=4, slot=1, Lr=1000, L_cap=1000, D=128, dp=32, tb=0, te=999):
        return f(None, dtype, q, kimp, k, wk, scores, None, None, B, Hq, Hkv, sg, G, slot, Lr,
                 L_cap, D, dp, tb, te)
    assert call(tb=-1) == INV and call(te=0) == INV and call(te=1001) == INV
    assert call(tb=5, te=5) == INV                                  # empty range
    assert call(k=FAKE + 768) == INV                                # k_cache without w_k
    assert call(k=FAKE + 768, wk=FAKE + 1024) == INV                # projecting needs t_end = L
    assert call(k=FAKE + 768, wk=FAKE + 1024, te=1000, D=96) == UNS
    assert call(k=FAKE, wk=FAKE + 1024, te=1000, kimp=FAKE) == INV  # kimp aliases k_cache
    assert call(slot=4) == INV and call(dp=24) == UNS and call(Hq=24) == UNS
    assert call(scores=MIS) == INV and call(q=None) == INV
