"""GPU parity of the decode path (raw scorer): project -> score -> select -> attend.

Workloads: the tiny fp32 decode step (B=1, one head, D=64, L=256, d'=16) and the
Llama-3.1-8B-shaped bf16 layer (32/8 heads, D=128, d'=32, 50% + sink 4 + window 64)
at a ragged size that spans several tiles and at the full L=32768, each over a few
decode steps that append one token.  Every stage is gated on the GPU's own upstream
result (see tests/parity.py); the independent oracle chain is reported.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import (ATOL, check_attend, check_project, check_select_exact, decode_step_gpu,
                    np64, pv_rounding_bound, check_pv_rounding, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import query_aware_sparse_imp_amd  # noqa: F401  (fails loudly if the library is missing)


def _run_decode(w, L, steps, layer=0, report=None):
    import query_aware_sparse_imp_amd as qa
    print(f"[decode] cfg={w.cfg} L={L} steps={steps} layer={layer}", flush=True)
    inp = to_device(synthetic.decode_layer(w, layer, L=L, extra=steps))
    dev = "cuda"
    L_cap = inp["L_cap"]
    kimp = torch.zeros(w.B, w.Hkv, L_cap, w.dprime, dtype=w.dtype, device=dev)
    qa.butler_project_keys(inp["k_cache_d"], inp["w_k_d"], kimp, 0, L)
    torch.cuda.synchronize()
    check_project(kimp, inp["k_cache"], inp["w_k"], 0, L)
    q_imp_slot = np64(inp["q_imp"])[:, :, 0, 0, :]                 # [B, Hq, d']
    for s in range(steps + 1):
        Lc = L + s
        if s > 0:
            qa.butler_project_keys(inp["k_cache_d"], inp["w_k_d"], kimp, Lc - 1, 1)
        r = decode_step_gpu(inp, kimp, Lc, qa.BUTLER_SCORE_RAW, q_imp=inp["q_imp_d"])
        torch.cuda.synchronize()
        if s > 0:
            check_project(kimp, inp["k_cache"], inp["w_k"], Lc - 1, Lc)
        kimp_np = np64(kimp[:, :, :Lc])
        want_s = oracle.score_raw(q_imp_slot[:, :, None, :], kimp_np, w.Hkv)
        got_s = np64(r["scores"])
        if w.dtype == torch.bfloat16:
            assert np.array_equal(got_s, want_s), "raw scores must be bit-exact"
        else:
            qbar = np.abs(q_imp_slot.reshape(w.B, w.Hkv, w.R, -1)).sum(2)
            mag = np.einsum("bgi,bgti->bgt", qbar, np.abs(kimp_np))[:, :, None, :]
            diff = got_s != want_s
            assert (np.abs(got_s - want_s) <= 1e-5 * mag)[diff].all()
        check_select_exact(r["idx"], r["count"], got_s, r["num"], r["den"], w.n_sink,
                           w.n_window)
        idx, cnt = r["idx"].cpu().numpy(), r["count"].cpu().numpy()
        check_attend(r["out"], inp["q"], inp["k_cache"], inp["v_cache"],
                     lambda b, g, i: idx[b, g, i, :cnt[b, g, i]], w.scale, w.dtype)
        # independent oracle chain (reported, not gated)
        kimp_or = oracle.project_keys(np64(inp["k_cache"][:, :, :Lc]), np64(inp["w_k"]),
                                      "bf16" if w.dtype == torch.bfloat16 else "f32")
        ind = oracle.decode_layer_step(q=np64(inp["q"])[:, :, 0], k_cache=np64(inp["k_cache"]),
                                       v_cache=np64(inp["v_cache"]), L=Lc, num=w.budget_num,
                                       den=w.budget_den, n_sink=w.n_sink, n_window=w.n_window,
                                       scale=w.scale, Hkv=w.Hkv, mode="raw",
                                       q_imp_slot=q_imp_slot, kimp=kimp_or)
        jac = []
        for b in range(w.B):
            for g in range(w.Hkv):
                a = set(idx[b, g, 0, :cnt[b, g, 0]].tolist())
                o = set(ind["sel"][b][g].tolist())
                jac.append(len(a & o) / len(a | o))
        err = float(np.abs(r["out"].cpu().double().numpy()[:, :, 0] - ind["out"]).max())
        print(f"  step {s}: L={Lc} independent chain: min Jaccard {min(jac):.6f}, "
              f"max-abs {err:.3e}", flush=True)
        if report is not None:
            report.append((Lc, min(jac), err))


def test_tiny_fp32_decode():
    w = synthetic.WORKLOADS[1]
    _run_decode(w, w.L, steps=2)


def test_layer_bf16_ragged_decode():
    w = synthetic.WORKLOADS[2]
    _run_decode(w, 4133, steps=3, layer=1)


def test_layer_bf16_full_size_decode():
    w = synthetic.WORKLOADS[2]
    rep = []
    _run_decode(w, w.L, steps=2, layer=0, report=rep)
    assert min(j for _, j, _ in rep) > 0.95


def test_decode_is_deterministic():
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2]
    inp = to_device(synthetic.decode_layer(w, 2, L=9000))
    kimp = torch.zeros(w.B, w.Hkv, 9000, w.dprime, dtype=w.dtype, device="cuda")
    qa.butler_project_keys(inp["k_cache_d"], inp["w_k_d"], kimp, 0, 9000)
    outs = [decode_step_gpu(inp, kimp, 9000, qa.BUTLER_SCORE_RAW, q_imp=inp["q_imp_d"])
            for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for key in ("scores", "idx", "count", "out"):
            assert torch.equal(o[key], outs[0][key]), key


def test_full_budget_is_dense_attention():
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2]
    L = 3000
    inp = to_device(synthetic.decode_layer(w, 3, L=L))
    kimp = torch.zeros(w.B, w.Hkv, L, w.dprime, dtype=w.dtype, device="cuda")
    qa.butler_project_keys(inp["k_cache_d"], inp["w_k_d"], kimp, 0, L)
    r = decode_step_gpu(inp, kimp, L, qa.BUTLER_SCORE_RAW, q_imp=inp["q_imp_d"], dense=True)
    torch.cuda.synchronize()
    assert (r["count"].cpu() == L).all()
    dense = oracle.dense_decode_attn(np64(inp["q"])[:, :, 0], np64(inp["k_cache"]),
                                     np64(inp["v_cache"]), L, w.scale)
    assert np.abs(r["out"].cpu().double().numpy()[:, :, 0] - dense).max() <= ATOL[w.dtype]


def test_zero_importance_queries_tie_to_lowest_indices():
    """Q_imp = 0 makes every raw score +0: the budget takes the lowest indices."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2]
    L = 2500
    inp = to_device(synthetic.decode_layer(w, 4, L=L))
    inp["q_imp_d"] = torch.zeros_like(inp["q_imp_d"])
    kimp = torch.zeros(w.B, w.Hkv, L, w.dprime, dtype=w.dtype, device="cuda")
    qa.butler_project_keys(inp["k_cache_d"], inp["w_k_d"], kimp, 0, L)
    r = decode_step_gpu(inp, kimp, L, qa.BUTLER_SCORE_RAW, q_imp=inp["q_imp_d"])
    torch.cuda.synchronize()
    x = L // 2
    want = sorted(set(range(x)) | set(range(L - w.n_window, L)))
    cnt = r["count"].cpu().numpy()
    idx = r["idx"].cpu().numpy()
    for g in range(w.Hkv):
        assert idx[0, g, 0, :cnt[0, g, 0]].tolist() == want


def test_scorer_histogram_matches_selection_without_it():
    """The selection gives bitwise the same result from the scorer's first-digit
    histogram as from its own counting pass, on short, mid and long rows."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2]
    for L in (3000, 9000, 70001, 300001):   # 300001: 128 scorer workgroups per row
        print(f"[hist] L={L}", flush=True)
        inp = to_device(synthetic.decode_layer(w, 5, L=L))
        kimp = torch.zeros(w.B, w.Hkv, L, w.dprime, dtype=w.dtype, device="cuda")
        qa.butler_project_keys(inp["k_cache_d"], inp["w_k_d"], kimp, 0, L)
        a = decode_step_gpu(inp, kimp, L, qa.BUTLER_SCORE_RAW, q_imp=inp["q_imp_d"], use_hist=True)
        b = decode_step_gpu(inp, kimp, L, qa.BUTLER_SCORE_RAW, q_imp=inp["q_imp_d"], use_hist=False)
        torch.cuda.synchronize()
        for key in ("scores", "idx", "count", "out"):
            assert torch.equal(a[key], b[key]), (L, key)
        check_select_exact(a["idx"], a["count"], np64(a["scores"]), w.budget_num, w.budget_den,
                           w.n_sink, w.n_window)


@pytest.mark.parametrize("cfg,L", [(1, 256), (1, 1), (2, 1), (2, 5001), (2, 32768),
                                   (2, 300001)])
def test_project_and_score_matches_separate_calls(cfg, L):
    """butler_project_and_score == butler_project_keys(L-1, 1) + butler_score(RAW): the
    K_imp row, every score and the first-digit histogram bit for bit, whatever stale value
    row L-1 of kimp held; with selection-cache flags the kept rows keep their scores and
    histogram but still get their K_imp row.  The K_imp row is also checked against the
    oracle's correctly rounded projection."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[cfg]
    print(f"[project+score] cfg={cfg} L={L}", flush=True)
    inp = to_device(synthetic.decode_layer(w, 0, L=L))
    dev = "cuda"
    k, wk, qi = inp["k_cache_d"], inp["w_k_d"], inp["q_imp_d"]
    kimp_a = torch.zeros(w.B, w.Hkv, L, w.dprime, dtype=w.dtype, device=dev)
    if L > 1:
        qa.butler_project_keys(k, wk, kimp_a, 0, L - 1)
    kimp_b = kimp_a.clone()
    kimp_b[:, :, L - 1] = 7.0                                   # stale row, overwritten
    sa = torch.empty(w.B, w.Hkv, 1, L, dtype=torch.float32, device=dev)
    sb = torch.empty_like(sa)
    ha = torch.zeros(w.B, w.Hkv, 1, 2048, dtype=torch.int32, device=dev)
    hb = torch.zeros_like(ha)
    qa.butler_project_keys(k, wk, kimp_a, L - 1, 1)
    qa.butler_score(qa.BUTLER_SCORE_RAW, qi, kimp_a, sa, Hkv=w.Hkv, L=L, radix_hist=ha)
    qa.butler_project_and_score(qi, k, wk, kimp_b, sb, Hkv=w.Hkv, L=L, radix_hist=hb)
    torch.cuda.synchronize()
    assert torch.equal(kimp_a, kimp_b)
    assert torch.equal(sa, sb)
    assert torch.equal(ha, hb) and int(ha.sum()) == w.B * w.Hkv * L
    check_project(kimp_b, inp["k_cache"], inp["w_k"], L - 1, L)
    # selection-cache flags: every other (b, KV head) kept
    keep = (torch.arange(w.B * w.Hkv, dtype=torch.int32, device=dev) % 2).view(w.B, w.Hkv)
    kimp_c = kimp_b.clone()
    kimp_c[:, :, L - 1] = -3.0
    sc = torch.full_like(sa, -5.0)
    hc = torch.zeros_like(ha)
    qa.butler_project_and_score(qi, k, wk, kimp_c, sc, Hkv=w.Hkv, L=L, radix_hist=hc, keep=keep)
    torch.cuda.synchronize()
    assert torch.equal(kimp_c, kimp_a)                          # written for kept rows too
    kept = keep.bool()
    assert (sc[kept] == -5.0).all() and int(hc[kept].abs().sum()) == 0
    assert torch.equal(sc[~kept], sa[~kept]) and torch.equal(hc[~kept], ha[~kept])


@pytest.mark.parametrize("L,Hq,num,den,use_hist", [
    (3001, 32, 1, 2, True),      # short row: the two calls' kernels
    (5001, 32, 1, 2, True),      # fused, ragged last chunk
    (32768, 32, 1, 2, True),     # fused, the layer workload's length
    (70001, 32, 1, 16, False),   # fused with 16 keys per thread, no scorer histogram
    (262144, 32, 1, 16, True),   # the long-context consumer layer: many candidates per row
    (9000, 8, 3, 10, True),      # R = 1
    (9000, 64, 1, 2, True),      # R = 8
    (9000, 32, 1, 1, True),      # budget takes every token
    (9000, 32, 0, 1, True),      # budget 0: sink and window only
    (32768, 32, 1, 2, "fo"),     # the budget excludes the sink and the window
    (3001, 32, 1, 2, "fo"),
    (150001, 32, 1, 16, "fo"),   # ... with many candidates per row (sorted regions)
])
def test_select_attend_matches_separate_calls(L, Hq, num, den, use_hist):
    """butler_select_attend == butler_select_topk + butler_sparse_decode_attn: idx and count
    bit for bit, the output within the bf16 probability rounding of the separate attention
    (per element, pv_rounding_bound: the two split the set differently) and within
    the bf16 bound of the oracle's attention over the same sets; three calls in a row (the
    selection's workspace state carries over between calls)."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2].replace(Hq=Hq)
    fo = use_hist == "fo"
    use_hist = use_hist is True
    print(f"[select+attend] L={L} Hq={Hq} budget={num}/{den} hist={use_hist} "
          f"budget_excludes_forced={fo}", flush=True)
    inp = to_device(synthetic.decode_layer(w, 0, L=L, with_qimp=False))
    dev = "cuda"
    k, v, q = inp["k_cache_d"], inp["v_cache_d"], inp["q_d"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(L + Hq)
    scores = torch.randn(w.B, w.Hkv, 1, L, generator=gen, device=dev) * 10.0
    cap = min(L, (L * num) // den + w.n_sink + w.n_window)

    def hist_of():
        """The first-digit histogram butler_score documents, counted from the scores (the
        order-preserving key: -0 as +0, sign set -> all bits flipped, else sign bit set)."""
        if not use_hist:
            return None
        bits = scores.view(torch.int32).to(torch.int64) & 0xffffffff
        bits = torch.where(bits == 0x80000000, torch.zeros_like(bits), bits)
        key = torch.where(bits >= 0x80000000, (~bits) & 0xffffffff, bits | 0x80000000)
        b = (key >> 21).view(w.B * w.Hkv, L)
        h = torch.zeros(w.B * w.Hkv, 2048, dtype=torch.int32, device=dev)
        h.scatter_add_(1, b, torch.ones_like(b, dtype=torch.int32))
        return h.view(w.B, w.Hkv, 1, 2048)
    idx_a = torch.full((w.B, w.Hkv, 1, cap), -1, dtype=torch.int32, device=dev)
    cnt_a = torch.zeros(w.B, w.Hkv, 1, dtype=torch.int32, device=dev)
    out_a = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
    qa.butler_select_topk(scores, num, den, w.n_sink, w.n_window, cnt_a, idx=idx_a,
                          radix_hist=hist_of(), budget_excludes_forced=fo)
    qa.butler_sparse_decode_attn(q, k, v, out_a, L=L, idx=idx_a, count=cnt_a,
                                 softmax_scale=w.scale)
    torch.cuda.synchronize()
    ia, ca = idx_a.cpu().numpy(), cnt_a.cpu().numpy()
    gate = pv_rounding_bound(inp["q"], inp["k_cache"], inp["v_cache"],
                             lambda b, j, i: ia[b, j, i, :ca[b, j, i]], w.scale)
    for rep in range(3):
        idx_b = torch.full_like(idx_a, -1)
        cnt_b = torch.zeros_like(cnt_a)
        out_b = torch.full_like(out_a, float("nan"))
        qa.butler_select_attend(scores, num, den, w.n_sink, w.n_window, cnt_b, idx_b, q, k, v,
                                out_b, L=L, softmax_scale=w.scale, radix_hist=hist_of(),
                                budget_excludes_forced=fo)
        torch.cuda.synchronize()
        assert torch.equal(cnt_a, cnt_b), rep
        assert torch.equal(idx_a, idx_b), rep
        d = check_pv_rounding(out_a, out_b, gate)
    check_select_exact(idx_b, cnt_b, np64(scores), num, den, w.n_sink, w.n_window,
                       exclude_forced=fo)
    ic, cc = idx_b.cpu().numpy(), cnt_b.cpu().numpy()
    err = check_attend(out_b, inp["q"], inp["k_cache"], inp["v_cache"],
                       lambda b, g, i: ic[b, g, i, :cc[b, g, i]], w.scale, w.dtype)
    print(f"  selected {int(cc.sum())}, fused vs separate max-abs {d:.2e}, vs oracle {err:.2e}",
          flush=True)


def test_select_attend_workspace_shared_across_lengths():
    """One workspace (the binding keys the selection calls' buffers by rows) serves calls of
    different lengths in turn: a long row (chunked selection fused with attention, whose
    state lives at the start of the buffer), a short row (per-row selection, then the
    separate attention, whose partials follow that state), the long row again, and a
    length in between.  Every call must give the same idx, count and output as the first
    call of its length on a fresh buffer (bitwise), and the sets the oracle's."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2]
    dev = "cuda"
    lengths = [70001, 3001, 70001, 9000, 3001, 70001]
    ins, ref = {}, {}
    for L in sorted(set(lengths)):
        inp = to_device(synthetic.decode_layer(w, 5, L=L, with_qimp=False))
        gen = torch.Generator(device=dev)
        gen.manual_seed(L)
        ins[L] = (inp, torch.randn(w.B, w.Hkv, 1, L, generator=gen, device=dev))
    for n, L in enumerate(lengths):
        inp, scores = ins[L]
        cap = w.cap(L)
        idx = torch.full((w.B, w.Hkv, 1, cap), -1, dtype=torch.int32, device=dev)
        cnt = torch.zeros(w.B, w.Hkv, 1, dtype=torch.int32, device=dev)
        out = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
        print(f"[shared workspace] call {n}: L={L}", flush=True)
        qa.butler_select_attend(scores, 1, 16, w.n_sink, w.n_window, cnt, idx, inp["q_d"],
                                inp["k_cache_d"], inp["v_cache_d"], out, L=L,
                                softmax_scale=w.scale)
        torch.cuda.synchronize()
        if L not in ref:
            ref[L] = (idx.clone(), cnt.clone(), out.clone())
            check_select_exact(idx, cnt, np64(scores), 1, 16, w.n_sink, w.n_window)
        else:
            assert torch.equal(idx, ref[L][0]) and torch.equal(cnt, ref[L][1]), (n, L)
            assert torch.equal(out, ref[L][2]), (n, L)


@pytest.mark.parametrize("cfg,L,sel_group", [(2, 5001, 0), (2, 300001, 0), (2, 32768, 1),
                                             (1, 256, 0)])
def test_score_tokens_split_equals_one_launch(cfg, L, sel_group):
    """butler_score_tokens: the cached tokens [0, L-1) scored first without projection,
    then the appended token with its K_imp row projected in the same launch, give bit for
    bit what butler_project_and_score gives over [0, L): the K_imp row, every score, the
    first-digit histogram.  A middle range [a, b) writes exactly entries a..b-1 (the
    others keep a planted value) and adds exactly their counts."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[cfg]
    print(f"[score tokens] cfg={cfg} L={L} sel_group={sel_group}", flush=True)
    inp = to_device(synthetic.decode_layer(w, 4, L=L))
    dev = "cuda"
    k, wk, qi = inp["k_cache_d"], inp["w_k_d"], inp["q_imp_d"]
    Hs = qa.selection_heads(w.Hq, w.Hkv, sel_group)
    base = torch.zeros(w.B, w.Hkv, L, w.dprime, dtype=w.dtype, device=dev)
    if L > 1:
        qa.butler_project_keys(k, wk, base, 0, L - 1)
    kimp_a, kimp_b = base.clone(), base.clone()
    kimp_b[:, :, L - 1] = 5.0                                   # stale row, overwritten
    sa = torch.empty(w.B, Hs, 1, L, dtype=torch.float32, device=dev)
    sb = torch.full_like(sa, float("nan"))
    ha = torch.zeros(w.B, Hs, 1, 2048, dtype=torch.int32, device=dev)
    hb = torch.zeros_like(ha)
    qa.butler_project_and_score(qi, k, wk, kimp_a, sa, Hkv=w.Hkv, L=L, radix_hist=ha,
                                sel_group=sel_group)
    qa.butler_score_tokens(qi, kimp_b, sb, Hkv=w.Hkv, L=L, t_begin=0, t_end=L - 1,
                           radix_hist=hb, sel_group=sel_group)
    qa.butler_score_tokens(qi, kimp_b, sb, Hkv=w.Hkv, L=L, t_begin=L - 1, t_end=L, k_cache=k,
                           w_k=wk, radix_hist=hb, sel_group=sel_group)
    torch.cuda.synchronize()
    assert torch.equal(kimp_a, kimp_b)
    assert torch.equal(sa, sb)
    assert torch.equal(ha, hb) and int(hb.sum()) == w.B * Hs * L
    # a middle range
    a, b = L // 3, max(L // 3 + 1, (2 * L) // 3)
    sc = torch.full_like(sa, -7.0)
    hc = torch.zeros_like(ha)
    qa.butler_score_tokens(qi, kimp_a, sc, Hkv=w.Hkv, L=L, t_begin=a, t_end=b, radix_hist=hc,
                           sel_group=sel_group)
    torch.cuda.synchronize()
    assert torch.equal(sc[..., a:b], sa[..., a:b])
    assert (sc[..., :a] == -7.0).all() and (sc[..., b:] == -7.0).all()
    assert int(hc.sum()) == w.B * Hs * (b - a)
