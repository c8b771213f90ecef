"""GPU parity of selection heads smaller than a GQA group (per-query-head selection).

The model card (Method) gives Q_imp one d'-vector per attention head but leaves open
whether the query heads of a KV head share their selected set.  With sel_group = 1
every query head scores, selects and attends on its own; sel_group = 2 shares a set
between two of the four heads of a Llama-3.1-8B KV head.  Each stage is gated on the
GPU's own upstream result, as in the other decode tests: raw scores bit-exact, the
selection bit-exact, attention within the bf16 bound of the oracle over the same sets.
Shapes: the Llama-shaped decode layer (32/8 heads, D = 128, d' = 32, 50% + 4 + 64) at a
ragged length, a mid length and the full 32768; the soft-voting scorer at B = 2; causal
prefill rows; the selection cache.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import ATOL, pv_rounding_bound, check_pv_rounding, bitmask_to_sets, check_project, check_select_exact, np64, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import query_aware_sparse_imp_amd  # noqa: F401  (fails loudly if the library is missing)


def _check_attend_heads(out, q, k_cache, v_cache, sets, scale, gs, R, atol):
    """Every query head h against the oracle over the set of selection head h // gs."""
    o = out.cpu().double().numpy()
    qn, kn, vn = np64(q), k_cache, v_cache
    B, Hq, Lq, _ = q.shape
    worst = 0.0
    for b in range(B):
        for h in range(Hq):
            for i in range(Lq):
                sel = np.asarray(sets(b, h // gs, i), np.int64)
                want = oracle.attend(qn[b, h, i][None], np64(kn[b, h // R, sel]),
                                     np64(vn[b, h // R, sel]), scale)[0]
                worst = max(worst, float(np.abs(o[b, h, i] - want).max()))
    assert worst <= atol, f"attention max-abs {worst} > {atol}"
    return worst


@pytest.mark.parametrize("L,gs,den", [(4133, 1, 2), (9000, 2, 2), (32768, 1, 2),
                                      (150001, 1, 16)])
def test_decode_chain_per_selection_head(L, gs, den):
    """project -> score -> select -> attend with sel_group = gs, then the fused
    project_and_score and select_attend calls on the same step.  The 1/16 budget (window
    128) at 150001 tokens gives every selection row thousands of candidates: the chunks
    sort them by coarse bin, in the fused pass too."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2]
    if den != 2:
        w = w.replace(budget_den=den, n_window=128)
    Hs = w.Hq // gs
    print(f"[sel_group] decode L={L} sel_group={gs} Hs={Hs} budget 1/{den}", flush=True)
    inp = to_device(synthetic.decode_layer(w, 1, L=L))
    dev = "cuda"
    k, v, q = inp["k_cache_d"], inp["v_cache_d"], inp["q_d"]
    kimp = torch.zeros(w.B, w.Hkv, L, w.dprime, dtype=w.dtype, device=dev)
    qa.butler_project_keys(k, inp["w_k_d"], kimp, 0, L)
    scores = torch.empty(w.B, Hs, 1, L, dtype=torch.float32, device=dev)
    hist = torch.zeros(w.B, Hs, 1, 2048, dtype=torch.int32, device=dev)
    qa.butler_score(qa.BUTLER_SCORE_RAW, inp["q_imp_d"], kimp, scores, Hkv=w.Hkv, L=L,
                    radix_hist=hist, sel_group=gs)
    cap = w.cap(L)
    idx = torch.full((w.B, Hs, 1, cap), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(w.B, Hs, 1, dtype=torch.int32, device=dev)
    qa.butler_select_topk(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window, cnt,
                          idx=idx, radix_hist=hist)
    out = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
    qa.butler_sparse_decode_attn(q, k, v, out, L=L, idx=idx, count=cnt, softmax_scale=w.scale,
                                 sel_group=gs)
    torch.cuda.synchronize()
    assert int(hist.abs().sum()) == 0
    check_project(kimp, inp["k_cache"], inp["w_k"], 0, L)
    qi = np64(inp["q_imp"])[:, :, 0]                               # [B, Hq, 1, d']
    want_s = oracle.score_raw(qi, np64(kimp), w.Hkv, sel_group=gs)
    got_s = np64(scores)
    assert np.array_equal(got_s, want_s), "raw per-selection-head scores must be bit-exact"
    check_select_exact(idx, cnt, got_s, w.budget_num, w.budget_den, w.n_sink, w.n_window)
    ic, cc = idx.cpu().numpy(), cnt.cpu().numpy()
    sets = lambda b, j, i: ic[b, j, i, :cc[b, j, i]]
    err = _check_attend_heads(out, inp["q"], inp["k_cache"], inp["v_cache"], sets, w.scale,
                              gs, w.R, ATOL[w.dtype])
    # the first two selection heads of each KV head really select different sets
    kvdiv = w.R // gs
    differ = sum(not np.array_equal(sets(0, g * kvdiv, 0), sets(0, g * kvdiv + 1, 0))
                 for g in range(w.Hkv))
    assert differ > 0
    print(f"  selected {int(cc.sum())}, attention max-abs {err:.2e}, "
          f"KV heads whose first two sets differ: {differ} of {w.Hkv}", flush=True)

    # fused projection + scoring: the last key row projected in the same launch
    kimp2 = kimp.clone()
    kimp2[:, :, L - 1].zero_()
    scores2 = torch.empty_like(scores)
    hist2 = torch.zeros_like(hist)
    qa.butler_project_and_score(inp["q_imp_d"], k, inp["w_k_d"], kimp2, scores2, Hkv=w.Hkv,
                                L=L, radix_hist=hist2, sel_group=gs)
    torch.cuda.synchronize()
    assert torch.equal(kimp2, kimp), "the fused call writes the same K_imp row"
    assert torch.equal(scores2, scores)
    assert torch.equal(hist2.sum(-1), torch.full_like(hist2.sum(-1), L))

    # fused selection + attention, twice (the workspace state carries over)
    gate = pv_rounding_bound(inp["q"], inp["k_cache"], inp["v_cache"], sets, w.scale,
                             sel_group=gs)
    for rep in range(2):
        idx_b = torch.full_like(idx, -1)
        cnt_b = torch.zeros_like(cnt)
        out_b = torch.empty_like(out)
        qa.butler_select_attend(scores2, w.budget_num, w.budget_den, w.n_sink, w.n_window,
                                cnt_b, idx_b, q, k, v, out_b, L=L, softmax_scale=w.scale,
                                radix_hist=hist2 if rep == 0 else None, sel_group=gs)
        torch.cuda.synchronize()
        assert torch.equal(cnt_b, cnt) and torch.equal(idx_b, idx), rep
        d = check_pv_rounding(out, out_b, gate)
    assert int(hist2.abs().sum()) == 0
    print(f"  fused calls: same K_imp row, scores, sets; output within {d:.2e}", flush=True)


def test_softvote_per_query_head():
    """Soft voting with one query head per set: each head's own softmax (relative 1e-5
    of the oracle), the selection exact on the GPU's scores, attention per head."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[3].replace(B=2, L=5000)
    print(f"[sel_group] softvote B={w.B} L={w.L} sel_group=1", flush=True)
    cache = synthetic.softvote_cache(w)
    q = synthetic.softvote_queries(w, 1)[0]
    dev = "cuda"
    k, v, qd = cache["k_cache"].to(dev), cache["v_cache"].to(dev), q.to(dev)
    L, Hs = w.L, w.Hq
    scores = torch.empty(w.B, Hs, 1, L, dtype=torch.float32, device=dev)
    hist = torch.zeros(w.B, Hs, 1, 2048, dtype=torch.int32, device=dev)
    qa.butler_score(qa.BUTLER_SCORE_SOFTVOTE, qd, k, scores, Hkv=w.Hkv, L=L,
                    softmax_scale=w.scale, radix_hist=hist, sel_group=1)
    cap = w.cap(L)
    idx = torch.full((w.B, Hs, 1, cap), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(w.B, Hs, 1, dtype=torch.int32, device=dev)
    qa.butler_select_topk(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window, cnt,
                          idx=idx, radix_hist=hist)
    out = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
    qa.butler_sparse_decode_attn(qd, k, v, out, L=L, idx=idx, count=cnt, softmax_scale=w.scale,
                                 sel_group=1)
    torch.cuda.synchronize()
    got = np64(scores)
    want = oracle.score_softvote(np64(q), np64(cache["k_cache"]), w.Hkv, w.scale, sel_group=1)
    err = np.abs(got - want)
    assert (err <= 1e-5 * np.abs(want) + 1e-30).all(), float(err.max())
    np.testing.assert_allclose(got.sum(-1), 1.0, atol=1e-3)
    check_select_exact(idx, cnt, got, w.budget_num, w.budget_den, w.n_sink, w.n_window)
    ic, cc = idx.cpu().numpy(), cnt.cpu().numpy()
    e = _check_attend_heads(out, q, cache["k_cache"], cache["v_cache"],
                            lambda b, j, i: ic[b, j, i, :cc[b, j, i]], w.scale, 1, w.R,
                            ATOL[w.dtype])
    print(f"  attention max-abs {e:.2e}", flush=True)


@pytest.mark.parametrize("gs", [1, 2])
def test_prefill_rows_per_selection_head(gs):
    """Causal prefill rows with sel_group = gs: the matrix-core scorer bit-exact, the
    bitmask selection exact, the bitmask attention per head on sampled rows."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[5].replace(B=1, E=256, F=128)
    L, Hs = 300, w.Hq // gs
    print(f"[sel_group] prefill L={L} sel_group={gs}", flush=True)
    inp = synthetic.prefill_inputs(w, L=L)
    dev = "cuda"
    q_imp = torch.empty(w.B, w.Hq, w.G, L, w.dprime, dtype=torch.bfloat16, device=dev)
    qa.butler_produce_queries(inp["h"].cuda(), inp["w1"].t().contiguous().cuda(),
                              inp["w2"].t().contiguous().cuda(), q_imp)
    k_d, v_d, q_d = inp["k_cache"].cuda(), inp["v_cache"].cuda(), inp["q"].cuda()
    kimp = torch.empty(w.B, w.Hkv, L, w.dprime, dtype=torch.bfloat16, device=dev)
    qa.butler_project_keys(k_d, inp["w_k"].cuda(), kimp, 0, L)
    c0, Lq = 172, 128                                  # the second chunk of a 300-token prompt
    Lk = c0 + Lq
    scores = torch.empty(w.B, Hs, Lq, Lk, dtype=torch.float32, device=dev)
    qa.butler_score(qa.BUTLER_SCORE_RAW, q_imp[:, :, :, c0:c0 + Lq].contiguous(), kimp, scores,
                    Hkv=w.Hkv, L=Lk, q_pos0=c0, causal=True, sel_group=gs)
    bm = torch.zeros(w.B, Hs, Lq, (Lk + 31) // 32, dtype=torch.int32, device=dev)
    cnt = torch.zeros(w.B, Hs, Lq, dtype=torch.int32, device=dev)
    qa.butler_select_topk(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window, cnt,
                          bitmask=bm, q_pos0=c0, causal=True)
    out = torch.empty(w.B, w.Hq, Lq, w.D, dtype=torch.float32, device=dev)
    qa.butler_sparse_decode_attn(q_d[:, :, c0:c0 + Lq].contiguous(), k_d, v_d, out, L=Lk,
                                 bitmask=bm, q_pos0=c0, softmax_scale=w.scale, sel_group=gs)
    torch.cuda.synchronize()
    qi = np64(q_imp)[:, :, 0, c0:c0 + Lq]
    want_s = oracle.score_raw(qi, np64(kimp)[:, :, :Lk], w.Hkv, causal=True, q_pos0=c0,
                              sel_group=gs)
    got_s = np64(scores)
    assert np.array_equal(got_s, want_s), "causal per-selection-head scores must be bit-exact"
    sets = bitmask_to_sets(bm, Lk)
    cn = cnt.cpu().numpy()
    rng = np.random.default_rng(gs)
    rows = [(b, j, i) for b in range(w.B) for j in range(Hs) for i in range(Lq)]
    rows = [rows[r] for r in sorted(rng.choice(len(rows), 300, replace=False))]
    for (b, j, i) in rows:
        L_r = c0 + i + 1
        want = oracle.select(got_s[b, j, i, :L_r], oracle.budget(L_r, 1, 2), w.n_sink,
                             w.n_window)
        assert np.array_equal(np.nonzero(sets[b, j, i])[0], want), (b, j, i)
        assert cn[b, j, i] == len(want)
    o = out.cpu().double().numpy()
    qn = np64(inp["q"])
    worst = 0.0
    for (b, j, i) in rows:
        sel = np.nonzero(sets[b, j, i])[0]
        for h in range(j * gs, (j + 1) * gs):
            want = oracle.attend(qn[b, h, c0 + i][None], np64(inp["k_cache"][b, h // w.R, sel]),
                                 np64(inp["v_cache"][b, h // w.R, sel]), w.scale)[0]
            worst = max(worst, float(np.abs(o[b, h, i] - want).max()))
    assert worst <= 2e-2, worst
    print(f"  rows checked {len(rows)}, attention max-abs {worst:.3e}", flush=True)


def test_selection_cache_per_query_head():
    """One keep flag per query head: the oracle's per-head cosine decides it (heads whose
    cosine lies within 1e-5 of the threshold are not compared)."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[3].replace(B=4)
    print("[sel_group] selection cache sel_group=1", flush=True)
    qs = synthetic.softvote_queries(w, 3)
    dev = "cuda"
    q_ref = torch.zeros(w.B, w.Hq, 1, w.D, dtype=w.dtype, device=dev)
    keep = torch.full((w.B, w.Hq), -1, dtype=torch.int32, device=dev)
    ref_np = np.zeros((w.B, w.Hq, w.D))
    thr = 0.9985
    for s, q in enumerate(qs):
        qa.butler_selection_cache(q.to(dev), q_ref, keep, Hkv=w.Hkv, threshold=thr, sel_group=1)
        torch.cuda.synchronize()
        want_keep, new_ref, cos = oracle.selection_cache(np64(q)[:, :, 0], ref_np, w.Hkv, thr,
                                                         sel_group=1)
        got = keep.cpu().numpy().astype(bool)
        clear = np.abs(cos - thr) > 1e-5
        assert np.array_equal(got[clear], want_keep[clear]), s
        got_ref = np64(q_ref)[:, :, 0]
        assert np.array_equal(got_ref[clear], new_ref[clear]), s
        ref_np = got_ref                                # the GPU's state carries on
        print(f"  step {s}: kept {int(got.sum())} of {got.size} heads "
              f"({int((~clear).sum())} within 1e-5 of the threshold)", flush=True)


@pytest.mark.parametrize("dtype,D,dp", [(torch.float32, 64, 16), (torch.bfloat16, 64, 32)])
def test_per_head_valu_paths(dtype, D, dp):
    """sel_group = 1 on the shapes that take the VALU kernels: raw and soft-vote scoring,
    the split attention of index lists (D = 64) and the unfused select+attend call (rows of
    at most 4096 tokens); two KV heads of two query heads each, B = 2."""
    import query_aware_sparse_imp_amd as qa
    dev = "cuda"
    B, Hq, Hkv, L = 2, 4, 2, 3001
    print(f"[sel_group] VALU paths dtype={dtype} D={D} d'={dp} L={L}", flush=True)
    g = torch.Generator().manual_seed(D + dp)
    st = lambda *shape: torch.randn(*shape, generator=g).to(dtype)
    k, v = st(B, Hkv, L, D), st(B, Hkv, L, D)
    q = st(B, Hq, 1, D)
    qi = st(B, Hq, 1, 1, dp)
    kimp = st(B, Hkv, L, dp)
    scale = 1.0 / D ** 0.5
    kd, vd, qd, qid, kid = (t.to(dev) for t in (k, v, q, qi, kimp))
    num, den, ns, nw = 1, 2, 4, 16
    cap = min(L, L * num // den + ns + nw)
    for mode in (qa.BUTLER_SCORE_RAW, qa.BUTLER_SCORE_SOFTVOTE):
        scores = torch.empty(B, Hq, 1, L, dtype=torch.float32, device=dev)
        if mode == qa.BUTLER_SCORE_RAW:
            qa.butler_score(mode, qid, kid, scores, Hkv=Hkv, L=L, sel_group=1)
        else:
            qa.butler_score(mode, qd, kd, scores, Hkv=Hkv, L=L, softmax_scale=scale, sel_group=1)
        idx = torch.full((B, Hq, 1, cap), -1, dtype=torch.int32, device=dev)
        cnt = torch.zeros(B, Hq, 1, dtype=torch.int32, device=dev)
        qa.butler_select_topk(scores, num, den, ns, nw, cnt, idx=idx)
        out = torch.empty(B, Hq, 1, D, dtype=torch.float32, device=dev)
        qa.butler_sparse_decode_attn(qd, kd, vd, out, L=L, idx=idx, count=cnt,
                                     softmax_scale=scale, sel_group=1)
        idx2 = torch.full_like(idx, -1)
        cnt2 = torch.zeros_like(cnt)
        out2 = torch.empty_like(out)
        qa.butler_select_attend(scores, num, den, ns, nw, cnt2, idx2, qd, kd, vd, out2, L=L,
                                softmax_scale=scale, sel_group=1)
        torch.cuda.synchronize()
        got = np64(scores)
        if mode == qa.BUTLER_SCORE_RAW:
            want = oracle.score_raw(np64(qi)[:, :, 0], np64(kimp), Hkv, sel_group=1)
            if dtype == torch.bfloat16:
                assert np.array_equal(got, want)
            else:
                mag = np.einsum("bhqi,bhti->bhqt", np.abs(np64(qi)[:, :, 0]),
                                np.abs(np.repeat(np64(kimp), 2, axis=1)))
                assert (np.abs(got - want) <= 1e-5 * mag).all()
        else:
            want = oracle.score_softvote(np64(q), np64(k), Hkv, scale, sel_group=1)
            assert (np.abs(got - want) <= 1e-5 * np.abs(want) + 1e-30).all()
        check_select_exact(idx, cnt, got, num, den, ns, nw)
        assert torch.equal(idx2, idx) and torch.equal(cnt2, cnt)
        assert float((out2 - out).abs().max()) <= 1e-5
        ic, cc = idx.cpu().numpy(), cnt.cpu().numpy()
        err = _check_attend_heads(out, q, k, v, lambda b, j, i: ic[b, j, i, :cc[b, j, i]],
                                  scale, 1, Hq // Hkv, ATOL[dtype])
        print(f"  mode {mode}: attention max-abs {err:.2e}", flush=True)
