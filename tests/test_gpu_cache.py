"""GPU parity of the selection cache (TokenSelect README, highlights, Selection Cache).

Soft-voting batched decode (B=2, 32/8 heads, D=128, 30% + 4 + 64) over the first steps
of the query walk, at a short row (per-row selection) and a long one (chunked
selection).  Every step: butler_selection_cache decides per (b, KV head) whether the
cached selection stands, then score and select skip the kept rows and attention runs
over the current index lists.  Gates:
  flags     equal to the oracle's float64 decision, except where the oracle's cosine lies
            within 1e-5 of the threshold (the device sums in float32);
  reference q_ref rows refreshed exactly where the flag is 0, bit-exact copies;
  kept rows index lists, counts and scores identical to the previous step's;
  selection bit-exact on the GPU's scores for every row (kept rows: the stored ones);
  attention max-abs 2e-2 over the current index lists.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import check_attend, check_select_exact, np64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("L,den", [(3001, 0), (9001, 0), (30001, 16)])
def test_selection_cache_softvote_walk(L, den):
    """den 16: the 1/16 budget, whose rows hold many candidates (chunk regions sorted by
    coarse bin), so kept rows skip that path's kernels and leave its workspace state."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[3].replace(B=2, L=L)
    if den:
        w = w.replace(budget_num=1, budget_den=den)
    threshold, steps = 0.9975, 6
    print(f"[cache] B={w.B} L={L} threshold={threshold} steps={steps}", flush=True)
    cache = synthetic.softvote_cache(w)
    qs = synthetic.softvote_queries(w, steps)
    dev = "cuda"
    k, v = cache["k_cache"].to(dev), cache["v_cache"].to(dev)
    q_ref = torch.zeros_like(qs[0], device=dev)
    keep = torch.zeros(w.B, w.Hkv, dtype=torch.int32, device=dev)
    cap = w.cap(L)
    scores = torch.zeros(w.B, w.Hkv, 1, L, dtype=torch.float32, device=dev)
    hist = torch.zeros(w.B, w.Hkv, 1, 2048, dtype=torch.int32, device=dev)
    idx = torch.zeros(w.B, w.Hkv, 1, cap, dtype=torch.int32, device=dev)
    cnt = torch.zeros(w.B, w.Hkv, 1, dtype=torch.int32, device=dev)
    out = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
    ref_np = np.zeros((w.B, w.Hq, w.D))
    prev = None
    kept_total = 0
    for s in range(steps):
        q = qs[s].to(dev)
        qa.butler_selection_cache(q, q_ref, keep, Hkv=w.Hkv, threshold=threshold)
        qa.butler_score(qa.BUTLER_SCORE_SOFTVOTE, q, k, scores, Hkv=w.Hkv, L=L,
                        softmax_scale=w.scale, radix_hist=hist, keep=keep)
        qa.butler_select_topk(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window, cnt,
                              idx=idx, radix_hist=hist, keep=keep)
        qa.butler_sparse_decode_attn(q, k, v, out, L=L, idx=idx, count=cnt,
                                     softmax_scale=w.scale)
        torch.cuda.synchronize()
        qn = np64(qs[s])[:, :, 0]
        okeep, _, cos = oracle.selection_cache(qn, ref_np, w.Hkv, threshold)
        gkeep = keep.cpu().numpy().astype(bool)
        band = np.abs(cos - threshold) <= 1e-5
        assert ((gkeep == okeep) | band).all(), (s, cos[gkeep != okeep])
        # the reference follows the device's decision
        ref_np = np.where(gkeep.repeat(w.R, axis=1)[:, :, None], ref_np, qn)
        assert np.array_equal(np64(q_ref)[:, :, 0], ref_np), s
        assert int(hist.abs().sum()) == 0
        cur = {"idx": idx.clone(), "cnt": cnt.clone(), "scores": scores.clone()}
        if prev is not None:
            for b in range(w.B):
                for g in range(w.Hkv):
                    if gkeep[b, g]:
                        assert torch.equal(cur["cnt"][b, g], prev["cnt"][b, g])
                        assert torch.equal(cur["idx"][b, g], prev["idx"][b, g])
                        assert torch.equal(cur["scores"][b, g], prev["scores"][b, g])
        else:
            assert not gkeep.any()          # a zero reference refreshes every row
        kept_total += int(gkeep.sum())
        check_select_exact(idx, cnt, np64(scores), w.budget_num, w.budget_den, w.n_sink,
                           w.n_window)
        ic, cc = idx.cpu().numpy(), cnt.cpu().numpy()
        check_attend(out, qs[s], cache["k_cache"], cache["v_cache"],
                     lambda b, g, i: ic[b, g, i, :cc[b, g, i]], w.scale, w.dtype)
        print(f"  step {s}: kept {int(gkeep.sum())} of {gkeep.size}, "
              f"cos in [{cos.min():.5f}, {cos.max():.5f}]", flush=True)
        prev = cur
    assert 0 < kept_total < steps * w.B * w.Hkv


@pytest.mark.parametrize("L0,den", [(3001, 2), (9001, 2), (30001, 16)])
def test_selection_cache_growing_cache_raw(L0, den):
    """A decode loop on the layer workload (raw scorer) whose cache grows by one token per
    step, the query walking (sigma 0.05) so some rows are kept and others refreshed.  Each
    step projects the appended key row inside the scoring launch, scores and selects the
    refreshed rows, and attends over the current lists.  A kept row must hold the previous
    step's set with the window re-taken at the current length (oracle.cached_selection),
    so the appended token is attended; one workspace (keyed by rows) serves every length.
    Gates: the appended K_imp row bit-exact for every head; keep flags as the oracle's
    float64 decision (band 1e-5); refreshed rows' scores bit-exact and their sets
    bit-exact on the GPU's scores; kept rows' sets and counts exact; attention within
    2e-2 of the oracle over the current sets."""
    import query_aware_sparse_imp_amd as qa
    steps, threshold = 6, 0.9975
    w = synthetic.WORKLOADS[2].replace(budget_num=1, budget_den=den)
    print(f"[cache-grow] L0={L0} budget 1/{den} steps={steps} threshold={threshold}", flush=True)
    inp = synthetic.decode_layer(w, 3, L=L0, extra=steps, with_qimp=False)
    qs = synthetic.softvote_queries(w, steps, layer=3)
    assert torch.equal(qs[0], inp["q"])                  # the walk starts at the layer's query
    dev = "cuda"
    k, v, wk = inp["k_cache"].to(dev), inp["v_cache"].to(dev), inp["w_k"].to(dev)
    L_cap = L0 + steps
    kimp = torch.zeros(w.B, w.Hkv, L_cap, w.dprime, dtype=w.dtype, device=dev)
    qa.butler_project_keys(k, wk, kimp, 0, L0)
    q_ref = torch.zeros_like(qs[0], device=dev)
    keep = torch.zeros(w.B, w.Hkv, dtype=torch.int32, device=dev)
    cap = w.cap(L_cap) + steps
    idx = torch.zeros(w.B, w.Hkv, 1, cap, dtype=torch.int32, device=dev)
    cnt = torch.zeros(w.B, w.Hkv, 1, dtype=torch.int32, device=dev)
    out = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
    ref_np = np.zeros((w.B, w.Hq, w.D))
    kn, wkn = np64(inp["k_cache"]), np64(inp["w_k"])
    prev = None
    kept_total = fresh_total = 0
    for s in range(steps):
        L = L0 + s + 1
        q = qs[s].to(dev)
        qimp = synthetic.qimp_standin(w, 3, qs[s], inp["w_k"]).to(dev)
        scores = torch.full((w.B, w.Hkv, 1, L), float("nan"), device=dev)
        hist = torch.zeros(w.B, w.Hkv, 1, 2048, dtype=torch.int32, device=dev)
        qa.butler_selection_cache(q, q_ref, keep, Hkv=w.Hkv, threshold=threshold)
        qa.butler_project_and_score(qimp, k, wk, kimp, scores, Hkv=w.Hkv, L=L, radix_hist=hist,
                                    keep=keep)
        qa.butler_select_topk(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window, cnt,
                              idx=idx, radix_hist=hist, keep=keep)
        qa.butler_sparse_decode_attn(q, k, v, out, L=L, idx=idx, count=cnt,
                                     softmax_scale=w.scale)
        torch.cuda.synchronize()
        assert int(hist.abs().sum()) == 0
        # the appended key row, for kept and refreshed rows alike
        want_row = oracle.project_keys(kn[:, :, L - 1], wkn, "bf16")
        assert np.array_equal(np64(kimp)[:, :, L - 1], want_row), s
        qn = np64(qs[s])[:, :, 0]
        okeep, _, cos = oracle.selection_cache(qn, ref_np, w.Hkv, threshold)
        gkeep = keep.cpu().numpy().astype(bool)
        assert ((gkeep == okeep) | (np.abs(cos - threshold) <= 1e-5)).all(), s
        ref_np = np.where(gkeep.repeat(w.R, axis=1)[:, :, None], ref_np, qn)
        if prev is None:
            assert not gkeep.any()
        got_s = np64(scores)
        want_s = oracle.score_raw(np64(qimp)[:, :, 0], np64(kimp)[:, :, :L], w.Hkv)
        ic, cc = idx.cpu().numpy(), cnt.cpu().numpy()
        sets = {}
        for b in range(w.B):
            for g in range(w.Hkv):
                got = ic[b, g, 0, :cc[b, g, 0]]
                if gkeep[b, g]:
                    want = oracle.cached_selection(prev[(b, g)], L, w.n_window)
                    assert L - 1 in got, (s, b, g)          # the appended token is attended
                    kept_total += 1
                else:
                    assert np.array_equal(got_s[b, g, 0], want_s[b, g, 0]), (s, b, g)
                    want = oracle.select(got_s[b, g, 0], w.budget(L), w.n_sink, w.n_window)
                    fresh_total += 1
                assert cc[b, g, 0] == len(want) and np.array_equal(got, want), (s, b, g)
                sets[(b, g)] = want
        err = check_attend(out, qs[s], inp["k_cache"], inp["v_cache"],
                           lambda b, g, i: sets[(b, g)], w.scale, w.dtype)
        print(f"  step {s} L={L}: kept {int(gkeep.sum())} of {gkeep.size}, "
              f"attention max-abs {err:.2e}", flush=True)
        prev = sets
    assert kept_total > 0 and fresh_total > w.B * w.Hkv
