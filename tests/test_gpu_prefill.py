"""GPU parity of the producer and of chunked causal prefill.

Producer f_theta: Q_imp = relu(LN(H) W1) W2 with the long-context decode shapes (one
row, E=4096, F=1024, 32 heads x G=4 x d'=32) and with a multi-row prefill block; gated
at max-abs 2e-2 against the oracle (the normalised row, hidden activation and output are
bf16, so single-ulp flips of the intermediates are expected and reported).

Chunked prefill (B, 32/8 heads, D=128, d'=32): Q_imp from the producer (slot 0), K_imp
projected for the whole sequence, then per chunk of query rows: causal raw scores
(bit-exact), per-row top-50% + sink 4 + window 64 into a bitmask (bit-exact on the
GPU's scores) and masked attention over each row's set (max-abs 2e-2).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import bitmask_to_sets, check_project, np64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _producer_case(w, rows, layer):
    import query_aware_sparse_imp_amd as qa
    print(f"[producer] B={w.B} rows={rows} E={w.E} F={w.F} layer={layer}", flush=True)
    h = synthetic.producer_hidden(w, layer, rows)
    wts = synthetic.producer_weights(w, layer)
    q_imp = torch.empty(w.B, w.Hq, w.G, rows, w.dprime, dtype=torch.bfloat16, device="cuda")
    # the library takes the weights in the [out, in] layout of a PyTorch Linear
    qa.butler_produce_queries(h.cuda(), wts["w1"].t().contiguous().cuda(),
                              wts["w2"].t().contiguous().cuda(), q_imp)
    torch.cuda.synchronize()
    want = oracle.produce_queries(np64(h), np64(wts["w1"]), np64(wts["w2"]), w.Hq, w.G,
                                  w.dprime, 1e-5)
    got = np64(q_imp)
    err = np.abs(got - want)
    u = oracle.ulps_bf16(got, want)
    print(f"  max-abs {err.max():.3e}, elements off by >=1 ulp: {(u > 0).mean():.4%}",
          flush=True)
    assert err.max() <= 2e-2
    return q_imp


def test_producer_decode_row():
    w = synthetic.WORKLOADS[4]
    _producer_case(w, 1, layer=4)


@pytest.mark.parametrize("B,E,F", [(4, 4096, 1024), (3, 576, 320), (2, 8192, 512)])
def test_producer_decode_rows_gemv_shapes(B, E, F):
    """Up to four decode rows take the GEMV: the largest batch, a ragged small shape (K not
    a multiple of 512) and the longest hidden row."""
    w = synthetic.WORKLOADS[4].replace(B=B, E=E, F=F)
    _producer_case(w, 1, layer=2)


def test_producer_few_rows_valu_gemm():
    """13 rows: more than the GEMV takes, fewer than the matrix-core tiles want."""
    w = synthetic.WORKLOADS[5].replace(B=1)
    _producer_case(w, 13, layer=3)


def test_producer_prefill_rows():
    w = synthetic.WORKLOADS[5]
    _producer_case(w, 77, layer=0)


def test_producer_prefill_chunk():
    """One 1024-row prefill chunk of both sequences (the matrix-core GEMM, split over K)."""
    w = synthetic.WORKLOADS[5]
    _producer_case(w, 1024, layer=1)


def _prefill_case(w, L, chunk):
    import query_aware_sparse_imp_amd as qa
    print(f"[prefill] B={w.B} L={L} chunk={chunk}", flush=True)
    inp = synthetic.prefill_inputs(w, L=L)
    dev = "cuda"
    q_imp = torch.empty(w.B, w.Hq, w.G, L, w.dprime, dtype=torch.bfloat16, device=dev)
    qa.butler_produce_queries(inp["h"].cuda(), inp["w1"].t().contiguous().cuda(),
                              inp["w2"].t().contiguous().cuda(), q_imp)
    k_d, v_d, q_d = inp["k_cache"].cuda(), inp["v_cache"].cuda(), inp["q"].cuda()
    kimp = torch.empty(w.B, w.Hkv, L, w.dprime, dtype=torch.bfloat16, device=dev)
    qa.butler_project_keys(k_d, inp["w_k"].cuda(), kimp, 0, L)
    torch.cuda.synchronize()
    check_project(kimp, inp["k_cache"], inp["w_k"], 0, L)
    qi = np64(q_imp)[:, :, 0]                                      # slot 0, [B, Hq, L, d']
    kn = np64(kimp)
    rng = np.random.default_rng(0)
    for c0 in range(0, L, chunk):
        Lq = min(chunk, L - c0)
        Lk = c0 + Lq
        scores = torch.empty(w.B, w.Hkv, Lq, Lk, dtype=torch.float32, device=dev)
        hist = torch.zeros(w.B, w.Hkv, Lq, 2048, dtype=torch.int32, device=dev)
        qa.butler_score(qa.BUTLER_SCORE_RAW, q_imp[:, :, :, c0:c0 + Lq].contiguous(), kimp,
                        scores, Hkv=w.Hkv, L=Lk, slot=0, q_pos0=c0, causal=True,
                        radix_hist=hist)
        bm = torch.zeros(w.B, w.Hkv, Lq, (Lk + 31) // 32, dtype=torch.int32, device=dev)
        cnt = torch.zeros(w.B, w.Hkv, Lq, dtype=torch.int32, device=dev)
        qa.butler_select_topk(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window, cnt,
                              bitmask=bm, q_pos0=c0, causal=True, radix_hist=hist)
        out = torch.empty(w.B, w.Hq, Lq, w.D, dtype=torch.float32, device=dev)
        qa.butler_sparse_decode_attn(q_d[:, :, c0:c0 + Lq].contiguous(), k_d, v_d, out, L=Lk,
                                     bitmask=bm, q_pos0=c0, softmax_scale=w.scale)
        torch.cuda.synchronize()
        assert int(hist.abs().sum()) == 0, "multi-row calls leave the histogram untouched"
        got_s = np64(scores)
        want_s = oracle.score_raw(qi[:, :, c0:c0 + Lq], kn[:, :, :Lk], w.Hkv, causal=True,
                                  q_pos0=c0)
        assert np.array_equal(got_s, want_s), f"causal raw scores differ in chunk at {c0}"
        sets = bitmask_to_sets(bm, Lk)
        cn = cnt.cpu().numpy()
        rows = [(b, g, i) for b in range(w.B) for g in range(w.Hkv) for i in range(Lq)]
        if len(rows) > 400:
            rows = [rows[j] for j in sorted(rng.choice(len(rows), 400, replace=False))]
        for (b, g, i) in rows:
            L_r = c0 + i + 1
            want = oracle.select(got_s[b, g, i, :L_r], oracle.budget(L_r, 1, 2), w.n_sink,
                                 w.n_window)
            assert np.array_equal(np.nonzero(sets[b, g, i])[0], want), (c0, b, g, i)
            assert cn[b, g, i] == len(want)
        o = out.cpu().double().numpy()
        qn = np64(inp["q"])
        worst = 0.0
        for (b, g, i) in rows:
            sel = np.nonzero(sets[b, g, i])[0]
            for r in range(w.R):
                h = g * w.R + r
                want = oracle.attend(qn[b, h, c0 + i][None], np64(inp["k_cache"][b, g, sel]),
                                     np64(inp["v_cache"][b, g, sel]), w.scale)[0]
                worst = max(worst, float(np.abs(o[b, h, i] - want).max()))
        assert worst <= 2e-2, worst
        print(f"  chunk {c0}: rows checked {len(rows)}, attention max-abs {worst:.3e}",
              flush=True)


def test_prefill_small_chunks():
    w = synthetic.WORKLOADS[5].replace(B=1, E=256, F=128)
    _prefill_case(w, L=300, chunk=128)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (4, 4), (4, 2)])
def test_prefill_small_chunks_head_groups(Hq, Hkv):
    """Groups of 8, 1 and 2 query heads per KV head: the causal scorer's instances for
    R = 8, 1 and 2, and the bitmask attention off the R = 4 path."""
    w = synthetic.WORKLOADS[5].replace(B=1, E=256, F=128, Hq=Hq, Hkv=Hkv)
    _prefill_case(w, L=300, chunk=128)


def test_prefill_llama_shape_one_chunk_pair():
    w = synthetic.WORKLOADS[5].replace(B=2)
    _prefill_case(w, L=2048, chunk=1024)


def _chunked_prefill(w, inp, L, chunk, two_streams):
    """Per chunk: producer on the chunk's hidden rows, K_imp of its keys, causal raw scores
    (the front), then per-row selection and masked attention (the back).  With two_streams,
    each chunk's back runs on a second stream after an event on its own front, beside the
    next chunks' fronts.  Outputs and bitmasks start poisoned (NaN, -1)."""
    import query_aware_sparse_imp_amd as qa
    dev = "cuda"
    h = inp["h"].cuda()
    w1, w2 = inp["w1"].t().contiguous().cuda(), inp["w2"].t().contiguous().cuda()
    k_d, v_d, q_d, wk = (inp["k_cache"].cuda(), inp["v_cache"].cuda(), inp["q"].cuda(),
                         inp["w_k"].cuda())
    kimp = torch.empty(w.B, w.Hkv, L, w.dprime, dtype=torch.bfloat16, device=dev)
    starts = list(range(0, L, chunk))
    outs, bms, cnts, keep = [], [], [], []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for c0 in starts:
        Lq = min(chunk, L - c0)
        Lk = c0 + Lq
        qimp = torch.empty(w.B, w.Hq, w.G, Lq, w.dprime, dtype=torch.bfloat16, device=dev)
        hc = h[:, c0:c0 + Lq].contiguous()
        qc = q_d[:, :, c0:c0 + Lq].contiguous()
        scores = torch.empty(w.B, w.Hkv, Lq, Lk, dtype=torch.float32, device=dev)
        bm = torch.full((w.B, w.Hkv, Lq, (Lk + 31) // 32), -1, dtype=torch.int32, device=dev)
        cnt = torch.full((w.B, w.Hkv, Lq), -1, dtype=torch.int32, device=dev)
        out = torch.full((w.B, w.Hq, Lq, w.D), float("nan"), dtype=torch.float32, device=dev)
        keep += [qimp, hc, qc, scores]
        qa.butler_produce_queries(hc, w1, w2, qimp)
        qa.butler_project_keys(k_d, wk, kimp, c0, Lq)
        qa.butler_score(qa.BUTLER_SCORE_RAW, qimp, kimp, scores, Hkv=w.Hkv, L=Lk, slot=0,
                        q_pos0=c0, causal=True)

        def back(scores=scores, bm=bm, cnt=cnt, out=out, qc=qc, c0=c0, Lk=Lk):
            qa.butler_select_topk(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window,
                                  cnt, bitmask=bm, q_pos0=c0, causal=True)
            qa.butler_sparse_decode_attn(qc, k_d, v_d, out, L=Lk, bitmask=bm, q_pos0=c0,
                                         softmax_scale=w.scale)

        if two_streams:
            e = torch.cuda.Event()
            e.record()
            with torch.cuda.stream(side):
                side.wait_event(e)
                back()
        else:
            back()
        outs.append(out)
        bms.append(bm)
        cnts.append(cnt)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return outs, bms, cnts


def test_prefill_two_streams_matches_one_stream():
    """The bench's two-stream prefill schedule (chunk c's selection and attention on a
    second stream beside chunk c+1's producer, projection and scores) gives the one-stream
    schedule's outputs, bitmasks and counts bit for bit (the one-stream path's parity with
    the oracle is checked by the tests above)."""
    w = synthetic.WORKLOADS[5].replace(B=2)
    L, chunk = 2048, 512
    print(f"[prefill two streams] B={w.B} L={L} chunk={chunk}", flush=True)
    inp = synthetic.prefill_inputs(w, L=L)
    one = _chunked_prefill(w, inp, L, chunk, two_streams=False)
    two = _chunked_prefill(w, inp, L, chunk, two_streams=True)
    for name, a, b in zip(("out", "bitmask", "count"), one, two):
        for c, (x, y) in enumerate(zip(a, b)):
            assert not torch.isnan(x).any() if x.is_floating_point() else (x != -1).any()
            assert torch.equal(x, y), f"{name} of chunk {c} differs between the schedules"


def _sample_rows(rng, B, Hkv, Lq, n):
    """n (b, g, i) rows of a chunk: its first and last rows of the first and last heads,
    the rest at random."""
    fixed = [(0, 0, 0), (B - 1, Hkv - 1, Lq - 1), (0, Hkv - 1, Lq - 2), (B - 1, 0, Lq // 2)]
    rnd = [(int(rng.integers(B)), int(rng.integers(Hkv)), int(rng.integers(Lq)))
           for _ in range(n - len(fixed))]
    return sorted(set(fixed + rnd))


def test_prefill_full_size_all_chunks_sampled():
    """The prefill workload at its stated size (B=2, L=8192, eight chunks of 1024 rows) in
    the launch configuration the bench times: per chunk the producer on the chunk's hidden
    rows (M = 2048), K_imp of the chunk's keys, causal raw scores against the prefix,
    per-row top 50% + 4 + 64 into a bitmask, masked attention of every row.  K_imp is
    compared whole; Q_imp, scores, sets and attention on sampled rows of every chunk
    (including the last rows of the last chunk, whose prefix is the whole sequence)."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[5]
    L, C = w.L, w.chunk
    print(f"[prefill-full] B={w.B} L={L} chunk={C}", flush=True)
    inp = synthetic.prefill_inputs(w, L=L)
    dev = "cuda"
    h_d = inp["h"].to(dev)
    w1 = inp["w1"].t().contiguous().to(dev)
    w2 = inp["w2"].t().contiguous().to(dev)
    k_d, v_d, q_d = inp["k_cache"].to(dev), inp["v_cache"].to(dev), inp["q"].to(dev)
    wk_d = inp["w_k"].to(dev)
    kimp = torch.empty(w.B, w.Hkv, L, w.dprime, dtype=torch.bfloat16, device=dev)
    hn, w1n, w2n = np64(inp["h"]), np64(inp["w1"]), np64(inp["w2"])
    qn, kc, vc = np64(inp["q"]), np64(inp["k_cache"]), np64(inp["v_cache"])
    rng = np.random.default_rng(5)
    for c0 in range(0, L, C):
        Lk = c0 + C
        qimp = torch.empty(w.B, w.Hq, w.G, C, w.dprime, dtype=torch.bfloat16, device=dev)
        qa.butler_produce_queries(h_d[:, c0:Lk].contiguous(), w1, w2, qimp)
        qa.butler_project_keys(k_d, wk_d, kimp, c0, C)
        scores = torch.empty(w.B, w.Hkv, C, Lk, dtype=torch.float32, device=dev)
        hist = torch.zeros(w.B, w.Hkv, C, 2048, dtype=torch.int32, device=dev)
        qa.butler_score(qa.BUTLER_SCORE_RAW, qimp, kimp, scores, Hkv=w.Hkv, L=Lk, slot=0,
                        q_pos0=c0, causal=True, radix_hist=hist)
        bm = torch.zeros(w.B, w.Hkv, C, (Lk + 31) // 32, dtype=torch.int32, device=dev)
        cnt = torch.zeros(w.B, w.Hkv, C, dtype=torch.int32, device=dev)
        qa.butler_select_topk(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window, cnt,
                              bitmask=bm, q_pos0=c0, causal=True, radix_hist=hist)
        out = torch.empty(w.B, w.Hq, C, w.D, dtype=torch.float32, device=dev)
        qa.butler_sparse_decode_attn(q_d[:, :, c0:Lk].contiguous(), k_d, v_d, out, L=Lk,
                                     bitmask=bm, q_pos0=c0, softmax_scale=w.scale)
        torch.cuda.synchronize()
        check_project(kimp, inp["k_cache"], inp["w_k"], c0, Lk)
        rows = _sample_rows(rng, w.B, w.Hkv, C, 24)
        # producer rows: every head and slot of the sampled token positions
        ts = sorted({i for (_, _, i) in rows})
        want_q = oracle.produce_queries(hn[:, [c0 + i for i in ts]], w1n, w2n, w.Hq, w.G,
                                        w.dprime, 1e-5)
        got_q = np64(qimp)[:, :, :, ts]
        qerr = float(np.abs(got_q - want_q).max())
        assert qerr <= 2e-2, (c0, qerr)
        qi, kn = np64(qimp)[:, :, 0], np64(kimp)
        sets = bitmask_to_sets(bm, Lk)
        cn, o = cnt.cpu().numpy(), out.cpu().double().numpy()
        worst = 0.0
        for (b, g, i) in rows:
            L_r = c0 + i + 1
            want_s = oracle.score_raw(qi[b:b + 1, g * w.R:(g + 1) * w.R, i:i + 1],
                                      kn[b:b + 1, g:g + 1, :Lk], 1, causal=True,
                                      q_pos0=c0 + i)[0, 0, 0]
            got_s = np64(scores[b, g, i])
            assert np.array_equal(got_s, want_s), ("scores", c0, b, g, i)
            want = oracle.select(got_s[:L_r], oracle.budget(L_r, w.budget_num, w.budget_den),
                                 w.n_sink, w.n_window)
            assert np.array_equal(np.nonzero(sets[b, g, i])[0], want), ("set", c0, b, g, i)
            assert cn[b, g, i] == len(want)
            for r in range(w.R):
                hh = g * w.R + r
                ref = oracle.attend(qn[b, hh, c0 + i][None], kc[b, g, want], vc[b, g, want],
                                    w.scale)[0]
                worst = max(worst, float(np.abs(o[b, hh, i] - ref).max()))
        assert worst <= 2e-2, (c0, worst)
        print(f"  chunk at {c0}: rows {len(rows)}, Q_imp max-abs {qerr:.2e}, "
              f"attention max-abs {worst:.2e}", flush=True)


def test_producer_whole_prompt_sampled():
    """The producer over the whole prompt of both sequences at once (M = 16384 rows: the
    matrix-core GEMM with one K split, its ReLU epilogue inside the GEMM), checked on
    sampled token positions, every head and slot."""
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[5]
    rows = w.L
    print(f"[producer] B={w.B} rows={rows} (whole prompt)", flush=True)
    h = synthetic.producer_hidden(w, 6, rows)
    wts = synthetic.producer_weights(w, 6)
    q_imp = torch.empty(w.B, w.Hq, w.G, rows, w.dprime, dtype=torch.bfloat16, device="cuda")
    qa.butler_produce_queries(h.cuda(), wts["w1"].t().contiguous().cuda(),
                              wts["w2"].t().contiguous().cuda(), q_imp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    ts = sorted(set([0, 1, 4095, 4096, rows - 1] + rng.integers(0, rows, 59).tolist()))
    want = oracle.produce_queries(np64(h)[:, ts], np64(wts["w1"]), np64(wts["w2"]), w.Hq, w.G,
                                  w.dprime, 1e-5)
    got = np64(q_imp)[:, :, :, ts]
    err = float(np.abs(got - want).max())
    u = oracle.ulps_bf16(got, want)
    print(f"  {len(ts)} positions: max-abs {err:.3e}, elements off by >=1 ulp: "
          f"{(u > 0).mean():.4%}", flush=True)
    assert err <= 2e-2
