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


def test_prefill_llama_shape_one_chunk_pair():
    w = synthetic.WORKLOADS[5].replace(B=2)
    _prefill_case(w, L=2048, chunk=1024)
