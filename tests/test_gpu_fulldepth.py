"""GPU parity of the long-context full-depth decode chain (TokenButler model card, Method
and Memory requirements) on the long-context workload's shapes at a shorter context.

Eight layers of one decode step, each appending one token: producers at layers 0 and 4
run f_theta on LN(H) (E = 4096, F = 1024, 32 heads x G = 4 slots x d' = 32); layer 0 is
dense; consumer layer l scores with slot (l - 1) mod 4 of its producer's Q_imp (slots 0,
1, 2 from layer 0's producer, slot 3 from layer 4's own output, then 0, 1, 2 from it),
inside the launch that projects the appended key row, then selects 1/16 + sink 4 +
window 128 and attends in the fused select+attend call -- the launch configuration of
the full-depth bench step.  The GPU side takes each layer's role from
query_aware_sparse_imp_amd.control; the oracle side from oracle.producer_of / slot_of.

Gates, stage by stage on the GPU's own upstream results:
  producer   Q_imp within 2e-2 of oracle.produce_queries;
  projection the appended K_imp row bit-exact;
  scores     bit-exact against oracle.score_raw on the producer's Q_imp, slot slot_of(l)
             (and different from any other slot's scores, so the slot really matters);
  selection  bit-exact (set, order, count) on the GPU's scores;
  attention  within 2e-2 of oracle.attend over the selected set; layer 0 over all tokens.
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


@pytest.mark.parametrize("L0", [20000])
def test_full_depth_chain_eight_layers(L0):
    import query_aware_sparse_imp_amd as qa
    from query_aware_sparse_imp_amd import control
    w = synthetic.WORKLOADS[4].replace(layers=8)
    L = L0 + 1
    dev = "cuda"
    plan = control.layer_plan(w.layers, w.G)
    print(f"[full-depth] layers={w.layers} G={w.G} L={L} budget {w.budget_num}/{w.budget_den}"
          f" + {w.n_sink} + {w.n_window}", flush=True)
    cap = w.cap(L)
    qimp = {}          # producer layer -> its Q_imp on the GPU [1, Hq, G, 1, d']
    slots_seen = set()
    for role in plan:
        l = role.layer
        assert role.producer == oracle.producer_of(l, w.G) and role.slot == oracle.slot_of(l, w.G)
        assert role.dense == (l == 0)
        if role.produces:
            h = synthetic.producer_hidden(w, l, 1)
            wts = synthetic.producer_weights(w, l)
            q_imp = torch.empty(w.B, w.Hq, w.G, 1, w.dprime, dtype=w.dtype, device=dev)
            qa.butler_produce_queries(h.to(dev), wts["w1"].t().contiguous().to(dev),
                                      wts["w2"].t().contiguous().to(dev), q_imp)
            torch.cuda.synchronize()
            want = oracle.produce_queries(np64(h), np64(wts["w1"]), np64(wts["w2"]), w.Hq, w.G,
                                          w.dprime, 1e-5)
            err = float(np.abs(np64(q_imp) - want).max())
            assert err <= 2e-2, (l, err)
            qimp[l] = q_imp
            print(f"  layer {l}: producer, Q_imp max-abs {err:.2e}", flush=True)
        inp = synthetic.decode_layer(w, l, L=L0, extra=1, with_qimp=False)
        k, v = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
        q, wk = inp["q"].to(dev), inp["w_k"].to(dev)
        out = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
        if role.dense:
            # every token: budget 1/1 whatever the scores hold
            scores = torch.full((w.B, w.Hkv, 1, L), float("nan"), device=dev)
            idx = torch.full((w.B, w.Hkv, 1, L), -1, dtype=torch.int32, device=dev)
            cnt = torch.zeros(w.B, w.Hkv, 1, dtype=torch.int32, device=dev)
            qa.butler_select_attend(scores, 1, 1, w.n_sink, w.n_window, cnt, idx, q, k, v, out,
                                    L=L, softmax_scale=w.scale)
            torch.cuda.synchronize()
            assert (cnt.cpu().numpy() == L).all()
            assert np.array_equal(idx.cpu().numpy()[0, :, 0], np.tile(np.arange(L), (w.Hkv, 1)))
            err = check_attend(out, inp["q"], inp["k_cache"], inp["v_cache"],
                               lambda b, g, i: np.arange(L), w.scale, w.dtype)
            print(f"  layer {l}: dense over {L} tokens, attention max-abs {err:.2e}", flush=True)
            continue
        kimp = torch.zeros(w.B, w.Hkv, L, w.dprime, dtype=w.dtype, device=dev)
        qa.butler_project_keys(k, wk, kimp, 0, L0)
        scores = torch.empty(w.B, w.Hkv, 1, L, dtype=torch.float32, device=dev)
        hist = torch.zeros(w.B, w.Hkv, 1, 2048, dtype=torch.int32, device=dev)
        idx = torch.full((w.B, w.Hkv, 1, cap), -1, dtype=torch.int32, device=dev)
        cnt = torch.zeros(w.B, w.Hkv, 1, dtype=torch.int32, device=dev)
        qa.butler_project_and_score(qimp[role.producer], k, wk, kimp, scores, Hkv=w.Hkv, L=L,
                                    slot=role.slot, radix_hist=hist)
        qa.butler_select_attend(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window, cnt,
                                idx, q, k, v, out, L=L, softmax_scale=w.scale, radix_hist=hist)
        torch.cuda.synchronize()
        assert int(hist.abs().sum()) == 0
        want_row = oracle.project_keys(np64(inp["k_cache"])[:, :, L - 1], np64(inp["w_k"]), "bf16")
        assert np.array_equal(np64(kimp)[:, :, L - 1], want_row), l
        # the oracle's own slot map picks the producer and the slot
        qp = np64(qimp[oracle.producer_of(l, w.G)])                   # [1, Hq, G, 1, d']
        s_or = oracle.slot_of(l, w.G)
        got_s = np64(scores)
        want_s = oracle.score_raw(qp[:, :, s_or], np64(kimp), w.Hkv)
        assert np.array_equal(got_s, want_s), f"layer {l}: raw scores (slot {s_or})"
        for other in range(w.G):
            if other != s_or:
                assert not np.array_equal(got_s, oracle.score_raw(qp[:, :, other], np64(kimp),
                                                                  w.Hkv)), (l, other)
        slots_seen.add(s_or)
        check_select_exact(idx, cnt, got_s, w.budget_num, w.budget_den, w.n_sink, w.n_window)
        ic, cc = idx.cpu().numpy(), cnt.cpu().numpy()
        err = check_attend(out, inp["q"], inp["k_cache"], inp["v_cache"],
                           lambda b, g, i: ic[b, g, i, :cc[b, g, i]], w.scale, w.dtype)
        print(f"  layer {l}: producer {role.producer} slot {role.slot}, selected "
              f"{int(cc.sum())}, attention max-abs {err:.2e}", flush=True)
    assert slots_seen == set(range(w.G))
