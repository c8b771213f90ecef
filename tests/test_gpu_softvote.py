"""GPU parity of the soft-voting decode path (TokenSelect scorer).

Batched decode: B sequences, 32 query / 8 KV heads, D=128, keys from a 95% N(0,1) /
5% clustered mixture, queries a random walk (sigma 0.05) over steps, 30% budget +
sink 4 + window 64.  Scores are gated at 1e-5 relative, selection bit-exact on the
GPU's scores, attention 2e-2 max-abs on the GPU's index lists.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import check_attend, check_select_exact, decode_step_gpu, np64, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _softvote_case(w, steps_to_check):
    import query_aware_sparse_imp_amd as qa
    print(f"[softvote] B={w.B} L={w.L} steps={steps_to_check}", flush=True)
    cache = synthetic.softvote_cache(w)
    qs = synthetic.softvote_queries(w, max(steps_to_check) + 1)
    inp = {"workload": w, "k_cache": cache["k_cache"], "v_cache": cache["v_cache"]}
    to_device(inp)
    kn, vn = np64(cache["k_cache"]), np64(cache["v_cache"])
    for s in steps_to_check:
        inp["q"] = qs[s]
        inp["q_d"] = qs[s].cuda()
        r = decode_step_gpu(inp, None, w.L, qa.BUTLER_SCORE_SOFTVOTE)
        torch.cuda.synchronize()
        got = np64(r["scores"])
        qn = np64(qs[s])
        worst = 0.0
        for b in range(w.B):
            for g in range(w.Hkv):
                want = oracle.score_softvote(qn[b:b + 1, g * w.R:(g + 1) * w.R],
                                             kn[b:b + 1, g:g + 1], 1, w.scale)[0, 0, 0]
                err = np.abs(got[b, g, 0] - want)
                assert (err <= 1e-5 * np.abs(want) + 1e-30).all(), (s, b, g, float(err.max()))
                worst = max(worst, float((err / np.maximum(np.abs(want), 1e-30)).max()))
                assert abs(got[b, g, 0].sum() - w.R) < 1e-3
        print(f"  step {s}: max relative score error {worst:.2e}", flush=True)
        check_select_exact(r["idx"], r["count"], got, w.budget_num, w.budget_den, w.n_sink,
                           w.n_window)
        idx, cnt = r["idx"].cpu().numpy(), r["count"].cpu().numpy()
        check_attend(r["out"], qs[s], cache["k_cache"], cache["v_cache"],
                     lambda b, g, i: idx[b, g, i, :cnt[b, g, i]], w.scale, w.dtype)


def test_softvote_ragged():
    w = synthetic.WORKLOADS[3].replace(B=2, L=3001)
    _softvote_case(w, [0, 1])


def test_softvote_full_size():
    w = synthetic.WORKLOADS[3]
    _softvote_case(w, [0, 1, 63])
