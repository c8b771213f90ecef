"""GPU parity of neighbour fetching for the prediction interval (TokenButler arXiv
abstract: prediction interval with neighbor fetching).

Two tests:
  random sets   butler_expand_neighbors on unsorted index lists with repeats and
                out-of-range entries, counts of 0, below, at and above cap_in, at lengths
                of 1 token, a ragged short row, one token past a 2^18-token segment of
                the kernel's LDS bitmask and three segments; widths 0, 1, 3 and 31.  The
                widened sets and their counts must equal the oracle's, bit for bit.
  interval      the raw-scorer Llama-3.1-8B-shaped layer (32/8 heads, 50% + 4 + 64): the
                predictor scores and selects at length L0, then for the next steps of the
                interval the selection is reused, widened by one neighbour on each side
                and by the window at the current length; the widened lists are bit-exact
                and attention over them is within the bf16 bound of the oracle's.
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
    import query_aware_sparse_imp_amd  # noqa: F401  (fails loudly if the library is missing)


def _random_lists(L, cap_in, B, Hkv, seed):
    r = np.random.default_rng(seed)
    idx = np.full((B, Hkv, cap_in), -1, np.int32)
    cnt = np.zeros((B, Hkv), np.int32)
    wanted = [0, cap_in, cap_in + 7, max(1, cap_in // 3), min(cap_in, 5), cap_in - 1]
    for row in range(B * Hkv):
        b, g = divmod(row, Hkv)
        c = max(0, wanted[row % len(wanted)])
        n = min(c, cap_in)
        vals = r.integers(-3, L + 3, size=n)
        if n >= 4:                        # segment edges and the row's own edges
            edge = [0, L - 1, min(L - 1, 262143), min(L - 1, 262144)]
            vals[:4] = edge
        idx[b, g, :n] = vals
        cnt[b, g] = c
    return idx, cnt


@pytest.mark.parametrize("L,width,n_window,cap_in", [
    (1, 0, 0, 4), (777, 1, 64, 200), (262145, 3, 128, 5000), (600000, 31, 128, 3000),
    (5000, 0, 0, 4096)])
def test_expand_random_sets(L, width, n_window, cap_in):
    import query_aware_sparse_imp_amd as qa
    B, Hkv = 2, 3
    print(f"[expand] L={L} width={width} window={n_window} cap_in={cap_in}", flush=True)
    idx_np, cnt_np = _random_lists(L, cap_in, B, Hkv, seed=L + width)
    cap_out = min(L, cap_in * (2 * width + 1) + n_window)
    idx = torch.from_numpy(idx_np).cuda()
    cnt = torch.from_numpy(cnt_np).cuda()
    out = torch.full((B, Hkv, cap_out), -7, dtype=torch.int32, device="cuda")
    cnt_out = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
    qa.butler_expand_neighbors(idx, cnt, out, cnt_out, L=L, width=width, n_window=n_window)
    torch.cuda.synchronize()
    o, co = out.cpu().numpy(), cnt_out.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            n = min(int(cnt_np[b, g]), cap_in)
            want = oracle.expand_neighbors(idx_np[b, g, :n], L, width, n_window)
            assert int(co[b, g]) == len(want), (b, g)
            assert len(want) <= cap_out
            assert np.array_equal(o[b, g, :len(want)], want), (b, g)
            assert (o[b, g, len(want):] == -7).all()           # nothing written past count


def test_prediction_interval_raw_decode():
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2]
    L0, interval, width = 4099, 4, 1
    print(f"[interval] cfg={w.cfg} L0={L0} interval={interval} width={width}", flush=True)
    inp = to_device(synthetic.decode_layer(w, 0, L=L0, extra=interval))
    dev = "cuda"
    kimp = torch.zeros(w.B, w.Hkv, inp["L_cap"], w.dprime, dtype=w.dtype, device=dev)
    qa.butler_project_keys(inp["k_cache_d"], inp["w_k_d"], kimp, 0, L0)
    r = decode_step_gpu(inp, kimp, L0, qa.BUTLER_SCORE_RAW, q_imp=inp["q_imp_d"])
    torch.cuda.synchronize()
    check_select_exact(r["idx"], r["count"], np64(r["scores"]), r["num"], r["den"], w.n_sink,
                       w.n_window)
    idx0 = r["idx"][:, :, 0].contiguous()
    cnt0 = r["count"][:, :, 0].contiguous()
    sel0 = idx0.cpu().numpy()
    c0 = cnt0.cpu().numpy()
    cap_in = idx0.shape[2]
    for s in range(1, interval):
        L = L0 + s
        cap_out = min(L, cap_in * (2 * width + 1) + w.n_window)
        out_idx = torch.empty(w.B, w.Hkv, 1, cap_out, dtype=torch.int32, device=dev)
        out_cnt = torch.empty(w.B, w.Hkv, 1, dtype=torch.int32, device=dev)
        qa.butler_expand_neighbors(idx0, cnt0, out_idx.view(w.B, w.Hkv, cap_out),
                                   out_cnt.view(w.B, w.Hkv), L=L, width=width,
                                   n_window=w.n_window)
        out = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
        qa.butler_sparse_decode_attn(inp["q_d"], inp["k_cache_d"], inp["v_cache_d"], out, L=L,
                                     idx=out_idx, count=out_cnt, softmax_scale=w.scale)
        torch.cuda.synchronize()
        oi, oc = out_idx.cpu().numpy(), out_cnt.cpu().numpy()
        for b in range(w.B):
            for g in range(w.Hkv):
                want = oracle.expand_neighbors(sel0[b, g, :c0[b, g]], L, width, w.n_window)
                assert oc[b, g, 0] == len(want)
                assert np.array_equal(oi[b, g, 0, :len(want)], want)
                assert L - 1 in set(want.tolist())              # the newest token is attended
        err = check_attend(out, inp["q"], inp["k_cache"], inp["v_cache"],
                           lambda b, g, i: oi[b, g, i, :oc[b, g, i]], w.scale, w.dtype)
        print(f"  step {s}: L={L} widened {int(oc.min())}..{int(oc.max())} of "
              f"{int(c0.max())} reused, attention max-abs {err:.3e}", flush=True)
