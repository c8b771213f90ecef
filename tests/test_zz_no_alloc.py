"""GPU test of butler_select_attend_noalloc, the entry point for callers that cannot
allocate: through the C ABI it must give bitwise the idx, count and attention output of
butler_select_attend (the same kernels on a caller workspace) on two calls in a row, the
second with a smaller input, both on the chunked path fused with attention and on the
short-row path (per-row selection, then the separate attention); the sets are also the
oracle's on the same scores and the outputs within 2e-2 of the oracle's attention."""
import numpy as np
import pytest
import torch

import synthetic
from parity import check_attend, check_select_exact, np64, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _call(qa, fn, inp, scores, L, num, den, w, hist):
    cap = min(L, (L * num) // den + w.n_sink + w.n_window)
    idx = torch.full((w.B, w.Hkv, 1, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(w.B, w.Hkv, 1, dtype=torch.int32, device="cuda")
    out = torch.full((w.B, w.Hq, 1, w.D), float("nan"), device="cuda")
    fn(scores, num, den, w.n_sink, w.n_window, cnt, idx, inp["q_d"], inp["k_cache_d"],
       inp["v_cache_d"], out, L=L, softmax_scale=w.scale, radix_hist=hist)
    return idx, cnt, out


def _hist_of(scores):
    """The scorer's first-digit histogram for these scores (order-preserving key >> 21)."""
    B, H, _, L = scores.shape
    bits = scores.view(torch.int32).to(torch.int64) & 0xffffffff
    bits = torch.where(bits == 0x80000000, torch.zeros_like(bits), bits)
    key = torch.where(bits >= 0x80000000, (~bits) & 0xffffffff, bits | 0x80000000)
    h = torch.zeros(B * H, 2048, dtype=torch.int32, device=scores.device)
    h.scatter_add_(1, (key >> 21).view(B * H, L), torch.ones(B * H, L, dtype=torch.int32,
                                                               device=scores.device))
    return h.view(B, H, 1, 2048)


@pytest.mark.parametrize("lengths,num,den,use_hist", [
    ((150001, 30001), 1, 16, False),   # chunked + fused, many candidates; then a shorter row
    ((32768, 9000), 1, 2, True),       # the layer workload's length, then a shorter one
    ((9000, 3001), 1, 2, True),        # the second call takes the short-row path
])
def test_noalloc_matches_select_attend(lengths, num, den, use_hist):
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2]
    for n, L in enumerate(lengths):
        print(f"[noalloc] call {n}: L={L} budget {num}/{den} hist={use_hist}", flush=True)
        inp = to_device(synthetic.decode_layer(w, 7, L=L, with_qimp=False))
        gen = torch.Generator(device="cuda")
        gen.manual_seed(1000 + L)
        scores = torch.randn(w.B, w.Hkv, 1, L, generator=gen, device="cuda")
        a = _call(qa, qa.butler_select_attend, inp, scores, L, num, den, w,
                  _hist_of(scores) if use_hist else None)
        b = _call(qa, qa.butler_select_attend_noalloc, inp, scores, L, num, den, w,
                  _hist_of(scores) if use_hist else None)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), (n, L)
        assert torch.equal(a[2], b[2]), (n, L)
        check_select_exact(b[0], b[1], np64(scores), num, den, w.n_sink, w.n_window)
        ic, cc = b[0].cpu().numpy(), b[1].cpu().numpy()
        err = check_attend(b[2], inp["q"], inp["k_cache"], inp["v_cache"],
                           lambda bb, g, i: ic[bb, g, i, :cc[bb, g, i]], w.scale, w.dtype)
        print(f"  equal to butler_select_attend; attention vs oracle {err:.2e}", flush=True)
