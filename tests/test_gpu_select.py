"""GPU selection against the oracle on hand-made score rows (bit-exact sets).

Covers ties (small-integer scores), -0 versus +0, NaN, +-inf, ragged lengths, budgets of
0, of exactly L and above L, sinks and windows longer than the row, and causal rows whose
length grows with the query position, with both index-list and bitmask outputs; under
both readings of the budget (over every token, or over the tokens outside the sink and
the window).
"""
import numpy as np
import pytest
import torch

import oracle
from parity import bitmask_to_sets

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SPECIAL = np.array([np.nan, -0.0, 0.0, np.inf, -np.inf, 1.0, -1.0], np.float32)


def _scores(rng, shape, kind):
    if kind == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    if kind == "ties":
        return rng.integers(-3, 4, shape).astype(np.float32)
    if kind == "special":
        s = rng.standard_normal(shape).astype(np.float32)
        m = rng.random(shape) < 0.3
        s[m] = SPECIAL[rng.integers(0, len(SPECIAL), int(m.sum()))]
        return s
    if kind == "equal":
        return np.full(shape, 0.5, np.float32)
    raise ValueError(kind)


def _run(scores_np, num, den, ns, nw, causal=False, q_pos0=0, fo=False):
    import query_aware_sparse_imp_amd as qa
    B, Hkv, Lq, L = scores_np.shape
    x = (L * num) // den
    cap = max(1, min(L, x + ns + nw))
    s = torch.from_numpy(scores_np).cuda()
    idx = torch.full((B, Hkv, Lq, cap), -7, dtype=torch.int32, device="cuda")
    bm = torch.zeros((B, Hkv, Lq, (L + 31) // 32), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, Hkv, Lq), dtype=torch.int32, device="cuda")
    qa.butler_select_topk(s, num, den, ns, nw, cnt, idx=idx, bitmask=bm, q_pos0=q_pos0,
                          causal=causal, budget_excludes_forced=fo)
    torch.cuda.synchronize()
    sets = bitmask_to_sets(bm, L)
    cnt_np, idx_np = cnt.cpu().numpy(), idx.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            for i in range(Lq):
                L_r = min(q_pos0 + i + 1, L) if causal else L
                want = oracle.select(scores_np[b, g, i, :L_r].astype(np.float64),
                                     oracle.budget(L_r, num, den), ns, nw, exclude_forced=fo)
                got = idx_np[b, g, i, :cnt_np[b, g, i]]
                assert cnt_np[b, g, i] == len(want), (L, num, den, ns, nw, b, g, i)
                assert np.array_equal(got, want), (L, num, den, ns, nw, b, g, i)
                assert np.array_equal(np.nonzero(sets[b, g, i])[0], want)


@pytest.mark.parametrize("kind", ["normal", "ties", "special", "equal"])
def test_select_rows_match_oracle(kind):
    rng = np.random.default_rng({"normal": 1, "ties": 2, "special": 3, "equal": 4}[kind])
    cases = [(1, 1, 2, 0, 0), (2, 1, 2, 1, 1), (31, 1, 2, 4, 16), (32, 3, 10, 4, 64),
             (33, 1, 16, 4, 128), (100, 0, 1, 3, 5), (257, 1, 1, 4, 16), (700, 1, 2, 4, 64),
             (1000, 5, 4, 0, 0), (1500, 1, 16, 4, 128), (2500, 1, 2, 4, 64),
             (4096, 1, 1, 4, 64), (4097, 1, 2, 4, 64), (8192, 0, 1, 4, 64),
             (12000, 5, 4, 4, 64), (20011, 1, 16, 4, 128), (40000, 3, 10, 4, 64),
             (100003, 1, 2, 0, 0),
             # more than 64 chunks of 4096 keys: few candidates indexed through LDS, and
             # many candidates sorted by coarse bin
             (600000, 1, 2, 4, 64), (300007, 1, 16, 4, 128)]
    for (L, num, den, ns, nw) in cases:
        print(f"[select] kind={kind} L={L} budget={num}/{den} sink={ns} window={nw}", flush=True)
        _run(_scores(rng, (1, 3, 1, L), kind), num, den, ns, nw)


@pytest.mark.parametrize("kind", ["normal", "ties", "special", "equal"])
@pytest.mark.parametrize("fo", [False, True])
def test_select_many_rows_match_oracle(kind, fo):
    """Calls with several query rows of up to 8192 tokens (one wave per row): every row
    length class, budgets of 0, below and at or above the pool, a row count that leaves a
    workgroup part-filled, and rows whose bitmask ends inside a 64-word store."""
    rng = np.random.default_rng({"normal": 41, "ties": 42, "special": 43, "equal": 44}[kind]
                                + (10 if fo else 0))
    cases = [(1, 1, 2, 0, 0), (31, 1, 2, 4, 16), (64, 3, 10, 4, 64), (65, 1, 16, 4, 128),
             (1000, 0, 1, 3, 5), (1024, 1, 2, 4, 64), (1025, 1, 1, 4, 16),
             (2048, 5, 4, 4, 64), (3000, 1, 2, 4, 64), (5000, 1, 16, 4, 128),
             (6200, 9, 10, 64, 1000), (8191, 1, 2, 4, 64), (8192, 1, 2, 4, 64)]
    for (L, num, den, ns, nw) in cases:
        print(f"[select-rows] kind={kind} fo={fo} L={L} budget={num}/{den} sink={ns} "
              f"window={nw}", flush=True)
        _run(_scores(rng, (1, 2, 3, L), kind), num, den, ns, nw, fo=fo)


def test_select_causal_rows():
    rng = np.random.default_rng(5)
    # row lengths in every per-row workgroup shape: 64 to 1024 threads, 4 to 64 keys each
    for (Lq, q_pos0, L) in ((37, 100, 137), (64, 0, 64), (40, 500, 540), (129, 1000, 1129),
                            (70, 2000, 2070), (40, 4500, 4540), (64, 6000, 6064),
                            (30, 7000, 7030), (33, 8159, 8192), (9, 16000, 16009),
                            (5, 30000, 30005), (3, 65533, 65536)):
        print(f"[select-causal] Lq={Lq} q_pos0={q_pos0} L={L}", flush=True)
        _run(_scores(rng, (2, 2, Lq, L), "ties"), 1, 2, 4, 64, causal=True, q_pos0=q_pos0)
        _run(_scores(rng, (1, 2, Lq, L), "normal"), 1, 2, 4, 64, causal=True, q_pos0=q_pos0)


@pytest.mark.parametrize("kind", ["normal", "ties", "special", "equal"])
def test_select_rows_excluding_forced_match_oracle(kind):
    """The budget counts only the tokens outside the sink and the window (|S| = x + |F| when
    the middle holds x tokens): the per-row kernel and the chunked schedule."""
    rng = np.random.default_rng({"normal": 31, "ties": 32, "special": 33, "equal": 34}[kind])
    cases = [(1, 1, 2, 4, 16), (31, 1, 2, 4, 16), (100, 0, 1, 3, 5), (257, 1, 1, 4, 16),
             (300, 9, 10, 4, 64), (4096, 1, 2, 4, 64), (4097, 1, 2, 4, 64),
             (20011, 1, 16, 4, 128), (40000, 3, 10, 64, 1000), (100003, 1, 2, 0, 0)]
    for (L, num, den, ns, nw) in cases:
        print(f"[select-excl] kind={kind} L={L} budget={num}/{den} sink={ns} window={nw}",
              flush=True)
        _run(_scores(rng, (1, 3, 1, L), kind), num, den, ns, nw, fo=True)


def test_select_causal_rows_excluding_forced():
    rng = np.random.default_rng(35)
    for (Lq, q_pos0, L) in ((37, 100, 137), (129, 1000, 1129)):
        print(f"[select-causal-excl] Lq={Lq} q_pos0={q_pos0} L={L}", flush=True)
        _run(_scores(rng, (1, 2, Lq, L), "ties"), 1, 2, 4, 64, causal=True, q_pos0=q_pos0,
             fo=True)


def test_select_workspace_shared_across_budgets():
    """One workspace, passed through the C entry point to calls of one shape with budgets
    that alternate between few candidates per row (50%: chunk regions in wave order) and
    many (1/16: regions sorted by coarse bin, with the double-buffered coarse histogram):
    the per-row state the chunk kernels keep in the workspace carries over from call to
    call, and every call's sets equal the oracle's."""
    import ctypes
    import query_aware_sparse_imp_amd as qa
    rng = np.random.default_rng(77)
    L, ns, nw = 300007, 4, 128
    s_np = rng.standard_normal((1, 3, 1, L)).astype(np.float32)
    s_np[0, 2, 0, ::7] = 1.5     # a flood of equal keys at the 1/16 threshold, ties cut by index
    s = torch.from_numpy(s_np).cuda()
    idx = torch.empty((1, 3, 1, L), dtype=torch.int32, device="cuda")
    cnt = torch.empty((1, 3, 1), dtype=torch.int32, device="cuda")
    budgets = [(1, 2), (1, 16), (1, 16), (1, 2), (1, 16), (3, 10), (1, 2), (1, 16)]

    def args(num, den):
        return (qa._ptr(s), None, None, num, den, ns, nw, 0, qa._ptr(idx), None, qa._ptr(cnt),
                1, 3, 1, L, L, 0, 0)
    need = max(qa.workspace_bytes(
        lambda ws, n, a=args(num, den): qa.lib.butler_select_topk(qa._stream(None), *a, ws, n))
        for (num, den) in budgets)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    nbytes = ctypes.c_size_t(need)
    for call, (num, den) in enumerate(budgets):
        print(f"[select-shared-ws] call {call} budget {num}/{den} L={L}", flush=True)
        idx.fill_(-7)
        cnt.zero_()
        rc = qa.lib.butler_select_topk(qa._stream(None), *args(num, den), ws.data_ptr(),
                                       ctypes.byref(nbytes))
        assert rc == 0, rc
        torch.cuda.synchronize()
        cnt_np, idx_np = cnt.cpu().numpy(), idx.cpu().numpy()
        for g in range(3):
            want = oracle.select(s_np[0, g, 0].astype(np.float64), oracle.budget(L, num, den),
                                 ns, nw)
            assert cnt_np[0, g, 0] == len(want), (call, num, den, g)
            assert np.array_equal(idx_np[0, g, 0, :cnt_np[0, g, 0]], want), (call, num, den, g)


@pytest.mark.parametrize("num,den", [(1, 2), (1, 16)])
def test_select_longest_row(num, den):
    """The longest decode row the chunked schedule takes (8388608 keys: 2048 chunks of 4096,
    the most the finishing pass indexes), with few (50%) and many (1/16) candidates."""
    rng = np.random.default_rng(8 + den)
    L = 8388608
    print(f"[select-longest] L={L} budget={num}/{den}", flush=True)
    _run(rng.standard_normal((1, 1, 1, L)).astype(np.float32), num, den, 4, 128)
