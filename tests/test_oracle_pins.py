"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against an independent fact: exact
rational arithmetic (``fractions.Fraction``) with its own round-to-nearest-
even, brute-force enumeration of subsets, a library routine that the oracle
does not call (torch's layer_norm / softmax / scaled_dot_product_attention,
torch's float32 -> bfloat16 conversion), a golden table derived from the
pages, or an invariant of the definition.  The mutation tests at the end
plant plausible mistakes in the oracle and check that these pins catch them.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import reference as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent exact rounding (Fraction based)
# ---------------------------------------------------------------------------

def frac_rne(fr: Fraction, p: int, emin: int = -126) -> float:
    """Round an exact rational to the binary format with p significant bits
    and minimum normal exponent emin, ties to even (no overflow handling)."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, emin) - (p - 1))
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * ulp)


def bf16_grid(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).double().numpy()


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_on_structured_float32_patterns():
    """All 2^16 upper halves x the lower halves that decide the rounding."""
    hi = np.arange(1 << 16, dtype=np.uint64) << np.uint64(16)
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF,
                     0x1234, 0x9ABC], dtype=np.uint64)
    bits = (hi[:, None] | lows[None, :]).ravel().astype(np.uint32)
    f = bits.view(np.float32)
    ours = ref.round_to_bf16(f.astype(np.float64))
    theirs = torch.from_numpy(f.copy()).to(torch.bfloat16).double().numpy()
    both_nan = np.isnan(ours) & np.isnan(theirs)
    assert np.all((ours == theirs) | both_nan)
    # sign of zero is kept
    z = np.signbit(ours[(ours == 0)]) == np.signbit(theirs[(theirs == 0)])
    assert z.all()


def test_bf16_rounding_random_float32_sample():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    ours = ref.round_to_bf16(f.astype(np.float64))
    theirs = torch.from_numpy(f.copy()).to(torch.bfloat16).double().numpy()
    assert np.all((ours == theirs) | (np.isnan(ours) & np.isnan(theirs)))


def test_bf16_single_rounding_golden():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "bf16_single_rounding.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for src, want, note in rows:
        got = ref.round_to_bf16(np.array([float.fromhex(src)]))[0]
        assert got == float.fromhex(want), (src, want, note, got.hex())


def test_bf16_rounding_of_float64_matches_exact_rationals():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))
    # plant exact ties and near-ties in float64 (below float32 resolution)
    base = ref.round_to_bf16(x[:1000])
    ulp = np.exp2(np.frexp(base)[1] - 8)
    x[:1000] = base + ulp / 2 * np.sign(base) + rng.choice([-1, 0, 1], 1000) * np.abs(base) * 2.0 ** -45
    got = ref.round_to_bf16(x)
    for xi, gi in zip(x, got):
        assert gi == frac_rne(Fraction(float(xi)), 8), (xi.hex(), gi)


def test_f32_rounding_matches_exact_rationals():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(2000) * np.exp2(rng.integers(-30, 30, 2000))
    got = ref.round_to_f32(x)
    for xi, gi in zip(x, got):
        assert gi == frac_rne(Fraction(float(xi)), 24), xi.hex()


# ---------------------------------------------------------------------------
# layer norm and producer
# ---------------------------------------------------------------------------

def test_layer_norm_matches_torch():
    rng = np.random.default_rng(5)
    h = rng.standard_normal((3, 7, 64)) * 3 + 1.5
    ours = ref.layer_norm(h, 1e-5)
    theirs = torch.nn.functional.layer_norm(torch.from_numpy(h), (64,), eps=1e-5).numpy()
    np.testing.assert_allclose(ours, theirs, rtol=0, atol=1e-12)


def test_produce_queries_matches_exact_mlp_and_layout():
    """f_theta = relu(x W1) W2 with bf16 storage of x, a and y, checked with
    exact rationals; the output layout is checked element by element."""
    rng = np.random.default_rng(6)
    B, Lq, E, F, Hq, G, dp = 2, 3, 8, 5, 3, 2, 2
    h = bf16_grid(rng, (B, Lq, E), 2.0)
    w1 = bf16_grid(rng, (E, F), 0.3)
    w2 = bf16_grid(rng, (F, Hq * G * dp), 0.3)
    got = ref.produce_queries(h, w1, w2, Hq, G, dp, eps=1e-5)
    assert got.shape == (B, Hq, G, Lq, dp)
    xhat = torch.nn.functional.layer_norm(torch.from_numpy(h), (E,), eps=1e-5).numpy()
    for b in range(B):
        for t in range(Lq):
            x = [frac_rne(Fraction(float(v)), 8) for v in xhat[b, t]]
            a = []
            for f in range(F):
                acc = sum(Fraction(x[e]) * Fraction(float(w1[e, f])) for e in range(E))
                a.append(frac_rne(max(acc, Fraction(0)), 8))
            for col in range(Hq * G * dp):
                y = frac_rne(sum(Fraction(a[f]) * Fraction(float(w2[f, col])) for f in range(F)), 8)
                head, rem = divmod(col, G * dp)
                slot, i = divmod(rem, dp)
                assert got[b, head, slot, t, i] == y, (b, t, col)


def test_slot_map_golden():
    rows = [list(map(int, ln.split())) for ln in open(os.path.join(GOLDEN, "slot_map_g4.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 32
    for layer, producer, slot, dense in rows:
        assert ref.producer_of(layer, 4) == producer
        assert ref.slot_of(layer, 4) == slot
        assert (layer == 0) == bool(dense)


def test_fixed_pc_policy_golden():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "fixed_pc_policy.txt"))
            if ln.strip() and not ln.startswith("#")]
    for policy, num, den, L, x in rows:
        assert ref.fixed_pc_fraction(policy) == (int(num), int(den))
        assert ref.budget(int(L), int(num), int(den)) == int(x)


# ---------------------------------------------------------------------------
# projection and scores
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,p", [("bf16", 8), ("f32", 24)])
def test_project_keys_matches_exact_rationals(dtype, p):
    rng = np.random.default_rng(8)
    D, dp, n = 16, 5, 7                      # non-square: a transposed W_K fails
    if dtype == "bf16":
        k = bf16_grid(rng, (n, D)); w = bf16_grid(rng, (D, dp), 0.25)
    else:
        k = rng.standard_normal((n, D)).astype(np.float32).astype(np.float64)
        w = (rng.standard_normal((D, dp)) * 0.25).astype(np.float32).astype(np.float64)
    got = ref.project_keys(k, w, dtype)
    for t in range(n):
        for j in range(dp):
            exact = sum(Fraction(float(k[t, d])) * Fraction(float(w[d, j])) for d in range(D))
            assert got[t, j] == frac_rne(exact, p), (t, j)


def test_score_raw_matches_exact_group_sums_and_causal_mask():
    rng = np.random.default_rng(9)
    B, Hkv, R, Lq, L, dp = 2, 3, 2, 3, 9, 4
    Hq = Hkv * R
    q = bf16_grid(rng, (B, Hq, Lq, dp))
    k = bf16_grid(rng, (B, Hkv, L, dp))
    got = ref.score_raw(q, k, Hkv, causal=True, q_pos0=4)
    for b in range(B):
        for g in range(Hkv):
            for i in range(Lq):
                for t in range(L):
                    if t > 4 + i:
                        assert got[b, g, i, t] == -np.inf
                        continue
                    exact = sum(Fraction(float(q[b, h, i, j])) * Fraction(float(k[b, g, t, j]))
                                for h in range(g * R, (g + 1) * R) for j in range(dp))
                    assert got[b, g, i, t] == frac_rne(exact, 24), (b, g, i, t)
    nc = ref.score_raw(q, k, Hkv)
    assert np.isfinite(nc).all()


def test_score_raw_bf16_sum_is_order_independent():
    """For bf16 inputs every partial sum is exact in float64, so any order of
    summation gives the same float64 value (the score is exactly rounded)."""
    rng = np.random.default_rng(10)
    q = bf16_grid(rng, (4, 32))
    k = bf16_grid(rng, (20000, 32))
    qbar = q.sum(axis=0)
    a = k @ qbar
    b = np.zeros(20000)
    for j in reversed(range(32)):
        b += k[:, j] * qbar[j]
    assert np.array_equal(a, b)


def test_softvote_reduces_to_softmax_and_sums_to_group_size():
    rng = np.random.default_rng(11)
    B, Hkv, R, Lq, L, D = 1, 2, 2, 2, 50, 16
    q = bf16_grid(rng, (B, Hkv * R, Lq, D))
    q[:, 0:R] = 0.0                            # group 0: all-zero queries -> uniform
    k = bf16_grid(rng, (B, Hkv, L, D))
    s = ref.score_softvote(q, k, Hkv, 0.25)
    np.testing.assert_allclose(s.sum(axis=-1), R, rtol=0, atol=1e-5)
    np.testing.assert_allclose(s[0, 0], R / L, rtol=1e-7)
    # R = 1 is a plain softmax of the scaled logits (torch)
    s1 = ref.score_softvote(q[:, 2:3], k[:, 1:2], 1, 0.25)
    z = torch.from_numpy(q[0, 2] @ k[0, 1].T * 0.25)
    want = torch.softmax(z, dim=-1).float().double().numpy()
    np.testing.assert_array_equal(s1[0, 0], want)
    # group 1 = sum of its two heads' softmaxes
    z2 = torch.from_numpy(q[0, 3] @ k[0, 1].T * 0.25)
    want2 = (torch.softmax(z, -1) + torch.softmax(z2, -1)).float().double().numpy()
    np.testing.assert_array_equal(s[0, 1], want2)


def test_softvote_causal_rows_normalise_over_prefix():
    rng = np.random.default_rng(12)
    q = bf16_grid(rng, (1, 2, 4, 8))
    k = bf16_grid(rng, (1, 1, 10, 8))
    s = ref.score_softvote(q, k, 1, 0.3, causal=True, q_pos0=3)
    for i in range(4):
        n = 3 + i + 1
        assert np.all(s[0, 0, i, n:] == -np.inf)
        assert abs(s[0, 0, i, :n].sum() - 2.0) < 1e-6


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def _dominates(s, t, u):
    a, b = s[t], s[u]
    a = -np.inf if np.isnan(a) else a
    b = -np.inf if np.isnan(b) else b
    return a > b or (a == b and t < u)


def brute_select(s, x, n_sink, n_window):
    L = len(s)
    k = min(x, L)
    winners = []
    for T in itertools.combinations(range(L), k):
        Ts = set(T)
        if all(_dominates(s, t, u) for t in Ts for u in range(L) if u not in Ts):
            winners.append(Ts)
    assert len(winners) == 1
    S = winners[0] | set(range(min(n_sink, L))) | set(range(max(0, L - n_window), L))
    return sorted(S)


def brute_max_sum(s, x):
    """Top-x as the max-sum subset, lexicographically smallest on ties."""
    best = None
    for T in itertools.combinations(range(len(s)), x):
        key = (-sum(s[t] for t in T), T)
        if best is None or key < best:
            best = key
    return sorted(best[1])


def test_select_matches_brute_force_enumeration():
    rng = np.random.default_rng(13)
    vals = np.array([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0, np.inf, -np.inf, np.nan])
    for trial in range(250):
        L = int(rng.integers(1, 12))
        s = vals[rng.integers(0, len(vals), L)] if trial % 2 else rng.standard_normal(L)
        x = int(rng.integers(0, L + 2))
        ns, nw = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        got = ref.select(s, x, ns, nw).tolist()
        assert got == brute_select(s, x, ns, nw), (s, x, ns, nw)
        if trial % 2 == 0 and 0 < x <= L:
            assert ref.select(s, x, 0, 0).tolist() == brute_max_sum(s, x)


def test_select_invariants():
    rng = np.random.default_rng(14)
    L = 500
    s = rng.standard_normal(L)
    for x in (0, 1, 10, 250, 499):
        S = set(ref.select(s, x, 4, 16).tolist())
        assert set(range(4)) <= S and set(range(L - 16, L)) <= S
        assert max(x, 20) <= len(S) <= min(L, x + 20)
        assert set(ref.select(s, x, 4, 16)) <= set(ref.select(s, x + 1, 4, 16))
    assert ref.select(s, L, 4, 16).tolist() == list(range(L))
    assert ref.select(s, 10 * L, 0, 0).tolist() == list(range(L))
    eq = np.full(L, 0.25)
    assert ref.select(eq, 30, 4, 16).tolist() == sorted(set(range(30)) | set(range(L - 16, L)))
    # positive scaling of the scores never changes the set
    assert ref.select(s * 3.5, 123, 4, 16).tolist() == ref.select(s, 123, 4, 16).tolist()


def brute_select_excluding_forced(s, x, n_sink, n_window):
    """Budget over the middle tokens only: the unique size-min(x, |M|) subset of the middle
    tokens M whose members all dominate every other middle token, plus sink and window."""
    L = len(s)
    F = set(range(min(n_sink, L))) | set(range(max(0, L - n_window), L))
    M = [t for t in range(L) if t not in F]
    k = min(x, len(M))
    winners = []
    for T in itertools.combinations(M, k):
        Ts = set(T)
        if all(_dominates(s, t, u) for t in Ts for u in M if u not in Ts):
            winners.append(Ts)
    assert len(winners) == 1
    return sorted(winners[0] | F)


def test_select_excluding_forced_matches_brute_force_and_invariants():
    """The other reading of the budget (the sink and the window are outside it): brute-force
    enumeration over the middle tokens, |S| = min(x, |M|) + |F|, no sink or window means the
    default reading, and a forced token that would have won a budget place frees it."""
    rng = np.random.default_rng(23)
    vals = np.array([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0, np.inf, -np.inf, np.nan])
    for trial in range(250):
        L = int(rng.integers(1, 12))
        sc = vals[rng.integers(0, len(vals), L)] if trial % 2 else rng.standard_normal(L)
        x = int(rng.integers(0, L + 2))
        ns, nw = int(rng.integers(0, 4)), int(rng.integers(0, 4))
        got = ref.select(sc, x, ns, nw, exclude_forced=True).tolist()
        assert got == brute_select_excluding_forced(sc, x, ns, nw), (sc, x, ns, nw)
        F = set(range(min(ns, L))) | set(range(max(0, L - nw), L))
        assert len(got) == min(x, L - len(F)) + len(F)
        assert ref.select(sc, x, 0, 0, exclude_forced=True).tolist() == ref.select(sc, x, 0, 0).tolist()
    # the two readings differ exactly when forced tokens take budget places
    sc = np.array([9.0, 8.0, 1.0, 2.0, 3.0, 4.0, 7.0])
    assert ref.select(sc, 2, 1, 1).tolist() == [0, 1, 6]            # token 0 used a place
    assert ref.select(sc, 2, 1, 1, exclude_forced=True).tolist() == [0, 1, 5, 6]


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def test_attend_matches_sdpa_dense_and_masked():
    rng = np.random.default_rng(15)
    R, n, D = 4, 37, 32
    q = rng.standard_normal((R, D)); k = rng.standard_normal((n, D)); v = rng.standard_normal((n, D))
    scale = 1 / math.sqrt(D)
    got = ref.attend(q, k, v, scale)
    Q, K, V = (torch.from_numpy(a)[None, None] for a in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(
        Q[0].unsqueeze(0), K.expand(1, 1, n, D), V.expand(1, 1, n, D), scale=scale)[0, 0].numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    mask = rng.random(n) < 0.4
    mask[0] = True
    idx = np.nonzero(mask)[0]
    got_m = ref.attend(q, k[idx], v[idx], scale)
    want_m = torch.nn.functional.scaled_dot_product_attention(
        Q[0].unsqueeze(0), K, V, attn_mask=torch.from_numpy(mask)[None, None, None, :],
        scale=scale)[0, 0].numpy()
    np.testing.assert_allclose(got_m, want_m, rtol=0, atol=1e-12)


def test_attend_special_cases():
    rng = np.random.default_rng(16)
    k = rng.standard_normal((9, 8)); v = rng.standard_normal((9, 8))
    q = rng.standard_normal((2, 8))
    assert np.array_equal(ref.attend(q, k[3:4], v[3:4], 0.5), np.repeat(v[3:4], 2, axis=0))
    np.testing.assert_allclose(ref.attend(np.zeros((1, 8)), k, v, 0.5)[0], v.mean(axis=0),
                               rtol=0, atol=1e-15)


def test_gqa_head_to_kv_head_map():
    """Query head h reads KV head h // R (consecutive groups)."""
    rng = np.random.default_rng(17)
    B, Hq, Hkv, L, D = 1, 4, 2, 6, 4
    k = rng.standard_normal((B, Hkv, L, D)); v = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, Hq, D))
    sel = [[np.array([2]), np.array([5])]]
    out = ref.sparse_decode_attn(q, k, v, sel, 0.5)
    for h in range(Hq):
        g = h // 2
        assert np.array_equal(out[0, h], v[0, g, sel[0][g][0]])


# ---------------------------------------------------------------------------
# selection heads (sel_group query heads share one selected set)
# ---------------------------------------------------------------------------

def _sel_heads_by_hand(Hq, Hkv, gs):
    """[(query heads, KV head)] of every selection head, listed one by one."""
    R = Hq // Hkv
    out = []
    for j in range(Hq // gs):
        heads = [j * gs + r for r in range(gs)]
        kvs = {h // R for h in heads}
        assert len(kvs) == 1                       # a selection head never spans KV heads
        out.append((heads, kvs.pop()))
    return out


@pytest.mark.parametrize("Hq,Hkv,gs", [(6, 3, 1), (8, 2, 2), (8, 2, 1), (8, 2, 4)])
def test_score_raw_per_selection_head_matches_exact_dots(Hq, Hkv, gs):
    """Raw scores of each selection head: the exact dot product of its own query heads'
    summed Q_imp with its KV head's K_imp (Fraction arithmetic, rounded once)."""
    rng = np.random.default_rng(40 + gs)
    B, Lq, L, dp = 2, 2, 7, 4
    q = bf16_grid(rng, (B, Hq, Lq, dp))
    k = bf16_grid(rng, (B, Hkv, L, dp))
    got = ref.score_raw(q, k, Hkv, sel_group=gs)
    groups = _sel_heads_by_hand(Hq, Hkv, gs)
    assert got.shape == (B, len(groups), Lq, L)
    for b in range(B):
        for j, (heads, kv) in enumerate(groups):
            for i in range(Lq):
                for t in range(L):
                    exact = sum(Fraction(float(q[b, h, i, c])) * Fraction(float(k[b, kv, t, c]))
                                for h in heads for c in range(dp))
                    assert got[b, j, i, t] == frac_rne(exact, 24), (b, j, i, t)
    if gs == Hq // Hkv:
        assert np.array_equal(got, ref.score_raw(q, k, Hkv))    # the default grouping


def test_softvote_per_query_head_is_each_heads_softmax():
    """sel_group = 1: the soft-voting score of query head h is h's own softmax over the
    keys of KV head h // R (torch softmax), and it ranks tokens as h's logits do."""
    rng = np.random.default_rng(44)
    B, Hq, Hkv, L, D = 1, 4, 2, 30, 8
    q = bf16_grid(rng, (B, Hq, 1, D))
    k = bf16_grid(rng, (B, Hkv, L, D))
    s = ref.score_softvote(q, k, Hkv, 0.35, sel_group=1)
    assert s.shape == (B, Hq, 1, L)
    for h in range(Hq):
        z = torch.from_numpy(q[0, h, 0] @ k[0, h // 2].T * 0.35)
        np.testing.assert_array_equal(s[0, h, 0], torch.softmax(z, -1).float().double().numpy())
        order_s = np.lexsort((np.arange(L), -s[0, h, 0]))
        order_z = np.lexsort((np.arange(L), -z.numpy()))
        assert np.array_equal(order_s, order_z)
    # two heads per set: the sum of the two softmaxes
    s2 = ref.score_softvote(q, k, Hkv, 0.35, sel_group=2)
    np.testing.assert_allclose(s2[0, :, 0].sum(-1), 2.0, atol=1e-6)


def test_attention_per_selection_head_matches_masked_sdpa():
    """Every query head attends over its own selection head's set: torch's
    scaled_dot_product_attention with a per-head boolean mask gives the same output
    (decode rows, and prefill rows through masked_attention_rows)."""
    rng = np.random.default_rng(45)
    B, Hq, Hkv, L, D = 2, 8, 2, 24, 8
    k = rng.standard_normal((B, Hkv, L, D)); v = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, Hq, D))
    for gs in (1, 2):
        Hs = Hq // gs
        sel = [[np.sort(rng.choice(L, size=int(rng.integers(1, L)), replace=False))
                for _ in range(Hs)] for _ in range(B)]
        got = ref.sparse_decode_attn(q, k, v, sel, 0.3, sel_group=gs)
        mask = torch.zeros(B, Hq, 1, L, dtype=torch.bool)
        for b in range(B):
            for h in range(Hq):
                mask[b, h, 0, sel[b][h // gs]] = True
        K = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
        V = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1))
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[:, :, None, :], K, V, attn_mask=mask, scale=0.3)[:, :, 0]
        np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-12)
        rows = ref.masked_attention_rows(q[:, :, None, :], k, v,
                                         [[[sel[b][j]] for j in range(Hs)] for b in range(B)],
                                         0.3, sel_group=gs)
        for (b, h, i), o in rows.items():
            np.testing.assert_allclose(o, want[b, h].numpy(), rtol=0, atol=1e-12)


def test_selection_cache_per_query_head():
    """sel_group = 1: one cosine per query head (numpy's norm and dot on each head)."""
    rng = np.random.default_rng(46)
    a = rng.standard_normal((2, 4, 8)); c = rng.standard_normal((2, 4, 8))
    c[1, 2] = a[1, 2] * 2.0                         # this head is kept at any threshold <= 1
    keep, new_ref, cos = oracle.selection_cache(a, c, 2, 0.999, sel_group=1)
    want = np.array([[np.dot(a[b, h], c[b, h]) / (np.linalg.norm(a[b, h]) * np.linalg.norm(c[b, h]))
                      for h in range(4)] for b in range(2)])
    assert cos.shape == (2, 4) and np.allclose(cos, want, rtol=0, atol=1e-15)
    assert keep[1, 2] and keep.sum() == 1
    assert np.array_equal(new_ref[1, 2], c[1, 2]) and np.array_equal(new_ref[0], a[0])


def test_decode_step_per_query_head_sets_differ_and_contain_forced():
    """Per-query-head selection on a layer whose two heads of a group prefer different
    tokens: the two sets differ, each holds its sink and window, and the group's shared
    set (the default) is neither of them."""
    d = _tiny_layer(seed=47, L=48)
    d["qi"][0, 1] = -d["qi"][0, 0]                # head 1 ranks in the reverse order of head 0
    kimp = ref.project_keys(d["k"], d["wk"], "bf16")
    kw = dict(q=d["q"], k_cache=d["k"], v_cache=d["v"], L=48, num=1, den=4, n_sink=2,
              n_window=3, scale=0.25, Hkv=d["Hkv"], mode="raw", q_imp_slot=d["qi"], kimp=kimp)
    per = ref.decode_layer_step(sel_group=1, **kw)
    grp = ref.decode_layer_step(**kw)
    s0, s1 = set(per["sel"][0][0].tolist()), set(per["sel"][0][1].tolist())
    assert s0 != s1
    for S in (s0, s1):
        assert {0, 1, 45, 46, 47} <= S and 12 <= len(S) <= 17
    assert set(grp["sel"][0][0].tolist()) not in (s0, s1)
    assert per["scores"].shape == (1, 4, 48) and grp["scores"].shape == (1, 2, 48)


# ---------------------------------------------------------------------------
# whole decode step: invariants the method's definition fixes
# ---------------------------------------------------------------------------

def _tiny_layer(seed=18, L=40, Hq=4, Hkv=2, D=16, dp=8):
    rng = np.random.default_rng(seed)
    return dict(q=bf16_grid(rng, (1, Hq, D)), k=bf16_grid(rng, (1, Hkv, L, D)),
                v=bf16_grid(rng, (1, Hkv, L, D)), qi=bf16_grid(rng, (1, Hq, dp)),
                wk=bf16_grid(rng, (D, dp), 0.25), L=L, Hkv=Hkv, D=D)


def _sdpa_dense(q, k, v, Hkv, scale):
    R = q.shape[1] // Hkv
    Q = torch.from_numpy(q)[:, :, None, :]
    K = torch.from_numpy(np.repeat(k, R, axis=1)); V = torch.from_numpy(np.repeat(v, R, axis=1))
    return torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[:, :, 0].numpy()


@pytest.mark.parametrize("mode", ["raw", "softvote"])
def test_full_budget_equals_dense_attention(mode):
    d = _tiny_layer()
    kimp = ref.project_keys(d["k"], d["wk"], "bf16")
    scale = 1 / math.sqrt(d["D"])
    for num, den in ((1, 1), (3, 2)):
        r = ref.decode_layer_step(q=d["q"], k_cache=d["k"], v_cache=d["v"], L=d["L"], num=num,
                                  den=den, n_sink=2, n_window=3, scale=scale, Hkv=d["Hkv"],
                                  mode=mode, q_imp_slot=d["qi"], kimp=kimp)
        np.testing.assert_allclose(r["out"], _sdpa_dense(d["q"], d["k"], d["v"], d["Hkv"], scale),
                                   rtol=0, atol=1e-12)


def test_sink_and_window_always_selected():
    d = _tiny_layer(L=64)
    kimp = ref.project_keys(d["k"], d["wk"], "bf16")
    r = ref.decode_layer_step(q=d["q"], k_cache=d["k"], v_cache=d["v"], L=64, num=1, den=8,
                              n_sink=4, n_window=8, scale=0.25, Hkv=d["Hkv"], mode="raw",
                              q_imp_slot=d["qi"], kimp=kimp)
    for g in range(d["Hkv"]):
        S = set(r["sel"][0][g].tolist())
        assert set(range(4)) | set(range(56, 64)) <= S
        assert 8 <= len(S) <= 20


# ---------------------------------------------------------------------------
# mutation checks: plausible mistakes in the oracle must fail a pin
# ---------------------------------------------------------------------------

def _pins_fail(monkeypatch, name, bad, test):
    monkeypatch.setattr(ref, name, bad)
    with pytest.raises(AssertionError):
        test()


def test_mutations_are_caught(monkeypatch):
    good_select = ref.select

    def select_ties_high(s, x, ns, nw):      # ties to the higher index
        s = np.asarray(s, np.float64)
        L = len(s)
        order = np.lexsort((-np.arange(L), -np.nan_to_num(s, nan=-np.inf)))[:min(x, L)]
        return np.unique(np.concatenate([order, np.arange(min(ns, L)),
                                         np.arange(max(0, L - nw), L)]))
    _pins_fail(monkeypatch, "select", select_ties_high, test_select_matches_brute_force_enumeration)
    monkeypatch.setattr(ref, "select", good_select)

    def select_no_window(s, x, ns, nw):
        return good_select(s, x, ns, 0)
    _pins_fail(monkeypatch, "select", select_no_window, test_select_invariants)
    monkeypatch.setattr(ref, "select", good_select)

    good_rb = ref.round_to_bf16
    _pins_fail(monkeypatch, "round_to_bf16",
               lambda x: np.asarray(x, np.float64).astype(np.float32).view(np.uint32)
               .__and__(np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64),
               test_bf16_rounding_random_float32_sample)          # truncation
    monkeypatch.setattr(ref, "round_to_bf16", good_rb)

    good_proj = ref.project_keys
    _pins_fail(monkeypatch, "project_keys",
               lambda k, w, dt: ref.round_storage(np.asarray(k) @ np.asarray(w)[::-1], dt),
               lambda: test_project_keys_matches_exact_rationals("bf16", 8))
    monkeypatch.setattr(ref, "project_keys", good_proj)

    good_ln = ref.layer_norm
    _pins_fail(monkeypatch, "layer_norm",
               lambda h, eps: (np.asarray(h) - np.mean(h, -1, keepdims=True))
               / np.sqrt(np.var(h, -1, ddof=1, keepdims=True) + eps),          # unbiased var
               test_layer_norm_matches_torch)
    monkeypatch.setattr(ref, "layer_norm", good_ln)

    good_sr = ref.score_raw

    def score_first_head_only(q, k, Hkv, causal=False, q_pos0=0):
        q = np.asarray(q, np.float64)
        R = q.shape[1] // Hkv
        return good_sr(q[:, ::R].repeat(R, axis=1) / R, k, Hkv, causal, q_pos0)
    _pins_fail(monkeypatch, "score_raw", score_first_head_only,
               test_score_raw_matches_exact_group_sums_and_causal_mask)
    monkeypatch.setattr(ref, "score_raw", good_sr)

    def score_kv_by_selection_index(q, k, Hkv, causal=False, q_pos0=0, sel_group=0):
        # a plausible slip: selection head j reads KV head j % Hkv instead of its own
        q = np.asarray(q, np.float64)
        Hq = q.shape[1]
        gs = sel_group or Hq // Hkv
        Hs = Hq // gs
        kk = np.asarray(k, np.float64)[:, np.arange(Hs) % Hkv]
        return good_sr(q, kk, Hs, causal, q_pos0)
    _pins_fail(monkeypatch, "score_raw", score_kv_by_selection_index,
               lambda: test_score_raw_per_selection_head_matches_exact_dots(8, 2, 1))
    monkeypatch.setattr(ref, "score_raw", good_sr)

    good_att = ref.attend
    _pins_fail(monkeypatch, "attend",
               lambda q, k, v, scale: good_att(q, k, v, 1.0),              # scale dropped
               test_attend_matches_sdpa_dense_and_masked)
    monkeypatch.setattr(ref, "attend", good_att)

    good_slot = ref.slot_of
    _pins_fail(monkeypatch, "slot_of", lambda layer, G: layer % G, test_slot_map_golden)
    monkeypatch.setattr(ref, "slot_of", good_slot)

    good_prod = ref.producer_of
    _pins_fail(monkeypatch, "producer_of", lambda layer, G: G * ((layer - 1) // G) if layer else 0,
               test_slot_map_golden)
    monkeypatch.setattr(ref, "producer_of", good_prod)


def test_selection_cache_pins():
    """Selection cache: exact cosines of hand-built vectors, the stacking of the group's
    heads into one vector, the zero-vector rule, scale invariance and the reference
    refresh.  (3,4).(4,3) / 25 = 24/25 exactly; a per-head mean of cosines would give a
    different value for heads of unequal norm, and that reading fails here."""
    # B=1, Hkv=1, R=2, D=2: heads h0, h1
    q = np.array([[[3.0, 4.0], [0.0, 0.0]]])
    ref = np.array([[[4.0, 3.0], [0.0, 0.0]]])
    keep, new_ref, cos = oracle.selection_cache(q, ref, 1, 0.96)
    assert cos[0, 0] == 24.0 / 25.0 and keep[0, 0] and np.array_equal(new_ref, ref)
    keep, new_ref, _ = oracle.selection_cache(q, ref, 1, 0.97)
    assert not keep[0, 0] and np.array_equal(new_ref, q)           # refreshed with q
    # stacking: heads (1,0),(0,10) vs (1,0),(10,0): stacked cos = 1/101, not mean(1, 0)
    q2 = np.array([[[1.0, 0.0], [0.0, 10.0]]])
    r2 = np.array([[[1.0, 0.0], [10.0, 0.0]]])
    _, _, c2 = oracle.selection_cache(q2, r2, 1, 0.5)
    assert abs(c2[0, 0] - 1.0 / 101.0) < 1e-15
    # zero vector: cos 0, always refreshed at a positive threshold
    z = np.zeros((1, 2, 2))
    keep, new_ref, cz = oracle.selection_cache(q, z, 1, 0.0001)
    assert cz[0, 0] == 0.0 and not keep[0, 0] and np.array_equal(new_ref, q)
    # scale invariance, opposite vectors, two KV heads handled independently
    rng = np.random.default_rng(5)
    a = rng.standard_normal((2, 4, 8))
    b = rng.standard_normal((2, 4, 8))
    _, _, c_ab = oracle.selection_cache(a, b, 2, 0.0)
    _, _, c_sc = oracle.selection_cache(3.0 * a, 0.5 * b, 2, 0.0)
    assert np.allclose(c_ab, c_sc, rtol=0, atol=1e-15)
    _, _, c_neg = oracle.selection_cache(a, -a, 2, 0.0)
    assert np.allclose(c_neg, -1.0, atol=1e-15)
    want = np.array([[np.dot(a[bb, 2 * g:2 * g + 2].ravel(), b[bb, 2 * g:2 * g + 2].ravel()) /
                      (np.linalg.norm(a[bb, 2 * g:2 * g + 2]) * np.linalg.norm(b[bb, 2 * g:2 * g + 2]))
                      for g in range(2)] for bb in range(2)])
    assert np.allclose(c_ab, want, rtol=0, atol=1e-15)


def test_fetch_rows_pins():
    """Selected-row fetch: a hand-worked gather (rows in set order, the KV head of each
    selection head, slots past the set left zero), and attention over the packed rows with
    positions 0..|S|-1 equals attention over the cache with the set (torch SDPA with a
    mask, per query head)."""
    k = np.arange(2 * 6 * 3, dtype=np.float64).reshape(1, 2, 6, 3)
    k = np.concatenate([k, k + 1000.0], axis=0)                  # B = 2
    v = -k
    sel = [[np.array([1, 4]), np.array([0]), np.array([5, 2, 3]), np.array([])],
           [np.array([3]), np.array([0, 1]), np.array([2]), np.array([4, 5])]]
    ks, vs = oracle.fetch_rows(k, v, sel, Hq=4, cap=3, sel_group=1)   # Hkv = 2, R = 2
    assert ks.shape == (2, 4, 3, 3)
    # selection head j reads KV head j // 2
    assert np.array_equal(ks[0, 0, :2], k[0, 0, [1, 4]]) and not ks[0, 0, 2].any()
    assert np.array_equal(ks[0, 1, :1], k[0, 0, [0]]) and not ks[0, 1, 1:].any()
    assert np.array_equal(ks[0, 2], k[0, 1, [5, 2, 3]])
    assert not ks[0, 3].any()
    assert np.array_equal(vs[1, 3, :2], v[1, 1, [4, 5]])
    # the default grouping: one set per KV head
    ks2, _ = oracle.fetch_rows(k, v, [[np.array([2, 0]), np.array([1])]] * 2, Hq=4, cap=2)
    assert np.array_equal(ks2[1, 0], k[1, 0, [2, 0]]) and np.array_equal(ks2[1, 1, :1], k[1, 1, [1]])
    # attention over the packed rows == attention over the cache with the set
    rng = np.random.default_rng(48)
    B, Hq, Hkv, L, D = 1, 4, 2, 20, 8
    kc = rng.standard_normal((B, Hkv, L, D)); vc = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, Hq, D))
    sets = [[np.sort(rng.choice(L, 7, replace=False)) for _ in range(Hq)]]
    kp, vp = oracle.fetch_rows(kc, vc, sets, Hq=Hq, cap=7, sel_group=1)
    packed = oracle.sparse_decode_attn(q, kp, vp, [[np.arange(7)] * Hq], 0.4)
    mask = torch.zeros(B, Hq, 1, L, dtype=torch.bool)
    for h in range(Hq):
        mask[0, h, 0, sets[0][h]] = True
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], torch.from_numpy(np.repeat(kc, 2, axis=1)),
        torch.from_numpy(np.repeat(vc, 2, axis=1)), attn_mask=mask, scale=0.4)[:, :, 0]
    np.testing.assert_allclose(packed, want.numpy(), rtol=0, atol=1e-12)


def test_expand_neighbors_pins():
    """Neighbour fetching: hand-worked sets (edges clipped, overlaps merged, the window at
    the current length, width 0, unordered and out-of-range input), then random rows
    against a morphological dilation of the selection's indicator vector (a convolution
    with a box of 2*width+1 ones), which forms the set by another route."""
    E = oracle.expand_neighbors
    assert E([4], 10, 1, 0).tolist() == [3, 4, 5]
    assert E([0], 10, 2, 0).tolist() == [0, 1, 2]                    # clipped at 0
    assert E([9], 10, 2, 0).tolist() == [7, 8, 9]                    # clipped at L - 1
    assert E([2, 4], 10, 1, 0).tolist() == [1, 2, 3, 4, 5]           # overlap merged once
    assert E([1], 10, 0, 3).tolist() == [1, 7, 8, 9]                 # window [L-3, L)
    assert E([1], 4, 0, 9).tolist() == [0, 1, 2, 3]                  # window wider than L
    assert E([5, 1, 5], 10, 0, 0).tolist() == [1, 5]                 # unordered, repeated
    assert E([-1, 12], 10, 3, 0).tolist() == []                      # outside [0, L) dropped
    assert E([], 10, 3, 2).tolist() == [8, 9]
    # a selection made at a shorter length, reused after the cache grew: the window moves
    assert E([0, 1, 2, 5, 6], 12, 1, 2).tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 10, 11]
    rng = np.random.default_rng(11)
    for trial in range(60):
        L = int(rng.integers(1, 400)) if trial % 3 else int(rng.integers(1, 8))
        w = int(rng.integers(0, 6))
        nw = int(rng.integers(0, 20))
        sel = rng.choice(L + 10, size=int(rng.integers(0, L + 1)), replace=True) - 5
        ind = np.zeros(L)
        inr = sel[(sel >= 0) & (sel < L)]
        ind[inr] = 1.0
        dil = np.convolve(ind, np.ones(2 * w + 1), mode="full")[w:w + L] > 0.5
        dil[max(0, L - nw):] = True
        assert np.array_equal(E(sel, L, w, nw), np.flatnonzero(dil))


def test_ulps_bf16_pins():
    """Distance along the bf16 grid: hand-worked pairs (equal values, -0 against +0,
    neighbours, a binade edge, a sign crossing through zero, the largest finite value
    against infinity), then every pair from a sample against the distance in an
    enumeration of all finite bf16 values sorted by value (a different route: positions
    in a sorted list, not bit arithmetic)."""
    U = lambda a, b: int(oracle.ulps_bf16(np.array([a]), np.array([b]))[0])
    tiny = 2.0 ** -133                               # smallest positive bf16 (subnormal)
    big = float.fromhex("0x1.fep127")                # largest finite bf16 (0x7F7F)
    assert U(1.0, 1.0) == 0 and U(0.0, -0.0) == 0
    assert U(1.0, 1.0 + 2.0 ** -7) == 1 and U(1.0 + 2.0 ** -7, 1.0) == 1
    assert U(2.0 - 2.0 ** -7, 2.0) == 1               # across a binade edge
    assert U(1.0, 2.0) == 128                          # one binade holds 128 values
    assert U(tiny, -tiny) == 2 and U(tiny, 0.0) == 1 and U(-tiny, -0.0) == 1
    assert U(-1.0, 1.0) == 2 * 0x3F80                  # through zero: both magnitudes
    assert U(big, np.inf) == 1 and U(-big, -np.inf) == 1
    # all finite bf16 values, -0 merged with +0, sorted by value
    pats = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    vals = pats.view(np.float32).astype(np.float64)
    grid = np.unique(vals[np.isfinite(vals)])          # unique also merges -0 and +0
    pos = {v: i for i, v in enumerate(grid.tolist())}
    rng = np.random.default_rng(13)
    a = grid[rng.integers(0, len(grid), 4000)]
    b = np.where(rng.random(4000) < 0.5, grid[rng.integers(0, len(grid), 4000)],
                 grid[np.clip(np.searchsorted(grid, a) + rng.integers(-3, 4, 4000), 0,
                              len(grid) - 1)])
    want = np.array([abs(pos[x] - pos[y]) for x, y in zip(a.tolist(), b.tolist())])
    assert np.array_equal(oracle.ulps_bf16(a, b), want)


def test_cached_selection_pins():
    """A kept row of the selection cache at a grown length: hand-worked sets, then random
    rows against the neighbour-fetching set with width 0 (another function, built as a
    Python set) and the invariants: the previous set survives below the new window, the
    window at the current length is always there, nothing at or past L."""
    C = oracle.cached_selection
    assert C([0, 1, 5, 9], 12, 3).tolist() == [0, 1, 5, 9, 10, 11]
    assert C([0, 1, 5, 9], 10, 3).tolist() == [0, 1, 5, 7, 8, 9]      # same length
    assert C([0, 3, 9, 11], 10, 2).tolist() == [0, 3, 8, 9]           # past L: dropped
    assert C([], 5, 9).tolist() == [0, 1, 2, 3, 4]                     # window wider than L
    assert C([2], 6, 0).tolist() == [2]
    rng = np.random.default_rng(17)
    for trial in range(80):
        L = int(rng.integers(1, 300))
        nw = int(rng.integers(0, 40))
        Lp = int(rng.integers(1, L + 1))
        prev = np.sort(rng.choice(Lp, size=int(rng.integers(0, Lp + 1)), replace=False))
        got = C(prev, L, nw)
        assert np.array_equal(got, oracle.expand_neighbors(prev, L, 0, nw))
        assert np.all(np.diff(got) > 0) and (len(got) == 0 or got[-1] < L)
        assert set(range(max(0, L - nw), L)) <= set(got.tolist())
        assert set(prev[prev < L].tolist()) <= set(got.tolist())


def test_masked_attention_rows_causal_prefill_matches_sdpa():
    """Prefill rows (Lq > 1): row i of a chunk at q_pos0 attends over its own selected set
    inside its causal prefix; torch SDPA with a per-(head, row) boolean mask gives the same
    outputs for every row of several chunks, per KV head and per query head."""
    rng = np.random.default_rng(49)
    B, Hq, Hkv, D, Lq, q_pos0 = 2, 4, 2, 8, 6, 5
    L = q_pos0 + Lq
    k = rng.standard_normal((B, Hkv, L, D)); v = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, Hq, Lq, D))
    for gs in (2, 1):
        Hs = Hq // gs
        sel = [[[np.sort(rng.choice(q_pos0 + i + 1, size=int(rng.integers(1, q_pos0 + i + 2)),
                                    replace=False)) for i in range(Lq)]
                for _ in range(Hs)] for _ in range(B)]
        got = ref.masked_attention_rows(q, k, v, sel, 0.45, sel_group=gs)
        assert len(got) == B * Hq * Lq
        mask = torch.zeros(B, Hq, Lq, L, dtype=torch.bool)
        for b in range(B):
            for h in range(Hq):
                for i in range(Lq):
                    mask[b, h, i, sel[b][h // gs][i]] = True
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1)),
            torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1)), attn_mask=mask, scale=0.45)
        for (b, h, i), o in got.items():
            np.testing.assert_allclose(o, want[b, h, i].numpy(), rtol=0, atol=1e-12)


def test_ulps_and_cached_selection_mutations_are_caught(monkeypatch):
    good_u = ref.ulps_bf16

    def ulps_no_sign(a, b):                       # a dropped sign: magnitudes only
        f = lambda x: np.asarray(x, np.float64).astype(np.float32).view(np.uint32).astype(np.int64) >> 16 & 0x7FFF
        return np.abs(f(a) - f(b))
    monkeypatch.setattr(oracle, "ulps_bf16", ulps_no_sign)
    with pytest.raises(AssertionError):
        test_ulps_bf16_pins()
    monkeypatch.setattr(oracle, "ulps_bf16", good_u)

    good_c = ref.cached_selection
    # the window taken at the earlier length: no token appended since is attended
    monkeypatch.setattr(oracle, "cached_selection",
                        lambda prev, L, nw: good_c(prev, max(int(np.max(prev, initial=0)) + 1, 1), nw)
                        if len(prev) else good_c(prev, L, nw))
    with pytest.raises(AssertionError):
        test_cached_selection_pins()
    monkeypatch.setattr(oracle, "cached_selection", good_c)
