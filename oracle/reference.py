"""CPU oracle for query-aware sparse decode (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this module.  The HIP library never calls it, and it imports
nothing from the HIP package: the two share only the seeded input generators
in ``synthetic/``.

Everything is plain numpy in float64 on values that are exactly the stored
(bf16 or fp32) inputs, and each stored result is rounded once, to nearest
even, into its storage type.  Sources, cited by page title and section:

* "Meta-Llama-3.1-8B-Instruct-Butler" model card (TokenButler), section
  *Method*: producer layers 0, G, 2G, ... read LN(H) and emit
  Q_imp = f_theta(LN(H)) with G slots; K_imp = K . W_K for every layer;
  a consumer at layer l uses slot (l - 1) mod G, scores every cached token,
  keeps a top-x subset under a fixed budget and adds a sink prefix and a
  recent window.  Section *Memory requirements*: default 50% per layer,
  layer 0 dense, ``fixed_<N>pc`` retains (100 - N)%, knobs
  ``min_sparse_index`` (sink) and ``sliding_window`` (window).
* "TokenButler: Token Importance is Predictable" (arXiv abstract page):
  selection is per token under a fixed budget, the full KV cache is kept.
* "TokenButler: Token Importance is Predictable" (arXiv abstract page):
  prediction interval with neighbor fetching -- the predictor's selection is
  reused between its runs, widened with the selected tokens' neighbours.
* TokenSelect README, first highlights: per-head Q.K criticality, per-head
  softmax, summed over heads ("soft voting"); Selection Cache: consecutive
  similar queries share one token selection.

Readings where the pages are silent (each listed in the design notes):
GQA head h belongs to KV head h // R; the raw scorer of a GQA group is the
group's summed Q_imp dotted with K_imp (the model card gives Q_imp one
vector per head but not whether a group shares its selection: ``sel_group``
query heads share one selected set, by default all R of a KV head, and
sel_group = 1 selects per query head); LN is LayerNorm without affine,
eps given, biased variance; f_theta is Linear -> ReLU -> Linear without
biases, output laid out head-major, then slot, then d'; ties in the top-x go
to the lower token index; -0 counts as +0 and NaN as -inf; the budget is
x = floor(L_r * num / den) taken over all L_r tokens, then unioned with the
sink [0, s) and the window [L_r - w, L_r); attention uses scale 1/sqrt(D).

Parity pins for every function live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def round_to_bf16(x) -> np.ndarray:
    """Round float64 values once, to nearest even, onto the bfloat16 grid.

    bfloat16 keeps 8 significant bits and float32's exponent range: the
    spacing at a value whose leading bit is 2^(e-1) is 2^(e-8), floored at
    the subnormal spacing 2^-133; a rounded magnitude of 2^128 or more
    overflows to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0.0)
    xf = x[fin]
    _, e = np.frexp(xf)                      # |xf| = m * 2^e, m in [0.5, 1)
    ulp_exp = np.maximum(e - 8, -133)
    scaled = np.ldexp(xf, -ulp_exp)          # exact: power-of-two scaling
    r = np.ldexp(np.rint(scaled), ulp_exp)   # rint: round half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def round_to_f32(x) -> np.ndarray:
    """Round float64 values once, to nearest even, onto the float32 grid."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_storage(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return round_to_f32(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# producer and slot map (model card, Method)
# ---------------------------------------------------------------------------

def producer_of(layer: int, G: int) -> int:
    """Producer layer whose Q_imp serves ``layer``: itself when layer % G == 0,
    otherwise the nearest producer below (producers sit at 0, G, 2G, ...)."""
    return G * (layer // G)


def slot_of(layer: int, G: int) -> int:
    """Slot of the producer's Q_imp that ``layer`` reads: (layer - 1) mod G."""
    return (layer - 1) % G


def layer_norm(h, eps: float) -> np.ndarray:
    """LN over the last axis: (h - mean) / sqrt(biased var + eps), no affine."""
    h = np.asarray(h, dtype=np.float64)
    mu = h.mean(axis=-1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=-1, keepdims=True)
    return (h - mu) / np.sqrt(var + eps)


def produce_queries(h, w1, w2, Hq: int, G: int, dprime: int, eps: float = 1e-5,
                    dtype: str = "bf16") -> np.ndarray:
    """Q_imp = f_theta(LN(H)) as [B, Hq, G, Lq, d'].

    h: [B, Lq, E]; w1: [E, F]; w2: [F, Hq*G*d'].  f_theta is
    relu(x . W1) . W2; the normalised input, the hidden activation and the
    output are each rounded to the storage type, as a bf16 pipeline stores
    them.  Output column (head*G + slot)*d' + i is Q_imp[b, head, slot, t, i].
    """
    h = np.asarray(h, dtype=np.float64)
    B, Lq, E = h.shape
    x = round_storage(layer_norm(h, eps), dtype)
    a = round_storage(np.maximum(x @ np.asarray(w1, np.float64), 0.0), dtype)
    y = round_storage(a @ np.asarray(w2, np.float64), dtype)
    assert y.shape[-1] == Hq * G * dprime
    return y.reshape(B, Lq, Hq, G, dprime).transpose(0, 2, 3, 1, 4).copy()


# ---------------------------------------------------------------------------
# key projection (model card, Method: K_imp = K . W_K)
# ---------------------------------------------------------------------------

def project_keys(k, w_k, dtype: str) -> np.ndarray:
    """K_imp = K . W_K for key rows k [..., D] and W_K [D, d'], rounded once."""
    return round_storage(np.asarray(k, np.float64) @ np.asarray(w_k, np.float64), dtype)


# ---------------------------------------------------------------------------
# scoring
# ---------------------------------------------------------------------------

def _causal_lengths(Lq: int, L: int, q_pos0: int, causal: bool) -> np.ndarray:
    if not causal:
        return np.full(Lq, L, dtype=np.int64)
    return np.minimum(q_pos0 + np.arange(Lq) + 1, L)


def selection_groups(Hq: int, Hkv: int, sel_group: int = 0):
    """(Hs, gs): selection heads per batch entry and query heads per selection head.
    Selection head j holds query heads [j*gs, (j+1)*gs) and reads KV head j*gs // R."""
    R = Hq // Hkv
    gs = R if not sel_group else sel_group
    assert Hq % Hkv == 0 and R % gs == 0, "sel_group must divide Hq / Hkv"
    return Hq // gs, gs


def score_raw(q_imp_slot, kimp, Hkv: int, causal: bool = False, q_pos0: int = 0,
              sel_group: int = 0) -> np.ndarray:
    """Raw importance scores [B, Hs, Lq, L], float32 values in float64.

    q_imp_slot: [B, Hq, Lq, d'] (the consumer's slot); kimp: [B, Hkv, L, d'].
    Score of token t for selection head j is (sum of Q_imp over j's query
    heads) . K_imp[t] of their KV head, summed in float64 and rounded once to
    float32.  By default j is a KV head and its query heads are its GQA group.
    For a causal row i (absolute position q_pos0 + i) tokens after it score -inf.
    """
    q = np.asarray(q_imp_slot, np.float64)
    k = np.asarray(kimp, np.float64)
    B, Hq, Lq, dp = q.shape
    Hs, gs = selection_groups(Hq, Hkv, sel_group)
    R = Hq // Hkv
    qbar = q.reshape(B, Hs, gs, Lq, dp).sum(axis=2)             # [B, Hs, Lq, d']
    kv_of = np.arange(Hs) * gs // R                              # KV head of each selection head
    s = round_to_f32(np.einsum("bgqi,bgti->bgqt", qbar, k[:, kv_of]))
    lens = _causal_lengths(Lq, k.shape[2], q_pos0, causal)
    t = np.arange(k.shape[2])
    s[:, :, t[None, :] >= lens[:, None]] = -np.inf
    return s


def softmax_last(z) -> np.ndarray:
    z = np.asarray(z, np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def score_softvote(q, k, Hkv: int, scale: float, causal: bool = False,
                   q_pos0: int = 0, sel_group: int = 0) -> np.ndarray:
    """Soft-voting scores [B, Hs, Lq, L] (TokenSelect README, highlights).

    q: [B, Hq, Lq, D]; k: [B, Hkv, L, D].  For each query head h the
    criticality of token t is its logit q_h . k_t * scale; each head's
    criticalities are normalised by a softmax over all cached tokens (the
    causal prefix for a causal row); the score of t for selection head j is
    the sum of those probabilities over j's query heads (by default the GQA
    group of a KV head), rounded to float32.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, Hq, Lq, D = q.shape
    Hs, gs = selection_groups(Hq, Hkv, sel_group)
    R = Hq // Hkv
    L = k.shape[2]
    kk = np.repeat(k, R, axis=1)                                 # [B, Hq, L, D]
    z = np.einsum("bhqd,bhtd->bhqt", q, kk) * scale
    lens = _causal_lengths(Lq, L, q_pos0, causal)
    t = np.arange(L)
    z[:, :, t[None, :] >= lens[:, None]] = -np.inf
    p = softmax_last(z)
    s = round_to_f32(p.reshape(B, Hs, gs, Lq, L).sum(axis=2))
    s[:, :, t[None, :] >= lens[:, None]] = -np.inf
    return s


# ---------------------------------------------------------------------------
# selection (model card, Method and Memory requirements)
# ---------------------------------------------------------------------------

def budget(L_r: int, num: int, den: int) -> int:
    """Fixed budget x = floor(L_r * num / den); fixed_<N>pc is num/den = (100-N)/100."""
    return (L_r * num) // den


def fixed_pc_fraction(policy: str):
    """'fixed_70pc' -> (30, 100): the retained fraction as num/den."""
    assert policy.startswith("fixed_") and policy.endswith("pc")
    n = int(policy[len("fixed_"):-2])
    return (100 - n, 100)


def select(scores_row, x: int, n_sink: int, n_window: int,
           exclude_forced: bool = False) -> np.ndarray:
    """Selected token set of one row, ascending int64.

    Top-x tokens by (score descending, index ascending) over the row's L_r
    tokens, unioned with the sink [0, n_sink) and the window
    [L_r - n_window, L_r).  -0 is +0 and NaN is -inf for the ordering.
    With exclude_forced (the other reading of the model card's Method and
    Memory requirements: the budget counts only the tokens that are neither
    sink nor window), the top-x is taken among those middle tokens only.
    """
    s = np.array(scores_row, dtype=np.float64)
    s[np.isnan(s)] = -np.inf
    s[s == 0.0] = 0.0
    L_r = s.shape[0]
    sink = np.arange(min(n_sink, L_r))
    window = np.arange(max(0, L_r - n_window), L_r)
    pool = np.arange(L_r)
    if exclude_forced:
        forced = np.zeros(L_r, bool)
        forced[sink] = True
        forced[window] = True
        pool = pool[~forced]
    order = pool[np.lexsort((pool, -s[pool]))]     # last key is primary
    top = order[:min(max(x, 0), pool.shape[0])]
    return np.unique(np.concatenate([top, sink, window]).astype(np.int64))


# ---------------------------------------------------------------------------
# attention over the selected set (model card, intro and Method)
# ---------------------------------------------------------------------------

def attend(q_heads, k_rows, v_rows, scale: float) -> np.ndarray:
    """Softmax attention of query heads [R, D] over the selected rows [n, D].

    o_h = sum_t softmax_t(q_h . k_t * scale) v_t, all in float64.
    """
    q = np.asarray(q_heads, np.float64)
    k = np.asarray(k_rows, np.float64)
    v = np.asarray(v_rows, np.float64)
    z = (q @ k.T) * scale                                        # [R, n]
    p = softmax_last(z)
    return p @ v


def sparse_decode_attn(q, k_cache, v_cache, sel, scale: float,
                       sel_group: int = 0) -> np.ndarray:
    """Decode attention [B, Hq, D] for one query token per head.

    q: [B, Hq, D]; caches [B, Hkv, L_cap, D]; sel[b][j] is the ascending
    selected index array of selection head j (by default KV head j).  Query
    head h attends to the set of selection head h // sel_group over the rows
    of KV head h // R.
    """
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    R = Hq // Hkv
    Hs, gs = selection_groups(Hq, Hkv, sel_group)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            idx = np.asarray(sel[b][h // gs], np.int64)
            out[b, h] = attend(q[b, h][None, :], np.asarray(k_cache[b, h // R])[idx],
                               np.asarray(v_cache[b, h // R])[idx], scale)[0]
    return out


def masked_attention_rows(q, k_cache, v_cache, sel_rows, scale: float,
                          rows: Optional[list] = None, sel_group: int = 0) -> dict:
    """Prefill attention for selected query rows.

    q: [B, Hq, Lq, D]; sel_rows[b][j][i] is row i's selected set of selection
    head j (by default KV head j).  Returns {(b, h, i): o[D]} for every
    (b, h, i) in ``rows`` (all rows if None).
    """
    q = np.asarray(q, np.float64)
    B, Hq, Lq, D = q.shape
    Hkv = k_cache.shape[1]
    R = Hq // Hkv
    Hs, gs = selection_groups(Hq, Hkv, sel_group)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Lq)]
    out = {}
    for (b, h, i) in rows:
        g = h // R
        idx = np.asarray(sel_rows[b][h // gs][i], np.int64)
        out[(b, h, i)] = attend(q[b, h, i][None, :], np.asarray(k_cache[b, g])[idx],
                                np.asarray(v_cache[b, g])[idx], scale)[0]
    return out


def dense_decode_attn(q, k_cache, v_cache, L: int, scale: float) -> np.ndarray:
    """Dense decode attention over tokens [0, L) (layer 0 of the model card)."""
    B, Hkv = k_cache.shape[:2]
    sel = [[np.arange(L) for _ in range(Hkv)] for _ in range(B)]
    return sparse_decode_attn(q, k_cache, v_cache, sel, scale)


# ---------------------------------------------------------------------------
# one decode step of one layer, chained
# ---------------------------------------------------------------------------

def decode_layer_step(*, q, k_cache, v_cache, L: int, num: int, den: int,
                      n_sink: int, n_window: int, scale: float, Hkv: int,
                      mode: str = "raw", q_imp_slot=None, kimp=None,
                      dense: bool = False, sel_group: int = 0) -> dict:
    """Score -> select -> attend for one decode layer at context L.

    q: [B, Hq, D]; raw mode needs q_imp_slot [B, Hq, d'] and kimp
    [B, Hkv, >=L, d']; softvote mode scores with q against the keys.
    Returns scores [B, Hs, L], the selected sets and the output [B, Hq, D]
    (Hs selection heads of sel_group query heads each; see selection_groups).
    """
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    kc = np.asarray(k_cache, np.float64)[:, :, :L]
    vc = np.asarray(v_cache, np.float64)[:, :, :L]
    if dense:
        sel = [[np.arange(L) for _ in range(Hkv)] for _ in range(B)]
        return {"scores": None, "sel": sel,
                "out": sparse_decode_attn(q, kc, vc, sel, scale)}
    if mode == "raw":
        s = score_raw(np.asarray(q_imp_slot, np.float64)[:, :, None, :],
                      np.asarray(kimp, np.float64)[:, :, :L], Hkv,
                      sel_group=sel_group)[:, :, 0]
    else:
        s = score_softvote(q[:, :, None, :], kc, Hkv, scale, sel_group=sel_group)[:, :, 0]
    x = budget(L, num, den)
    sel = [[select(s[b, j], x, n_sink, n_window) for j in range(s.shape[1])]
           for b in range(B)]
    return {"scores": s, "sel": sel,
            "out": sparse_decode_attn(q, kc, vc, sel, scale, sel_group=sel_group)}


def selection_cache(q, q_ref, Hkv: int, threshold: float, sel_group: int = 0):
    """TokenSelect README, highlights, Selection Cache: consecutive similar queries share
    one token selection.  q, q_ref: [B, Hq, D] (one decode step).  Per (b, selection
    head) -- by default a KV head and its R query heads -- the cosine similarity of the
    head's query heads stacked into one vector (float64; 0 when either vector is zero)
    with the reference the cached selection was made for.
    Returns (keep [B, Hs] bool: cos >= threshold, new q_ref: q where not kept, cos)."""
    q = np.asarray(q, dtype=np.float64)
    ref = np.asarray(q_ref, dtype=np.float64)
    B, Hq, D = q.shape
    Hs, gs = selection_groups(Hq, Hkv, sel_group)
    a = q.reshape(B, Hs, gs * D)
    c = ref.reshape(B, Hs, gs * D)
    na = np.sqrt((a * a).sum(-1))
    nc = np.sqrt((c * c).sum(-1))
    dot = (a * c).sum(-1)
    den = na * nc
    cos = np.where(den > 0, dot / np.where(den > 0, den, 1.0), 0.0)
    keep = cos >= threshold
    new_ref = np.where(keep[:, :, None, None], c.reshape(B, Hs, gs, D),
                       a.reshape(B, Hs, gs, D)).reshape(B, Hq, D)
    return keep, new_ref, cos


def fetch_rows(k_cache, v_cache, sel, Hq: int, cap: int, sel_group: int = 0):
    """Selected-row fetch from a KV cache kept off the GPU (TokenButler arXiv abstract:
    latency against dense attention with the KV cache offloaded to the CPU).  Only the
    rows of each selected set cross to the GPU, packed in set order: for selection head
    j of batch b, k_sel[b, j, p] = k_cache[b, kv(j), sel[b][j][p]] for p < |S|; slots
    p >= |S| stay zero here.  k_cache, v_cache: [B, Hkv, L, D]; returns (k_sel, v_sel),
    each [B, Hs, cap, D] float64."""
    k = np.asarray(k_cache, np.float64)
    v = np.asarray(v_cache, np.float64)
    B, Hkv, _, D = k.shape
    Hs, gs = selection_groups(Hq, Hkv, sel_group)
    R = Hq // Hkv
    ks = np.zeros((B, Hs, cap, D))
    vs = np.zeros((B, Hs, cap, D))
    for b in range(B):
        for j in range(Hs):
            rows = np.asarray(sel[b][j], np.int64)[:cap]
            ks[b, j, :len(rows)] = k[b, j * gs // R, rows]
            vs[b, j, :len(rows)] = v[b, j * gs // R, rows]
    return ks, vs


def expand_neighbors(sel, L: int, width: int, n_window: int) -> np.ndarray:
    """Neighbour fetching for the prediction interval (TokenButler arXiv abstract page:
    prediction interval with neighbor fetching).  The abstract only names the method; the
    reading taken here: between predictor runs the last selection ``sel`` (token indices of
    one row, any order) is reused at the current length L, every reused token brings the
    tokens within ``width`` positions of it, and the recent window [L - n_window, L) is
    added so tokens appended since the selection are attended.  Indices outside [0, L) are
    dropped.  Returns the ascending int64 set."""
    out = set()
    for t in np.asarray(sel, np.int64).tolist():
        if 0 <= t < L:
            for u in range(t - width, t + width + 1):
                if 0 <= u < L:
                    out.add(u)
    out.update(range(max(0, L - n_window), L))
    return np.array(sorted(out), dtype=np.int64)


def cached_selection(sel_prev, L: int, n_window: int) -> np.ndarray:
    """A kept row of the selection cache at the current length L (TokenSelect README,
    highlights, Selection Cache: consecutive similar queries share one token selection;
    model card, Method: the set always holds a recent window).  The reading taken: the
    selection made for an earlier query (any earlier length) is reused, and the window is
    re-taken at the current length, so every token appended since is attended:
        S = (sel_prev restricted to [0, L))  U  [max(0, L - n_window), L)
    Returns the ascending int64 set."""
    prev = np.asarray(sel_prev, np.int64)
    prev = prev[(prev >= 0) & (prev < L)]
    window = np.arange(max(0, L - n_window), L, dtype=np.int64)
    return np.union1d(prev, window).astype(np.int64)


def ulps_bf16(a, b) -> np.ndarray:
    """Distance between two bf16-valued arrays, counted in bf16 values: the number of
    steps from one to the other along the ordered bf16 grid (-0 and +0 are one point;
    the largest finite value and infinity are one step apart).  Each bf16 pattern maps
    to an integer that grows with the value: the magnitude bits for a positive value,
    their negation for a negative one."""
    def ordered(x):
        x = np.asarray(x, np.float64).astype(np.float32)
        u = x.view(np.uint32).astype(np.int64) >> 16
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("math", "np", "Optional",
                                                                   "annotations")]
