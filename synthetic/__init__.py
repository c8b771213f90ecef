"""Seeded synthetic inputs for the query-aware sparse-decode workloads.

This module is the only code that the oracle (``oracle/``) and the HIP path
(``query_aware_sparse_imp_amd``) have in common.  It draws random tensors and
shapes them into the five workloads; it holds none of the method's own
arithmetic (no layer norm, no producer, no key projection, no scoring, no
selection, no attention).  The only non-trivial operations here are input
preparation that the workloads' descriptions ask for: heavy-hitter keys pushed
along a query direction, clustered keys, a query random walk, the Q_imp
stand-in for the workloads that have no producer, and the RoPE'd Q/K/V of the
prefill workload.

Every draw comes from ``numpy.random.default_rng(SeedSequence([cfg, layer,
tag, step, *sub]))`` as float32 ``standard_normal`` (or ``choice`` /
``integers`` for positions), so any single (layer, tag, step, head) stream can
be regenerated on its own.  Storage rounding to bfloat16 uses torch's own
float32 -> bfloat16 conversion (round-to-nearest-even).

The workloads are Llama-3.1-8B shaped (32 query heads, 8 KV heads, head dim
128, hidden size 4096, 32 layers, RoPE base 500000), as named on the
TokenButler model card (the page's title and intro).  They stand in for the
long-context benchmarks the pages evaluate on (RULER, LongBench,
InfiniteBench, TokenSelect's passkey prompt), none of which is used here.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

# Seed-stream tags.
T_K, T_V, T_Q, T_QIMP, T_WK, T_H, T_W1, T_W2 = 1, 2, 3, 4, 5, 6, 7, 8
T_HEAVY, T_MIX, T_CENT, T_WALK, T_NEWKV, T_WQKV = 9, 10, 11, 12, 13, 14

SCORE_RAW, SCORE_SOFTVOTE = 0, 1


def rng(cfg: int, layer: int, tag: int, step: int = 0, *sub: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg, layer, tag, step, *sub]))


def normal(shape, cfg: int, layer: int, tag: int, step: int = 0, *sub: int,
           std: float = 1.0) -> np.ndarray:
    x = rng(cfg, layer, tag, step, *sub).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def storage(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float32 numpy -> torch CPU tensor in the storage dtype (RNE for bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and policy of one workload (sizes of one decode layer)."""
    cfg: int
    name: str
    dtype: torch.dtype
    B: int
    Hq: int
    Hkv: int
    D: int
    dprime: int
    L: int
    budget_num: int
    budget_den: int
    n_sink: int
    n_window: int
    score_mode: int = SCORE_RAW
    G: int = 1
    layers: int = 1
    E: int = 4096
    F: int = 1024
    wk_std: Optional[float] = None      # None -> 1/sqrt(D)
    heavy_frac: float = 0.0
    chunk: int = 0                       # prefill query chunk
    steps: int = 1

    @property
    def R(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def budget(self, L_r: int) -> int:
        return (L_r * self.budget_num) // self.budget_den

    def cap(self, L_r: int) -> int:
        return min(L_r, self.budget(L_r) + self.n_sink + self.n_window)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


BF16 = torch.bfloat16
F32 = torch.float32

WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny-fp32-decode L=256 D=64 d'=16 50%+4+16", F32, B=1, Hq=1, Hkv=1,
                D=64, dprime=16, L=256, budget_num=1, budget_den=2, n_sink=4, n_window=16),
    2: Workload(2, "llama3-8b-layer-decode L=32768 50%+4+64 raw", BF16, B=1, Hq=32, Hkv=8,
                D=128, dprime=32, L=32768, budget_num=1, budget_den=2, n_sink=4,
                n_window=64, heavy_frac=0.01),
    3: Workload(3, "batched-softvote-decode B=16 L=16384 30%+4+64", BF16, B=16, Hq=32,
                Hkv=8, D=128, dprime=32, L=16384, budget_num=3, budget_den=10, n_sink=4,
                n_window=64, score_mode=SCORE_SOFTVOTE, steps=64),
    4: Workload(4, "long-context-full-depth-decode L=262144 32 layers G=4 1/16+4+128", BF16,
                B=1, Hq=32, Hkv=8, D=128, dprime=32, L=262144, budget_num=1, budget_den=16,
                n_sink=4, n_window=128, G=4, layers=32, wk_std=0.02, heavy_frac=0.01),
    5: Workload(5, "prefill-chunked-causal B=2 L=8192 chunk 1024 50%+4+64", BF16, B=2,
                Hq=32, Hkv=8, D=128, dprime=32, L=8192, budget_num=1, budget_den=2,
                n_sink=4, n_window=64, G=4, wk_std=0.02, chunk=1024),
}


# ---------------------------------------------------------------------------
# decode-layer inputs (workloads 1, 2, 4 and the single-layer sweeps)
# ---------------------------------------------------------------------------

def _query(w: Workload, layer: int, dtype) -> np.ndarray:
    """Attention query of one layer, [B, Hq, 1, D], fixed across decode steps."""
    return normal((w.B, w.Hq, 1, w.D), w.cfg, layer, T_Q)


def _w_k(w: Workload, layer: int) -> np.ndarray:
    std = w.wk_std if w.wk_std is not None else 1.0 / math.sqrt(w.D)
    return normal((w.D, w.dprime), w.cfg, layer, T_WK, std=std)


def _keys_for_head(w: Workload, layer: int, b: int, g: int, L: int,
                   q_dir: Optional[np.ndarray]) -> np.ndarray:
    k = normal((L, w.D), w.cfg, layer, T_K, 0, b, g)
    if w.heavy_frac > 0.0 and q_dir is not None:
        n_hh = int(round(w.heavy_frac * L))
        pos = rng(w.cfg, layer, T_HEAVY, 0, b, g).choice(L, size=n_hh, replace=False)
        k[pos] += np.float32(3.0) * q_dir[None, :]
    return k


def _heavy_direction(qb: np.ndarray, g: int, R: int) -> np.ndarray:
    """Unit vector along the summed query of GQA group g (qb: [Hq, D] float32)."""
    s = qb[g * R:(g + 1) * R].astype(np.float64).sum(axis=0)
    return (s / np.linalg.norm(s)).astype(np.float32)


def decode_layer(w: Workload, layer: int = 0, L: Optional[int] = None,
                 extra: int = 0, heads: Optional[Sequence[tuple]] = None,
                 with_qimp: bool = True) -> Dict[str, object]:
    """Inputs of one decode layer at context length L.

    The cache holds ``L + extra`` rows: rows [0, L) are the prompt's keys and
    values, rows L, L+1, ... are the tokens that decode steps 0, 1, ... append
    (drawn from their own streams).  ``heads`` restricts generation to the
    listed (b, g) KV heads; the others are left zero (used by sampled checks
    at the full sizes).
    """
    L = w.L if L is None else L
    L_cap = L + extra
    q = _query(w, layer, w.dtype)
    q_st = storage(q, w.dtype)
    qf = q_st.float().numpy()
    k = np.zeros((w.B, w.Hkv, L_cap, w.D), np.float32)
    v = np.zeros((w.B, w.Hkv, L_cap, w.D), np.float32)
    todo = heads if heads is not None else [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    for (b, g) in todo:
        direction = _heavy_direction(qf[b, :, 0], g, w.R) if w.heavy_frac > 0 else None
        k[b, g, :L] = _keys_for_head(w, layer, b, g, L, direction)
        v[b, g, :L] = normal((L, w.D), w.cfg, layer, T_V, 0, b, g)
        for s in range(extra):
            kv = normal((2, w.D), w.cfg, layer, T_NEWKV, s, b, g)
            k[b, g, L + s] = kv[0]
            v[b, g, L + s] = kv[1]
    out = {
        "workload": w, "layer": layer, "L": L, "L_cap": L_cap,
        "q": q_st,
        "k_cache": storage(k, w.dtype),
        "v_cache": storage(v, w.dtype),
        "w_k": storage(_w_k(w, layer), w.dtype),
    }
    if with_qimp and w.G == 1:
        out["q_imp"] = qimp_standin(w, layer, out["q"], out["w_k"])
    return out


def qimp_standin(w: Workload, layer: int, q_st: torch.Tensor, wk_st: torch.Tensor) -> torch.Tensor:
    """Q_imp for the workloads without a producer, [B, Hq, 1, 1, d'].

    The tiny workload draws Q_imp directly from N(0,1).  The single-layer
    bf16 workload uses the attention query pushed through the same W_K as
    the keys, rounded to bf16, so that the skew planted in the keys is seen
    by the importance scores too.
    """
    if w.cfg == 1:
        x = normal((w.B, w.Hq, 1, 1, w.dprime), w.cfg, layer, T_QIMP)
        return storage(x, w.dtype)
    x = q_st.double() @ wk_st.double()            # [B, Hq, 1, d']
    return x.float().to(w.dtype).reshape(w.B, w.Hq, 1, 1, w.dprime)


# ---------------------------------------------------------------------------
# producer inputs (workloads 4 and 5)
# ---------------------------------------------------------------------------

def producer_weights(w: Workload, layer: int) -> Dict[str, torch.Tensor]:
    w1 = normal((w.E, w.F), w.cfg, layer, T_W1, std=0.02)
    w2 = normal((w.F, w.Hq * w.G * w.dprime), w.cfg, layer, T_W2, std=0.02)
    return {"w1": storage(w1, w.dtype), "w2": storage(w2, w.dtype)}


def producer_hidden(w: Workload, layer: int, rows: int) -> torch.Tensor:
    """Hidden states fed to a producer, [B, rows, E], N(0,1)."""
    return storage(normal((w.B, rows, w.E), w.cfg, layer, T_H), w.dtype)


# ---------------------------------------------------------------------------
# soft-voting batched decode (workload 3)
# ---------------------------------------------------------------------------

def softvote_cache(w: Workload, layer: int = 0,
                   heads: Optional[Sequence[tuple]] = None) -> Dict[str, torch.Tensor]:
    """Keys: 95% N(0,1), 5% around 8 random centroids (sigma 0.2); V ~ N(0,1)."""
    L = w.L
    k = np.zeros((w.B, w.Hkv, L, w.D), np.float32)
    v = np.zeros((w.B, w.Hkv, L, w.D), np.float32)
    n_mix = int(math.floor(0.05 * L))
    todo = heads if heads is not None else [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    for (b, g) in todo:
        kk = normal((L, w.D), w.cfg, layer, T_K, 0, b, g)
        cent = normal((8, w.D), w.cfg, layer, T_CENT, 0, b, g)
        r = rng(w.cfg, layer, T_MIX, 0, b, g)
        pos = r.choice(L, size=n_mix, replace=False)
        which = r.integers(0, 8, size=n_mix)
        noise = normal((n_mix, w.D), w.cfg, layer, T_MIX, 1, b, g, std=0.2)
        kk[pos] = cent[which] + noise
        k[b, g] = kk
        v[b, g] = normal((L, w.D), w.cfg, layer, T_V, 0, b, g)
    return {"k_cache": storage(k, w.dtype), "v_cache": storage(v, w.dtype)}


def softvote_queries(w: Workload, steps: int, layer: int = 0) -> list:
    """Query of each decode step: a random walk of sigma 0.05, stored in bf16."""
    q = storage(normal((w.B, w.Hq, 1, w.D), w.cfg, layer, T_Q), w.dtype)
    out = [q]
    for s in range(1, steps):
        step = normal((w.B, w.Hq, 1, w.D), w.cfg, layer, T_WALK, s, std=0.05)
        q = storage(q.float().numpy() + step, w.dtype)
        out.append(q)
    return out


# ---------------------------------------------------------------------------
# prefill (workload 5)
# ---------------------------------------------------------------------------

def _rope(x: np.ndarray, base: float = 500000.0) -> np.ndarray:
    """Rotate-half RoPE over the last dim of x: [..., T, D], positions 0..T-1."""
    T, D = x.shape[-2], x.shape[-1]
    half = D // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / D)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half].astype(np.float64), x[..., half:].astype(np.float64)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def prefill_inputs(w: Workload, L: Optional[int] = None, layer: int = 0) -> Dict[str, object]:
    """Hidden states, producer weights, W_K and the RoPE'd Q, K, V of one layer."""
    L = w.L if L is None else L
    H = normal((w.B, L, w.E), w.cfg, layer, T_H)
    Hs = storage(H, w.dtype)
    Hf = Hs.float().numpy()
    out = {"workload": w, "L": L, "h": Hs, "w_k": storage(_w_k(w, layer), w.dtype)}
    out.update(producer_weights(w, layer))
    for j, (name, heads) in enumerate((("q", w.Hq), ("k_cache", w.Hkv), ("v_cache", w.Hkv))):
        W = storage(normal((w.E, heads * w.D), w.cfg, layer, T_WQKV, j, std=0.02), w.dtype)
        x = (Hf.reshape(-1, w.E) @ W.float().numpy()).reshape(w.B, L, heads, w.D)
        x = x.transpose(0, 2, 1, 3)                     # [B, heads, L, D]
        if name != "v_cache":
            x = _rope(x)
        out[name] = storage(np.ascontiguousarray(x, dtype=np.float32), w.dtype)
    return out
