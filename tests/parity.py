"""Stage-chained parity helpers shared by the GPU tests.

Selection is discontinuous, so each GPU stage is compared with the oracle fed the
GPU's own upstream result (after that upstream result passed its own gate):

  project  : bit-exact -- K_imp is the exact dot product rounded once, as in the oracle
  score    : RAW bit-exact (float64-exact sum rounded once to float32); SOFTVOTE
             relative error <= 1e-5 of the score
  select   : bit-exact set, order and count on the GPU's scores
  attend   : max-abs <= 2e-2 (bf16) / 1e-4 (fp32) on the GPU's index lists
  chain    : the fully independent oracle chain must select the same sets except for
             tokens whose oracle score lies within 1e-5 (relative) of the k-th score
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import query_aware_sparse_imp_amd as qa

ATOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else \
        t.detach().cpu().double().numpy()


def dstr(dtype) -> str:
    return "bf16" if dtype == torch.bfloat16 else "f32"


def check_project(kimp_gpu: torch.Tensor, k_cache: torch.Tensor, w_k: torch.Tensor,
                  lo: int, hi: int, heads=None) -> int:
    """Compares K_imp rows [lo, hi) with the oracle: every element must be identical
    (both sides round the exact dot product once).  Returns the rows compared."""
    B, Hkv = k_cache.shape[:2]
    heads = heads or [(b, g) for b in range(B) for g in range(Hkv)]
    ndiff = 0
    for (b, g) in heads:
        want = oracle.project_keys(np64(k_cache[b, g, lo:hi]), np64(w_k), dstr(k_cache.dtype))
        got = np64(kimp_gpu[b, g, lo:hi])
        bad = int((got != want).sum())
        if bad:
            u = oracle.ulps_bf16(got, want).max() if k_cache.dtype == torch.bfloat16 else None
            raise AssertionError(f"K_imp differs in {bad} elements at head {(b, g)} "
                                 f"(max ulps {u})")
        ndiff += hi - lo
    return ndiff


def threshold_band(scores_row: np.ndarray, x: int, mag_row: np.ndarray) -> np.ndarray:
    """Tokens whose score lies within 1e-5 relative of the x-th largest score.  The
    band uses max(|tau|, the magnitude sum of the token's dot product), the error
    bound of a dot product, so it does not vanish when tau is near zero."""
    if x <= 0 or x >= len(scores_row):
        return np.zeros(len(scores_row), bool)
    s = np.where(np.isnan(scores_row), -np.inf, scores_row)
    tau = np.sort(s)[::-1][x - 1]
    scale = np.maximum(abs(tau), mag_row)
    return np.abs(s - tau) <= 1e-5 * scale


def check_select_exact(idx_gpu, count_gpu, scores_gpu_np, num, den, n_sink, n_window,
                       causal=False, q_pos0=0, rows=None, exclude_forced=False) -> None:
    """GPU selection == oracle selection on the GPU's own scores (bit-exact)."""
    B, Hkv, Lq, L = scores_gpu_np.shape
    cnt = count_gpu.cpu().numpy()
    idx = idx_gpu.cpu().numpy() if idx_gpu is not None else None
    rows = rows or [(b, g, i) for b in range(B) for g in range(Hkv) for i in range(Lq)]
    for (b, g, i) in rows:
        L_r = min(q_pos0 + i + 1, L) if causal else L
        want = oracle.select(scores_gpu_np[b, g, i, :L_r], oracle.budget(L_r, num, den),
                             n_sink, n_window, exclude_forced)
        assert cnt[b, g, i] == len(want), f"count {cnt[b, g, i]} != {len(want)} at {(b, g, i)}"
        if idx is not None:
            got = idx[b, g, i, :cnt[b, g, i]]
            assert np.array_equal(got, want), f"index list differs at {(b, g, i)}"


def bitmask_to_sets(bitmask: torch.Tensor, L: int) -> np.ndarray:
    words = bitmask.cpu().numpy().astype(np.uint32)
    bits = np.unpackbits(words.view(np.uint8).reshape(*words.shape, 4), axis=-1,
                         bitorder="little")
    return bits.reshape(*words.shape[:-1], -1)[..., :L].astype(bool)


def check_attend(out_gpu, q, k_cache, v_cache, sets, scale, dtype, heads=None) -> float:
    """GPU attention vs oracle attention on the same selected sets; returns max-abs."""
    o = out_gpu.cpu().double().numpy()
    B, Hq, Lq, D = q.shape
    Hkv = k_cache.shape[1]
    R = Hq // Hkv
    qn = np64(q)
    worst = 0.0
    heads = heads or [(b, g, i) for b in range(B) for g in range(Hkv) for i in range(Lq)]
    for (b, g, i) in heads:
        sel = np.asarray(sets(b, g, i), np.int64)
        want = oracle.attend(qn[b, g * R:(g + 1) * R, i], np64(k_cache[b, g, sel]),
                             np64(v_cache[b, g, sel]), scale)
        err = float(np.max(np.abs(o[b, g * R:(g + 1) * R, i] - want)))
        worst = max(worst, err)
    assert worst <= ATOL[dtype], f"attention max-abs {worst} > {ATOL[dtype]}"
    return worst


def decode_step_gpu(inp: dict, kimp: torch.Tensor, L: int, mode: int, q_imp=None, slot=0,
                    dense=False, use_hist=True) -> dict:
    """score -> select -> attend on the GPU for one decode layer at context L (with the
    scorer's first-digit histogram handed to the selection unless use_hist is False)."""
    w = inp["workload"]
    dev = kimp.device if kimp is not None else inp["k_cache_d"].device
    B, Hkv = w.B, w.Hkv
    scores = torch.empty(B, Hkv, 1, L, dtype=torch.float32, device=dev)
    k_d, v_d, q_d = inp["k_cache_d"], inp["v_cache_d"], inp["q_d"]
    if dense:
        num, den = 1, 1
    else:
        num, den = w.budget_num, w.budget_den
    cap = min(L, (L * num) // den + w.n_sink + w.n_window)
    hist = torch.zeros(B, Hkv, 1, 2048, dtype=torch.int32, device=dev) if use_hist else None
    if mode == qa.BUTLER_SCORE_RAW:
        qa.butler_score(mode, q_imp, kimp, scores, Hkv=Hkv, L=L, slot=slot, radix_hist=hist)
    else:
        qa.butler_score(mode, q_d, k_d, scores, Hkv=Hkv, L=L, softmax_scale=w.scale,
                        radix_hist=hist)
    idx = torch.full((B, Hkv, 1, cap), -1, dtype=torch.int32, device=dev)
    count = torch.zeros(B, Hkv, 1, dtype=torch.int32, device=dev)
    qa.butler_select_topk(scores, num, den, w.n_sink, w.n_window, count, idx=idx,
                          radix_hist=hist)
    if hist is not None:
        torch.cuda.synchronize()
        assert int(hist.abs().sum()) == 0, "the selection must leave the histogram zeroed"
    out = torch.empty(B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
    qa.butler_sparse_decode_attn(q_d, k_d, v_d, out, L=L, idx=idx, count=count,
                                 softmax_scale=w.scale)
    return {"scores": scores, "idx": idx, "count": count, "out": out, "num": num, "den": den}


def pv_rounding_bound(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, sets,
                      scale: float, sel_group: int = 0) -> np.ndarray:
    """Per-element gate [B, Hq, D] for two GPU attention outputs over the same selected sets
    that split them differently (the fused select+attend call against the separate calls).

    The matrix-core P.V rounds every probability p_t = exp(z_t - m) to bf16 (8 significant
    bits: a rounding error of at most 2^-8 p_t, uniform over +-half an ulp, so of standard
    deviation at most 2^-8 p_t / sqrt(3)), while the normaliser sums the unrounded p_t.
    The two outputs use different running maxima m, so their roundings are independent;
    element d of head h differs by sum_t (e1_t - e2_t) v_td / sum_t p_t, whose standard
    deviation is at most sqrt(2) * 2^-8 / sqrt(3) * sqrt(sum_t p_t^2 v_td^2) / sum_t p_t.
    The gate is six of those (a chance below 2e-9 per element) plus 1e-5 for float32
    summation order, computed from the row's own probabilities (float64, the oracle's
    logits).  It never exceeds the worst case 2 * 2^-8 * sum_t p_t |v_td| / sum_t p_t.
    sets(b, j, i) is the selected set of selection head j."""
    qn, kn, vn = np64(q), np64(k_cache), np64(v_cache)
    B, Hq, _, D = qn.shape
    Hkv = kn.shape[1]
    R = Hq // Hkv
    gs = sel_group or R
    sig = math.sqrt(2.0) * 2.0 ** -8 / math.sqrt(3.0)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            sel = np.asarray(sets(b, h // gs, 0), np.int64)
            kr, vr = kn[b, h // R, sel], vn[b, h // R, sel]
            z = (kr @ qn[b, h, 0]) * scale
            p = np.exp(z - z.max())
            stat = 6.0 * sig * np.sqrt((p[:, None] ** 2 * vr ** 2).sum(0)) / p.sum()
            worst = 2.0 * 2.0 ** -8 * (p[:, None] * np.abs(vr)).sum(0) / p.sum()
            out[b, h] = np.minimum(stat, worst) + 1e-5
    return out


def check_pv_rounding(out_a: torch.Tensor, out_b: torch.Tensor, bound: np.ndarray) -> float:
    """|out_a - out_b| within the per-element gate of pv_rounding_bound; returns the largest
    difference."""
    d = np.abs(out_a.cpu().double().numpy()[:, :, 0] - out_b.cpu().double().numpy()[:, :, 0])
    bad = d > bound
    assert not bad.any(), (f"fused vs separate: {int(bad.sum())} elements over the gate, "
                           f"worst {float((d - bound).max()):.3e} above it")
    return float(d.max())


def to_device(inp: dict, device="cuda") -> dict:
    for key in ("k_cache", "v_cache", "q", "w_k", "q_imp"):
        if key in inp:
            inp[key + "_d"] = inp[key].to(device)
    return inp


def scale_of(D: int) -> float:
    return 1.0 / math.sqrt(D)
