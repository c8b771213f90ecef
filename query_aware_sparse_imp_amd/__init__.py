"""Python binding of libbutler: query-aware sparse decode on AMD MI355X (gfx950).

Argument marshalling only.  Every function here takes torch tensors that already
live on the GPU, checks their shapes, dtypes and contiguity, and calls the C entry
point of the same name in ``libbutler.so`` with raw device pointers, sizes and the
current HIP stream.  All compute happens in the library's HIP kernels; there is no
fallback.  Importing this package fails loudly if the library has not been built
(``python query_aware_sparse_imp_amd/csrc/build.py``).
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional, Tuple

import torch

__all__ = [
    "BUTLER_OK", "BUTLER_SCORE_RAW", "BUTLER_SCORE_SOFTVOTE", "ButlerError", "lib", "LIB_PATH",
    "butler_project_keys", "butler_produce_queries", "butler_score", "butler_project_and_score",
    "butler_score_tokens",
    "butler_select_topk",
    "butler_sparse_decode_attn", "butler_select_attend", "butler_select_attend_noalloc",
    "butler_selection_cache",
    "butler_expand_neighbors",
    "butler_status_string",
    "butler_abi_version", "declared_symbols", "workspace_bytes",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbutler.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "butler.h")

BUTLER_OK = 0
BUTLER_F32, BUTLER_BF16 = 0, 1
BUTLER_SCORE_RAW, BUTLER_SCORE_SOFTVOTE = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python query_aware_sparse_imp_amd/csrc/build.py`")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.POINTER(ctypes.c_size_t)
_SIGS = {
    "butler_status_string": ([_i], ctypes.c_char_p),
    "butler_abi_version": ([], _i),
    "butler_project_keys": ([_vp, _i, _vp, _vp, _vp] + [_i] * 7, _i),
    "butler_produce_queries": ([_vp, _i, _vp, _vp, _vp, _vp] + [_i] * 7 + [_f, _vp, _sz], _i),
    "butler_score": ([_vp, _i, _i, _vp, _vp, _vp, _vp, _vp] + [_i] * 12 + [_f, _vp, _sz], _i),
    "butler_project_and_score": ([_vp, _i] + [_vp] * 7 + [_i] * 10, _i),
    "butler_score_tokens": ([_vp, _i] + [_vp] * 7 + [_i] * 12, _i),
    "butler_select_topk": ([_vp, _vp, _vp, _vp] + [_i] * 5 + [_vp, _vp, _vp] + [_i] * 7 +
                           [_vp, _sz], _i),
    "butler_selection_cache": ([_vp, _i, _vp, _vp, _vp] + [_i] * 5 + [_f], _i),
    "butler_select_attend": ([_vp, _i, _vp, _vp] + [_i] * 5 + [_vp] * 6 + [_i] * 8 +
                             [_f, _vp, _sz], _i),
    "butler_select_attend_noalloc": ([_vp, _i, _vp, _vp] + [_i] * 5 + [_vp] * 6 + [_i] * 8 +
                                     [_f], _i),
    "butler_expand_neighbors": ([_vp] * 5 + [_i] * 7, _i),
    "butler_sparse_decode_attn": ([_vp, _i] + [_vp] * 7 + [_i] * 10 + [_f, _vp, _sz], _i),
    "butler_fetch_rows": ([_vp, _i] + [_vp] * 6 + [_i] * 7, _i),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class ButlerError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {butler_status_string(status)} ({status})")
        self.status = status


def butler_status_string(status: int) -> str:
    return lib.butler_status_string(status).decode()


def butler_abi_version() -> int:
    return lib.butler_abi_version()


def declared_symbols() -> list:
    """Function names declared in include/butler.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(butler_\w+)\s*\(", text)))


def _check_hist(h: Optional[torch.Tensor], rows: tuple) -> None:
    if h is not None and (tuple(h.shape) != (*rows, 2048) or h.element_size() != 4):
        raise ValueError("radix_hist must be 32-bit [B, Hs, Lq, 2048]")


def _check_keep(k: Optional[torch.Tensor], shape: tuple) -> None:
    if k is not None and (tuple(k.shape) != shape or k.dtype != torch.int32):
        raise ValueError("keep must be int32 [B, Hs]")


def selection_heads(Hq: int, Hkv: int, sel_group: int = 0) -> int:
    """Hs, the selected sets per batch entry: sel_group query heads share one set (0: the
    Hq // Hkv heads of a KV head; 1: one set per query head)."""
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    R = Hq // Hkv
    g = R if sel_group == 0 else sel_group
    if g <= 0 or R % g:
        raise ValueError(f"sel_group must be 0 or a divisor of Hq / Hkv = {R}")
    return Hq // g


def _check(fn: str, status: int) -> None:
    if status != BUTLER_OK:
        raise ButlerError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BUTLER_BF16
    if t.dtype == torch.float32:
        return BUTLER_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _ptr_host_ok(t: torch.Tensor) -> int:
    """A device tensor, or a pinned host tensor (which the GPU can map)."""
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError("tensor must live on the GPU or in pinned host memory")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# Workspaces: one zero-initialised buffer per (entry point, device, key).  The library
# leaves the accumulators inside a workspace zero after every call, so a buffer is reused
# by every later call with the same key on one stream.  The key is the call shape, except
# for the selection calls, whose state between calls depends only on their rows: they key
# by rows and grow the buffer (a new zeroed one) when a longer row needs more.
_WS: Dict[tuple, torch.Tensor] = {}


def _workspace(name: str, nbytes: int, device: torch.device, shape: tuple):
    """(pointer, size cell) of the workspace to pass; (None, None) when none is needed."""
    if nbytes == 0:
        return None, None
    key = (name, device.index if device.index is not None else torch.cuda.current_device(),
           shape)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf.data_ptr(), ctypes.c_size_t(buf.numel())


def _byref(n):
    return None if n is None else ctypes.byref(n)


def workspace_bytes(query) -> int:
    """Runs a size query: ``query(ws_ptr, ws_bytes_ptr)`` with ws = NULL."""
    n = ctypes.c_size_t(0)
    _check("workspace query", query(None, ctypes.byref(n)))
    return n.value


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def butler_project_keys(k_cache: torch.Tensor, w_k: torch.Tensor, kimp: torch.Tensor,
                        pos0: int, n_new: int, stream=None) -> None:
    """kimp[:, :, pos0:pos0+n_new] = k_cache[:, :, pos0:pos0+n_new] @ w_k (see butler.h)."""
    B, Hkv, L_cap, D = k_cache.shape
    dp = w_k.shape[1]
    if w_k.shape != (D, dp) or kimp.shape != (B, Hkv, L_cap, dp):
        raise ValueError("shape mismatch")
    if not (k_cache.dtype == w_k.dtype == kimp.dtype):
        raise TypeError("k_cache, w_k and kimp must share a dtype")
    _check("butler_project_keys", lib.butler_project_keys(
        _stream(stream), _dtype_code(k_cache), _ptr(k_cache), _ptr(w_k), _ptr(kimp),
        B, Hkv, L_cap, D, dp, pos0, n_new))


def butler_produce_queries(h: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
                           q_imp: torch.Tensor, ln_eps: float = 1e-5, stream=None) -> None:
    """q_imp [B, Hq, G, Lq, d'] = reshape(relu(LN(h) @ w1.T) @ w2.T) (see butler.h).
    w1 [F, E] and w2 [Hq*G*d', F] are in the [out, in] layout of a PyTorch Linear."""
    B, Lq, E = h.shape
    F = w1.shape[0]
    _, Hq, G, Lq2, dp = q_imp.shape
    if w1.shape != (F, E) or w2.shape != (Hq * G * dp, F) or Lq2 != Lq or q_imp.shape[0] != B:
        raise ValueError("shape mismatch")
    dt = _dtype_code(h)
    args = (dt, _ptr(h), _ptr(w1), _ptr(w2), _ptr(q_imp), B, Lq, E, F, Hq, G, dp, ln_eps)
    need = workspace_bytes(lambda ws, n: lib.butler_produce_queries(_stream(stream), *args, ws, n))
    ws, n = _workspace("produce", need, h.device, (B, Lq, E, F, Hq, G, dp))
    _check("butler_produce_queries",
           lib.butler_produce_queries(_stream(stream), *args, ws, _byref(n)))


def butler_score(mode: int, q: torch.Tensor, keys: torch.Tensor, scores: torch.Tensor, *,
                 Hkv: int, L: int, slot: int = 0, q_pos0: int = 0, causal: bool = False,
                 softmax_scale: float = 1.0, radix_hist: Optional[torch.Tensor] = None,
                 keep: Optional[torch.Tensor] = None, sel_group: int = 0, stream=None) -> None:
    """Importance scores [B, Hs, Lq, L] (see butler.h).

    RAW: q = q_imp [B, Hq, G, Lq, d'], keys = kimp [B, Hkv, L_cap, d'].
    SOFTVOTE: q = [B, Hq, Lq, D], keys = k_cache [B, Hkv, L_cap, D].
    sel_group: query heads per selected set (0: all Hq // Hkv of a KV head, Hs = Hkv;
    1: per query head, Hs = Hq).
    radix_hist: optional zero-filled int32/uint32 [B, Hs, Lq, 2048] that collects the
    first radix digit of every score for butler_select_topk.
    keep: optional int32 [B, Hs] from butler_selection_cache; rows with keep != 0 are
    skipped (single-row calls).
    """
    if mode == BUTLER_SCORE_RAW:
        B, Hq, G, Lq, dk = q.shape
    else:
        B, Hq, Lq, dk = q.shape
        G = 1
    Bk, Hk, L_cap, dk2 = keys.shape
    Hs = selection_heads(Hq, Hkv, sel_group)
    if (Bk, Hk, dk2) != (B, Hkv, dk) or scores.shape != (B, Hs, Lq, L):
        raise ValueError("shape mismatch")
    if q.dtype != keys.dtype or scores.dtype != torch.float32:
        raise TypeError("dtype mismatch")
    _check_hist(radix_hist, (B, Hs, Lq))
    _check_keep(keep, (B, Hs))
    args = (mode, _dtype_code(q), _ptr(q), _ptr(keys), _ptr(scores), _ptr(radix_hist),
            _ptr(keep), B, Hq, Hkv, sel_group, G, slot, Lq, L, L_cap, dk, q_pos0, int(causal),
            softmax_scale)
    need = workspace_bytes(lambda ws, n: lib.butler_score(_stream(stream), *args, ws, n))
    ws, n = _workspace("score", need, q.device, tuple(args[7:]))
    _check("butler_score", lib.butler_score(_stream(stream), *args, ws, _byref(n)))


def butler_project_and_score(q_imp: torch.Tensor, k_cache: torch.Tensor, w_k: torch.Tensor,
                             kimp: torch.Tensor, scores: torch.Tensor, *, Hkv: int, L: int,
                             slot: int = 0, radix_hist: Optional[torch.Tensor] = None,
                             keep: Optional[torch.Tensor] = None, sel_group: int = 0,
                             stream=None) -> None:
    """Projects key row L - 1 into kimp and scores tokens [0, L) in one launch: the same as
    butler_project_keys(pos0=L-1, n_new=1) then butler_score(RAW) (see butler.h).
    q_imp [B, Hq, G, 1, d'], k_cache [B, Hkv, L_cap, D], w_k [D, d'],
    kimp [B, Hkv, L_cap, d'], scores [B, Hs, 1, L]; sel_group as in butler_score."""
    B, Hq, G, Lq, dp = q_imp.shape
    Bk, Hk, L_cap, D = k_cache.shape
    Hs = selection_heads(Hq, Hkv, sel_group)
    if Lq != 1 or (Bk, Hk) != (B, Hkv) or w_k.shape != (D, dp):
        raise ValueError("shape mismatch")
    if kimp.shape != (B, Hkv, L_cap, dp) or scores.shape != (B, Hs, 1, L):
        raise ValueError("shape mismatch")
    if not (q_imp.dtype == k_cache.dtype == w_k.dtype == kimp.dtype) or \
            scores.dtype != torch.float32:
        raise TypeError("dtype mismatch")
    _check_hist(radix_hist, (B, Hs, 1))
    _check_keep(keep, (B, Hs))
    _check("butler_project_and_score", lib.butler_project_and_score(
        _stream(stream), _dtype_code(q_imp), _ptr(q_imp), _ptr(k_cache), _ptr(w_k), _ptr(kimp),
        _ptr(scores), _ptr(radix_hist), _ptr(keep), B, Hq, Hkv, sel_group, G, slot, L, L_cap, D,
        dp))


def butler_score_tokens(q_imp: torch.Tensor, kimp: torch.Tensor, scores: torch.Tensor, *,
                        Hkv: int, L: int, t_begin: int, t_end: int, slot: int = 0,
                        k_cache: Optional[torch.Tensor] = None,
                        w_k: Optional[torch.Tensor] = None,
                        radix_hist: Optional[torch.Tensor] = None,
                        keep: Optional[torch.Tensor] = None, sel_group: int = 0,
                        stream=None) -> None:
    """Raw scores of tokens [t_begin, t_end) of decode rows of length L (see butler.h);
    with k_cache and w_k (t_end == L) row L - 1 of kimp is projected first.
    q_imp [B, Hq, G, 1, d'], kimp [B, Hkv, L_cap, d'], scores [B, Hs, 1, L]."""
    B, Hq, G, Lq, dp = q_imp.shape
    Bk, Hk, L_cap, dp2 = kimp.shape
    Hs = selection_heads(Hq, Hkv, sel_group)
    if Lq != 1 or (Bk, Hk, dp2) != (B, Hkv, dp) or scores.shape != (B, Hs, 1, L):
        raise ValueError("shape mismatch")
    D = 0
    if k_cache is not None or w_k is not None:
        if k_cache is None or w_k is None:
            raise ValueError("k_cache and w_k go together")
        D = k_cache.shape[3]
        if k_cache.shape != (B, Hkv, L_cap, D) or w_k.shape != (D, dp):
            raise ValueError("shape mismatch")
        if not (k_cache.dtype == w_k.dtype == kimp.dtype):
            raise TypeError("dtype mismatch")
    if q_imp.dtype != kimp.dtype or scores.dtype != torch.float32:
        raise TypeError("dtype mismatch")
    _check_hist(radix_hist, (B, Hs, 1))
    _check_keep(keep, (B, Hs))
    _check("butler_score_tokens", lib.butler_score_tokens(
        _stream(stream), _dtype_code(q_imp), _ptr(q_imp), _ptr(kimp), _ptr(k_cache), _ptr(w_k),
        _ptr(scores), _ptr(radix_hist), _ptr(keep), B, Hq, Hkv, sel_group, G, slot, L, L_cap, D,
        dp, int(t_begin), int(t_end)))


def butler_select_topk(scores: torch.Tensor, budget_num: int, budget_den: int, n_sink: int,
                       n_window: int, count: torch.Tensor, idx: Optional[torch.Tensor] = None,
                       bitmask: Optional[torch.Tensor] = None, *, q_pos0: int = 0,
                       causal: bool = False, radix_hist: Optional[torch.Tensor] = None,
                       keep: Optional[torch.Tensor] = None,
                       budget_excludes_forced: bool = False, stream=None) -> None:
    """Top-x + sink + window per row of scores [B, Hs, Lq, L] (see butler.h).  keep: as in
    butler_score; kept rows leave idx, bitmask and count as they were.
    budget_excludes_forced: the top-x ranks only the tokens outside the sink and the window."""
    B, Hkv, Lq, L = scores.shape
    cap = 0
    if idx is not None:
        if idx.shape[:3] != (B, Hkv, Lq) or idx.dtype != torch.int32:
            raise ValueError("idx must be int32 [B, Hkv, Lq, cap]")
        cap = idx.shape[3]
    if bitmask is not None:
        if bitmask.shape != (B, Hkv, Lq, (L + 31) // 32) or bitmask.dtype not in (torch.int32, torch.uint32):
            raise ValueError("bitmask must be 32-bit [B, Hkv, Lq, ceil(L/32)]")
    if count.shape != (B, Hkv, Lq) or count.dtype != torch.int32:
        raise ValueError("count must be int32 [B, Hkv, Lq]")
    _check_hist(radix_hist, (B, Hkv, Lq))
    _check_keep(keep, (B, Hkv))
    args = (_ptr(scores), _ptr(radix_hist), _ptr(keep), budget_num, budget_den, n_sink, n_window,
            int(bool(budget_excludes_forced)), _ptr(idx), _ptr(bitmask), _ptr(count), B, Hkv, Lq,
            L, cap, q_pos0, int(causal))
    need = workspace_bytes(lambda ws, n: lib.butler_select_topk(_stream(stream), *args, ws, n))
    ws, n = _workspace("select", need, scores.device, (B * Hkv * Lq,))
    _check("butler_select_topk",
           lib.butler_select_topk(_stream(stream), *args, ws, _byref(n)))


def butler_sparse_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              out: torch.Tensor, *, L: int, idx: Optional[torch.Tensor] = None,
                              count: Optional[torch.Tensor] = None,
                              bitmask: Optional[torch.Tensor] = None, q_pos0: int = 0,
                              softmax_scale: float, sel_group: int = 0, stream=None) -> None:
    """Attention of q [B, Hq, Lq, D] over the selected tokens (see butler.h): idx
    [B, Hs, Lq, cap] and count [B, Hs, Lq], or bitmask [B, Hs, Lq, ceil(L/32)];
    sel_group as in butler_score."""
    B, Hq, Lq, D = q.shape
    Bk, Hkv, L_cap, D2 = k_cache.shape
    if (Bk, D2) != (B, D) or v_cache.shape != k_cache.shape or out.shape != (B, Hq, Lq, D):
        raise ValueError("shape mismatch")
    if out.dtype != torch.float32 or not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    Hs = selection_heads(Hq, Hkv, sel_group)
    cap = 0
    if idx is not None:
        if idx.shape[:3] != (B, Hs, Lq) or count is None or count.shape != (B, Hs, Lq):
            raise ValueError("idx [B, Hs, Lq, cap] and count [B, Hs, Lq] required")
        cap = idx.shape[3]
    if bitmask is not None and tuple(bitmask.shape) != (B, Hs, Lq, (L + 31) // 32):
        raise ValueError("bitmask must be [B, Hs, Lq, ceil(L/32)]")
    args = (_dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(idx), _ptr(count),
            _ptr(bitmask), _ptr(out), B, Hq, Hkv, sel_group, D, Lq, L, L_cap, cap, q_pos0,
            softmax_scale)
    need = workspace_bytes(
        lambda ws, n: lib.butler_sparse_decode_attn(_stream(stream), *args, ws, n))
    ws, n = _workspace("attn", need, q.device, tuple(args[8:]))
    _check("butler_sparse_decode_attn",
           lib.butler_sparse_decode_attn(_stream(stream), *args, ws, _byref(n)))


def butler_select_attend(scores: torch.Tensor, budget_num: int, budget_den: int, n_sink: int,
                         n_window: int, count: torch.Tensor, idx: torch.Tensor, q: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, out: torch.Tensor, *,
                         L: int, softmax_scale: float,
                         radix_hist: Optional[torch.Tensor] = None,
                         budget_excludes_forced: bool = False, sel_group: int = 0,
                         stream=None) -> None:
    """butler_select_topk then butler_sparse_decode_attn for one decode step (see butler.h).
    scores [B, Hs, 1, L]; idx [B, Hs, 1, cap], count [B, Hs, 1] (written);
    q [B, Hq, 1, D]; caches [B, Hkv, L_cap, D]; out [B, Hq, 1, D] float32;
    sel_group as in butler_score."""
    B, Hs, Lq, Ls = scores.shape
    Bq, Hq, Lq2, D = q.shape
    Bk, Hkv, L_cap, D2 = k_cache.shape
    if Lq != 1 or Lq2 != 1 or Ls != L or (Bq, Bk, D2) != (B, B, D):
        raise ValueError("shape mismatch")
    if Hs != selection_heads(Hq, Hkv, sel_group):
        raise ValueError("scores must have Hs = Hq / sel_group selection heads")
    if v_cache.shape != k_cache.shape or out.shape != (B, Hq, 1, D):
        raise ValueError("shape mismatch")
    if idx.shape[:3] != (B, Hs, 1) or count.shape != (B, Hs, 1):
        raise ValueError("idx [B, Hs, 1, cap] and count [B, Hs, 1] required")
    if scores.dtype != torch.float32 or out.dtype != torch.float32 or \
            not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    _check_hist(radix_hist, (B, Hs, 1))
    args = (_dtype_code(q), _ptr(scores), _ptr(radix_hist), budget_num, budget_den, n_sink,
            n_window, int(bool(budget_excludes_forced)), _ptr(idx), _ptr(count), _ptr(q),
            _ptr(k_cache), _ptr(v_cache), _ptr(out), B, Hq, Hkv, sel_group, D, L, L_cap,
            idx.shape[3], float(softmax_scale))
    need = workspace_bytes(lambda ws, n: lib.butler_select_attend(_stream(stream), *args, ws, n))
    # the selection state comes first and depends on the rows only; the attention part
    # behind it is rewritten by every call
    ws, n = _workspace("select_attend", need, q.device, (B * Hs,))
    _check("butler_select_attend",
           lib.butler_select_attend(_stream(stream), *args, ws, _byref(n)))


def butler_select_attend_noalloc(scores: torch.Tensor, budget_num: int, budget_den: int,
                                 n_sink: int, n_window: int, count: torch.Tensor,
                                 idx: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                                 v_cache: torch.Tensor, out: torch.Tensor, *, L: int,
                                 softmax_scale: float, radix_hist: Optional[torch.Tensor] = None,
                                 budget_excludes_forced: bool = False, sel_group: int = 0,
                                 stream=None) -> None:
    """butler_select_attend on the library's own fixed scratch array: no workspace is
    passed or allocated (see butler.h).  Same arguments and results."""
    B, Hs, Lq, Ls = scores.shape
    Bq, Hq, Lq2, D = q.shape
    Bk, Hkv, L_cap, D2 = k_cache.shape
    if Lq != 1 or Lq2 != 1 or Ls != L or (Bq, Bk, D2) != (B, B, D):
        raise ValueError("shape mismatch")
    if Hs != selection_heads(Hq, Hkv, sel_group):
        raise ValueError("scores must have Hs = Hq / sel_group selection heads")
    if v_cache.shape != k_cache.shape or out.shape != (B, Hq, 1, D):
        raise ValueError("shape mismatch")
    if idx.shape[:3] != (B, Hs, 1) or count.shape != (B, Hs, 1):
        raise ValueError("idx [B, Hs, 1, cap] and count [B, Hs, 1] required")
    if scores.dtype != torch.float32 or out.dtype != torch.float32 or \
            not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    _check_hist(radix_hist, (B, Hs, 1))
    _check("butler_select_attend_noalloc", lib.butler_select_attend_noalloc(
        _stream(stream), _dtype_code(q), _ptr(scores), _ptr(radix_hist), budget_num, budget_den,
        n_sink, n_window, int(bool(budget_excludes_forced)), _ptr(idx), _ptr(count), _ptr(q),
        _ptr(k_cache), _ptr(v_cache), _ptr(out), B, Hq, Hkv, sel_group, D, L, L_cap,
        idx.shape[3], float(softmax_scale)))


def butler_selection_cache(q: torch.Tensor, q_ref: torch.Tensor, keep: torch.Tensor, *,
                           Hkv: int, threshold: float, sel_group: int = 0, stream=None) -> None:
    """keep[b, j] = cos(q of selection head j, q_ref of j) >= threshold; refreshes q_ref
    where not (see butler.h).  q, q_ref: [B, Hq, 1, D]; keep: int32 [B, Hs]; sel_group as
    in butler_score."""
    B, Hq, Lq, D = q.shape
    Hs = selection_heads(Hq, Hkv, sel_group)
    if q_ref.shape != q.shape or Lq != 1 or keep.shape != (B, Hs) or keep.dtype != torch.int32:
        raise ValueError("shape mismatch")
    if q_ref.dtype != q.dtype:
        raise TypeError("dtype mismatch")
    _check("butler_selection_cache", lib.butler_selection_cache(
        _stream(stream), _dtype_code(q), _ptr(q), _ptr(q_ref), _ptr(keep), B, Hq, Hkv,
        sel_group, D, float(threshold)))


def butler_expand_neighbors(idx: torch.Tensor, count: torch.Tensor, idx_out: torch.Tensor,
                            count_out: torch.Tensor, *, L: int, width: int, n_window: int,
                            stream=None) -> None:
    """Widens a reused selection with its tokens' neighbours and the window at length L
    (see butler.h).  idx: int32 [B, Hs, cap_in]; count: int32 [B, Hs];
    idx_out: int32 [B, Hs, cap_out]; count_out: int32 [B, Hs]."""
    if idx.dim() != 3 or idx_out.dim() != 3 or idx.shape[:2] != idx_out.shape[:2]:
        raise ValueError("shape mismatch")
    B, Hkv, cap_in = idx.shape
    for t in (idx, count, idx_out, count_out):
        if t.dtype != torch.int32:
            raise TypeError("int32 tensors expected")
    if count.shape != (B, Hkv) or count_out.shape != (B, Hkv):
        raise ValueError("count must be [B, Hkv]")
    _check("butler_expand_neighbors", lib.butler_expand_neighbors(
        _stream(stream), _ptr(idx), _ptr(count), _ptr(idx_out), _ptr(count_out), B, Hkv,
        int(L), cap_in, idx_out.shape[2], int(width), int(n_window)))


def butler_fetch_rows(idx: torch.Tensor, count: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, k_sel: torch.Tensor, v_sel: torch.Tensor, *,
                      Hq: int, sel_group: int = 0, stream=None) -> None:
    """Packs the selected K and V rows of each selected set into k_sel / v_sel (see
    butler.h).  k_cache, v_cache: [B, Hkv, L_cap, D] on the GPU or in pinned host memory
    (read across the host link); idx [B, Hs, 1, cap], count [B, Hs, 1] int32;
    k_sel, v_sel [B, Hs, cap, D] on the GPU."""
    B, Hkv, L_cap, D = k_cache.shape
    Hs = selection_heads(Hq, Hkv, sel_group)
    if v_cache.shape != k_cache.shape or idx.dim() != 4 or idx.shape[:3] != (B, Hs, 1):
        raise ValueError("shape mismatch")
    cap = idx.shape[3]
    if count.shape != (B, Hs, 1) or k_sel.shape != (B, Hs, cap, D) or v_sel.shape != k_sel.shape:
        raise ValueError("shape mismatch")
    if idx.dtype != torch.int32 or count.dtype != torch.int32:
        raise TypeError("idx and count must be int32")
    if not (k_cache.dtype == v_cache.dtype == k_sel.dtype == v_sel.dtype):
        raise TypeError("dtype mismatch")
    _check("butler_fetch_rows", lib.butler_fetch_rows(
        _stream(stream), _dtype_code(k_cache), _ptr(idx), _ptr(count), _ptr_host_ok(k_cache),
        _ptr_host_ok(v_cache), _ptr(k_sel), _ptr(v_sel), B, Hq, Hkv, sel_group, D, L_cap, cap))
