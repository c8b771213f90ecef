"""GPU parity of the selected-row fetch from a KV cache in pinned host memory.

TokenButler's arXiv abstract compares decode latency against dense attention with the KV
cache offloaded to the CPU; with selection only the selected rows cross the host link.
The cache here lives in pinned host memory (torch pin_memory, allocated by the HIP
runtime); K_imp, the scores and the selection stay on the GPU.  Gates:
  * the packed rows are the oracle's gather bit for bit, slots past the count untouched;
  * attention over the packed rows (positions 0..count-1) equals attention over the
    device-resident cache with the selected index list bit for bit (same rows, same order,
    same split plan), and is within the bf16 bound of the oracle;
  * a device-resident cache (a plain gather), fp32 at D = 64, clamped out-of-range indices,
    per-query-head sets.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import ATOL, check_select_exact, np64, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import query_aware_sparse_imp_amd  # noqa: F401  (fails loudly if the library is missing)


def _pinned(t: torch.Tensor) -> torch.Tensor:
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    assert h.is_pinned()
    return h


def _iota(B, Hs, cap, dev):
    return torch.arange(cap, dtype=torch.int32, device=dev).expand(B, Hs, 1, cap).contiguous()


@pytest.mark.parametrize("L,gs", [(32768, 0), (9000, 1)])
def test_offloaded_cache_decode_step(L, gs):
    import query_aware_sparse_imp_amd as qa
    w = synthetic.WORKLOADS[2]
    Hs = qa.selection_heads(w.Hq, w.Hkv, gs)
    print(f"[fetch] host-resident cache L={L} sel_group={gs} Hs={Hs}", flush=True)
    inp = to_device(synthetic.decode_layer(w, 2, L=L))
    dev = "cuda"
    k_host, v_host = _pinned(inp["k_cache"]), _pinned(inp["v_cache"])
    kimp = torch.empty(w.B, w.Hkv, L, w.dprime, dtype=w.dtype, device=dev)
    qa.butler_project_keys(inp["k_cache_d"], inp["w_k_d"], kimp, 0, L)
    scores = torch.empty(w.B, Hs, 1, L, dtype=torch.float32, device=dev)
    hist = torch.zeros(w.B, Hs, 1, 2048, dtype=torch.int32, device=dev)
    qa.butler_score(qa.BUTLER_SCORE_RAW, inp["q_imp_d"], kimp, scores, Hkv=w.Hkv, L=L,
                    radix_hist=hist, sel_group=gs)
    cap = w.cap(L)
    idx = torch.full((w.B, Hs, 1, cap), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(w.B, Hs, 1, dtype=torch.int32, device=dev)
    qa.butler_select_topk(scores, w.budget_num, w.budget_den, w.n_sink, w.n_window, cnt,
                          idx=idx, radix_hist=hist)
    sentinel = torch.tensor(7.0, dtype=w.dtype)
    k_sel = torch.full((w.B, Hs, cap, w.D), float(sentinel), dtype=w.dtype, device=dev)
    v_sel = torch.full_like(k_sel, float(sentinel))
    qa.butler_fetch_rows(idx, cnt, k_host, v_host, k_sel, v_sel, Hq=w.Hq, sel_group=gs)
    out_packed = torch.empty(w.B, w.Hq, 1, w.D, dtype=torch.float32, device=dev)
    qa.butler_sparse_decode_attn(inp["q_d"], k_sel, v_sel, out_packed, L=cap,
                                 idx=_iota(w.B, Hs, cap, dev), count=cnt, softmax_scale=w.scale)
    out_direct = torch.empty_like(out_packed)
    qa.butler_sparse_decode_attn(inp["q_d"], inp["k_cache_d"], inp["v_cache_d"], out_direct, L=L,
                                 idx=idx, count=cnt, softmax_scale=w.scale, sel_group=gs)
    torch.cuda.synchronize()
    check_select_exact(idx, cnt, np64(scores), w.budget_num, w.budget_den, w.n_sink, w.n_window)
    ic, cc = idx.cpu().numpy(), cnt.cpu().numpy()
    sets = [[ic[b, j, 0, :cc[b, j, 0]] for j in range(Hs)] for b in range(w.B)]
    want_k, want_v = oracle.fetch_rows(np64(inp["k_cache"]), np64(inp["v_cache"]), sets, w.Hq,
                                       cap, sel_group=gs)
    got_k, got_v = np64(k_sel), np64(v_sel)
    for b in range(w.B):
        for j in range(Hs):
            n = cc[b, j, 0]
            assert np.array_equal(got_k[b, j, :n], want_k[b, j, :n]), (b, j)
            assert np.array_equal(got_v[b, j, :n], want_v[b, j, :n]), (b, j)
            assert (got_k[b, j, n:] == 7.0).all() and (got_v[b, j, n:] == 7.0).all(), (b, j)
    assert torch.equal(out_packed, out_direct), "same rows in the same order: same output"
    # and against the oracle over the sets
    o = out_packed.cpu().double().numpy()[:, :, 0]
    want = oracle.sparse_decode_attn(np64(inp["q"])[:, :, 0], np64(inp["k_cache"]),
                                     np64(inp["v_cache"]), sets, w.scale, sel_group=gs)
    err = float(np.abs(o - want).max())
    assert err <= ATOL[w.dtype], err
    print(f"  fetched {int(cc.sum())} rows per tensor; attention max-abs {err:.2e}", flush=True)


def test_device_cache_gather_fp32_and_clamped_indices():
    """A device-resident cache (plain gather), fp32 at D = 64, with ragged counts, a count
    above cap and index entries outside [0, L_cap) (clamped to the last row)."""
    import query_aware_sparse_imp_amd as qa
    dev = "cuda"
    B, Hq, Hkv, L_cap, D, cap = 2, 4, 2, 777, 64, 300
    g = torch.Generator().manual_seed(3)
    k = torch.randn(B, Hkv, L_cap, D, generator=g)
    v = torch.randn(B, Hkv, L_cap, D, generator=g)
    idx = torch.randint(0, L_cap, (B, Hkv, 1, cap), generator=g, dtype=torch.int32)
    idx[0, 0, 0, 5] = -3
    idx[1, 1, 0, 7] = L_cap + 40
    cnt = torch.tensor([[[1], [299]], [[cap + 50], [17]]], dtype=torch.int32)
    for where in ("device", "pinned"):
        kc = k.to(dev) if where == "device" else _pinned(k)
        vc = v.to(dev) if where == "device" else _pinned(v)
        ks = torch.full((B, Hkv, cap, D), -9.0, device=dev)
        vs = torch.full_like(ks, -9.0)
        qa.butler_fetch_rows(idx.to(dev), cnt.to(dev), kc, vc, ks, vs, Hq=Hq)
        torch.cuda.synchronize()
        clamped = idx.clamp(0, L_cap - 1).numpy()
        sets = [[clamped[b, j, 0, :min(int(cnt[b, j, 0]), cap)] for j in range(Hkv)]
                for b in range(B)]
        wk, wv = oracle.fetch_rows(k.double().numpy(), v.double().numpy(), sets, Hq, cap)
        gk, gv = ks.cpu().double().numpy(), vs.cpu().double().numpy()
        for b in range(B):
            for j in range(Hkv):
                n = min(int(cnt[b, j, 0]), cap)
                assert np.array_equal(gk[b, j, :n], wk[b, j, :n]), (where, b, j)
                assert np.array_equal(gv[b, j, :n], wv[b, j, :n]), (where, b, j)
                assert (gk[b, j, n:] == -9.0).all(), (where, b, j)
        print(f"  {where}: ragged rows packed exactly", flush=True)


def test_pageable_host_memory_is_rejected():
    """Pageable host memory never reaches a kernel: the binding refuses an unpinned CPU
    tensor, and the C entry point itself answers INVALID_ARG for such a pointer.  (The
    count is 0, so even a launch would read no cache row.)"""
    import query_aware_sparse_imp_amd as qa
    dev = "cuda"
    k = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)            # pageable
    idx = torch.zeros(1, 1, 1, 8, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, 1, 1, dtype=torch.int32, device=dev)
    ks = torch.empty(1, 1, 8, 64, dtype=torch.bfloat16, device=dev)
    vs = torch.empty_like(ks)
    with pytest.raises(ValueError):
        qa.butler_fetch_rows(idx, cnt, k, k.clone(), ks, vs, Hq=1)
    arr = np.zeros(1 * 1 * 64 * 64 + 64, dtype=np.uint16)
    base = arr.ctypes.data + (-arr.ctypes.data) % 16                  # 16-byte aligned
    rc = qa.lib.butler_fetch_rows(None, 1, idx.data_ptr(), cnt.data_ptr(), base, base,
                                  ks.data_ptr(), vs.data_ptr(), 1, 1, 1, 0, 64, 64, 8)
    assert rc == -1
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 64), (torch.float32, 128)])
def test_fetch_rows_row_widths(dtype, D):
    """The other row widths of the fetch (8 and 32 sixteen-byte pieces per row), from
    pinned host memory, per query head (B = 1, 4 query heads on 2 KV heads)."""
    import query_aware_sparse_imp_amd as qa
    dev = "cuda"
    B, Hq, Hkv, L_cap, cap = 1, 4, 2, 5000, 1500
    g = torch.Generator().manual_seed(D)
    k = torch.randn(B, Hkv, L_cap, D, generator=g).to(dtype)
    v = torch.randn(B, Hkv, L_cap, D, generator=g).to(dtype)
    idx = torch.stack([torch.sort(torch.randperm(L_cap, generator=g)[:cap])[0]
                       for _ in range(Hq)]).to(torch.int32).reshape(B, Hq, 1, cap)
    cnt = torch.tensor([[[cap], [1], [777], [0]]], dtype=torch.int32)
    ks = torch.full((B, Hq, cap, D), 3.0, dtype=dtype, device=dev)
    vs = torch.full_like(ks, 3.0)
    qa.butler_fetch_rows(idx.to(dev), cnt.to(dev), _pinned(k), _pinned(v), ks, vs, Hq=Hq,
                         sel_group=1)
    torch.cuda.synchronize()
    sets = [[idx[0, j, 0, :int(cnt[0, j, 0])].numpy() for j in range(Hq)]]
    wk, wv = oracle.fetch_rows(np64(k), np64(v), sets, Hq, cap, sel_group=1)
    gk, gv = np64(ks), np64(vs)
    for j in range(Hq):
        n = int(cnt[0, j, 0])
        assert np.array_equal(gk[0, j, :n], wk[0, j, :n]) and np.array_equal(gv[0, j, :n], wv[0, j, :n])
        assert (gk[0, j, n:] == 3.0).all() and (gv[0, j, n:] == 3.0).all()
    print(f"  {dtype} D={D}: packed rows exact", flush=True)
