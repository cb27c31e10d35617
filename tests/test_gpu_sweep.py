"""Seeded random sweep of the whole path against the CPU oracle: random
geometries (1-16 query heads per KV head, d 64 or 128, bf16 or fp32),
lengths from empty to thousands of tokens, k and window from 0 up, permuted
or interleaved block placement; each case checks the fused step against its
three calls (bit for bit) and the oracle, a cached call with a wider window
at the same lengths (bit for bit the boundary call: a window never starts
below the lists' clip point), and calls on segment records at later lengths
against the oracle (ZoomR Sec. 3.4: the selection kept between semantic
boundaries, the window growing from its boundary start). Other seeds run the
same workloads through staging from pinned host pools, the no-allocation
step, dense attention, and the consensus set with its zoomed attention."""
import sys

import numpy as np
import pytest
import torch

from hierarchical_sparse_kv_amd import synth, zr
from oracle import zr_oracle as O
from tests import parity_helpers as P

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zr.lib()
    yield
    torch.cuda.synchronize()


def _dev(x):
    return torch.as_tensor(np.ascontiguousarray(x), device="cuda")


def _geometry(rng, g16=True):
    dtype = ["bf16", "f32"][rng.integers(0, 2)]
    Hkv = int([1, 2, 4, 8][rng.integers(0, 4)])
    Gs = [1, 2, 4, 8, 16] if g16 else [1, 2, 4, 8]
    G = int(Gs[rng.integers(0, len(Gs))])
    d = int([64, 128][rng.integers(0, 2)])
    return dtype, Hkv, G, d


@pytest.mark.parametrize("case", range(24))
def test_sweep_step_cached_and_records(case):
    rng = np.random.default_rng(777000 + case)
    dtype, Hkv, G, d = _geometry(rng)
    wide = case % 4 == 3
    B = int(rng.integers(1, 33)) if not wide else int(rng.integers(40, 90))
    lens = rng.integers(0, 5000 if not wide else 1500, B)
    lens[rng.random(B) < 0.2] = rng.integers(0, 60)
    back = int(rng.integers(0, 40))
    k = int(rng.integers(0, 30)) if case % 5 else int(rng.integers(30, 200))
    W = int(rng.integers(0, 400))
    th = ("uniform", 1, int(rng.integers(2, 500))) if case % 7 else ("uniform", 1, 12)
    paging = ["permuted", "interleaved"][rng.integers(0, 2)]
    say(f"[sweep] {case}: {dtype} B{B} Hkv{Hkv} G{G} d{d} k{k} W{W} back{back} {paging}")
    w = synth.make_workload(1, seed=case, device="cuda", seq_lens=lens.tolist(), overrides=dict(
        B=B, dtype=dtype, d=d, Hq=Hkv * G, Hkv=Hkv, thought=th, k=k, window=W, paging=paging))
    h = P.host(w)
    st = zr.step_from_workload(w)
    st.step()
    torch.cuda.synchronize()
    fused = st.out.clone()
    sel = st.sel.cpu().numpy()
    scores = st.scores.cpu().numpy()[:w.n_total]
    st.step_calls()
    torch.cuda.synchronize()
    assert torch.equal(fused, st.out)
    ref = P.oracle_step(w, h)
    assert np.all(np.abs(scores - ref["scores"])
                  <= np.spacing(np.abs(ref["scores"]).astype(np.float32)))
    if P.compare_selection(sel, ref["scores"], w.seq_ptr, k, w.Hkv):
        ref = P.oracle_step(w, h, sel=sel)
    assert float(np.max(np.abs(fused.cpu().numpy() - ref["out"]))) <= P.TOL[dtype]
    # a wider window at the same lengths starts where the lists were clipped
    st.cached_attn(W + 9)
    torch.cuda.synchronize()
    assert torch.equal(st.out, fused)
    # records at a boundary T0 = T - back, calls at T0 + i
    T0 = np.maximum(w.seq_lens - back, 0).astype(np.int32)
    sb = zr.DeviceStep(w.q, w.k_pool, w.v_pool, w.block_table, T0, w.seq_ptr, w.th_start,
                       w.th_len, w.summary_keys, w.max_per_seq, k, W, w.scale, st.max_attended)
    sb.step()
    torch.cuda.synchronize()
    sel0 = sb.sel.cpu().numpy()
    sb.reuse_plan(back)
    for i in sorted({0, back // 2, back}):
        sb.reuse_attn(seq_lens=_dev(np.minimum(T0 + i, w.seq_lens).astype(np.int32)))
        torch.cuda.synchronize()
        ok = (T0 + i) <= w.seq_lens  # rows whose T0 + i is cached
        if not ok.any():
            continue
        Ti = np.minimum(T0 + i, w.seq_lens)  # (the other rows are not compared)
        ref_i = O.sparse_decode_step(h["q"], h["k_pool"], h["v_pool"], w.block_table, Ti,
                                     w.seq_ptr, w.th_start, w.th_len, h["kbar"], k, W + i,
                                     w.scale, sel=sel0)
        err = float(np.max(np.abs(sb.out.cpu().numpy()[ok] - ref_i["out"][ok])))
        assert err <= P.TOL[dtype], (i, err)


@pytest.mark.parametrize("case", range(18))
def test_sweep_staging_noalloc_dense_zoom(case):
    rng = np.random.default_rng(888000 + case)
    kind = ["stage", "zoom", "noalloc_dense"][case % 3]
    dtype, Hkv, G, d = _geometry(rng, g16=False)
    say(f"[sweep] {case}: {kind} {dtype} Hkv{Hkv} G{G} d{d}")
    if kind != "zoom":
        B = int(rng.integers(1, 20))
        lens = rng.integers(0, 3000, B)
        lens[rng.random(B) < 0.2] = rng.integers(0, 40)
        k, W = int(rng.integers(0, 20)), int(rng.integers(0, 300))
        w = synth.make_workload(1, seed=case, device="cuda", seq_lens=lens.tolist(), overrides=dict(
            B=B, dtype=dtype, d=d, Hq=Hkv * G, Hkv=Hkv,
            thought=("uniform", 1, int(rng.integers(2, 400))), k=k, window=W))
        h = P.host(w)
        st = zr.step_from_workload(w)
        st.step()
        torch.cuda.synchronize()
        sel = st.sel.clone()
        out_dev = st.out.clone()
        if kind == "stage":
            kp, vp = w.k_pool.cpu().pin_memory(), w.v_pool.cpu().pin_memory()
            hs = zr.DeviceStep(w.q, kp, vp, w.block_table, w.seq_lens, w.seq_ptr, w.th_start,
                               w.th_len, w.summary_keys, w.max_per_seq, k, W, w.scale,
                               st.max_attended)
            blocks = -(-st.max_attended // 16) + 2 * k + 2
            sg = zr.Staging(hs, int(min(blocks, w.max_blocks + 1)))
            hs.stage(sg, sel=sel, window=W)
            hs.attend_staged(sg)
            torch.cuda.synchronize()
            assert int(sg.dropped.sum().item()) == 0
            assert torch.equal(hs.out, out_dev)
            hs.sparse_attn(sel=sel)  # zero-copy reads of the host pools
            torch.cuda.synchronize()
            assert torch.equal(hs.out, out_dev)
        else:
            so = zr.step_from_workload(w)
            so.step_noalloc()
            torch.cuda.synchronize()
            assert torch.equal(so.out, out_dev)
            st.dense_attn()
            torch.cuda.synchronize()
            ref_d = O.dense_decode_step(h["q"], h["k_pool"], h["v_pool"], w.block_table,
                                        w.seq_lens, w.scale)
            assert float(np.max(np.abs(st.out.cpu().numpy() - ref_d))) <= P.TOL[dtype]
        ref = P.oracle_step(w, h, sel=sel.cpu().numpy())
        assert float(np.max(np.abs(out_dev.cpu().numpy() - ref["out"]))) <= P.TOL[dtype]
        return
    B = int(rng.integers(1, 6))
    w = synth.make_workload(5, seed=case, device="cuda", overrides=dict(
        B=B, dtype=dtype, d=d, Hq=Hkv * G, Hkv=Hkv, seq_len=("uniform", 600, 3000),
        thought=("uniform", 20, int(rng.integers(40, 300))),
        summary=("uniform", 1, int(rng.integers(2, 30))), prompt=int(rng.integers(0, 300)),
        window=int(rng.integers(0, 400)), k=int(rng.integers(1, 10)), c=int(rng.integers(1, 6))))
    n_layers = int(rng.integers(1, 5))
    c, n_prompt = w.extra["c"], w.extra["prompt"]
    back = int(rng.integers(0, 30))
    T0 = np.maximum(w.seq_lens - back, 0).astype(np.int32)
    st = zr.DeviceStep(w.q, w.k_pool, w.v_pool, w.block_table, T0, w.seq_ptr, w.th_start,
                       w.th_len, w.summary_keys, w.max_per_seq, w.k, w.window, w.scale,
                       int(w.seq_lens.max()))
    sel = np.full((n_layers, w.B, w.Hkv, w.k), -1, np.int32)
    for l in range(n_layers):
        for b in range(w.B):
            n = int(w.seq_ptr[b + 1] - w.seq_ptr[b])
            for g in range(w.Hkv):
                m = min(w.k, n)
                if m:
                    sel[l, b, g, :m] = np.sort(rng.choice(n, size=m, replace=False))
    votes = torch.empty(w.n_total, dtype=torch.int32, device="cuda")
    cons = torch.empty((w.B, c), dtype=torch.int32, device="cuda")
    agree = torch.empty(w.B, dtype=torch.float32, device="cuda")
    st.consensus(_dev(sel), c, votes, cons, agree)
    torch.cuda.synchronize()
    v_ref, c_ref, _ = O.consensus(sel, w.seq_ptr, c)
    assert np.array_equal(votes.cpu().numpy(), v_ref)
    assert np.array_equal(cons.cpu().numpy(), c_ref)
    ss, sl = w.extra["sum_start"], w.extra["sum_len"]
    st.zoom_attn(_dev(ss), _dev(sl), votes, cons, c, n_prompt)
    torch.cuda.synchronize()
    h = P.host(w)

    def ref_at(i):
        return O.zoom_decode_step(h["q"], h["k_pool"], h["v_pool"], w.block_table, T0 + i,
                                  w.seq_ptr, w.th_start, w.th_len, ss, sl, v_ref, c_ref,
                                  n_prompt, w.window + i, w.scale)["out"]

    assert float(np.max(np.abs(st.out.cpu().numpy() - ref_at(0)))) <= P.TOL[dtype]
    if back:
        st.cached_attn(w.window + back, seq_lens=_dev(T0 + back))
        torch.cuda.synchronize()
        assert float(np.max(np.abs(st.out.cpu().numpy() - ref_at(back)))) <= P.TOL[dtype]
    st.reuse_plan(back, seq_lens=_dev(T0))
    for i in sorted({0, back}):
        st.reuse_attn(seq_lens=_dev(T0 + i))
        torch.cuda.synchronize()
        assert float(np.max(np.abs(st.out.cpu().numpy() - ref_at(i)))) <= P.TOL[dtype], i
