"""GPU parity of ZoomR's multi-granularity path (zr_consensus,
zr_zoom_decode_attn) against the CPU oracle, on the prompt + regular +
summary segment layout of ZoomR Sec. 3.5's worked example."""
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


def _zoom_workload(**over):
    base = dict(B=3, seq_len=("uniform", 2500, 4000))
    base.update(over)
    return synth.make_workload(5, device="cuda", overrides=base)


def _random_sels(w, n_layers, k, seed):
    """Distinct ascending local indices per (layer, sequence, KV head) row."""
    rng = np.random.default_rng(seed)
    sel = np.full((n_layers, w.B, w.Hkv, k), -1, np.int32)
    for l in range(n_layers):
        for b in range(w.B):
            n = int(w.seq_ptr[b + 1] - w.seq_ptr[b])
            # skew the choice so that some thoughts collect many votes
            p = rng.dirichlet(np.full(max(n, 1), 0.3))[:n] if n else None
            for g in range(w.Hkv):
                m = min(k, n)
                if m:
                    sel[l, b, g, :m] = np.sort(rng.choice(n, size=m, replace=False, p=p))
    return sel


def _dev(x):
    return torch.as_tensor(np.ascontiguousarray(x), device="cuda")


@pytest.mark.parametrize("thought,summary,c", [(("uniform", 100, 400), ("uniform", 10, 30), 2),
                                               (("uniform", 100, 400), ("uniform", 10, 30), 40),
                                               (("uniform", 3, 8), ("uniform", 1, 3), 7)])
def test_consensus_parity(thought, summary, c):
    w = _zoom_workload(thought=thought, summary=summary)
    st = zr.step_from_workload(w)
    sel = _random_sels(w, 4, w.k, seed=c)
    votes = torch.empty(max(w.n_total, 1), dtype=torch.int32, device="cuda")
    cons = torch.empty((w.B, c), dtype=torch.int32, device="cuda")
    agree = torch.empty(w.B, dtype=torch.float32, device="cuda")
    st.consensus(_dev(sel), c, votes, cons, agree)
    torch.cuda.synchronize()
    v_ref, c_ref, a_ref = O.consensus(sel, w.seq_ptr, c)
    say(f"[gpu] consensus c={c}: thoughts per seq {np.diff(w.seq_ptr).tolist()}")
    assert np.array_equal(votes.cpu().numpy()[:w.n_total], v_ref)
    assert np.array_equal(cons.cpu().numpy(), c_ref)
    assert np.max(np.abs(agree.cpu().numpy() - a_ref)) <= 1e-6


@pytest.mark.parametrize("k", [12, 70])
def test_consensus_repeated_and_out_of_range_indices(k):
    """Rows with repeated indices in any order, -1 holes and indices at or past
    the sequence's thought count: a row gives each thought one vote however
    often it lists it (ZoomR Sec. 3.3: v_i is a sum of set-membership
    indicators), as the oracle counts; k = 70 crosses several batches of row
    entries in the kernel."""
    w = _zoom_workload()
    st = zr.step_from_workload(w)
    rng = np.random.default_rng(77 + k)
    n_layers, c = 3, 3
    sel = np.full((n_layers, w.B, w.Hkv, k), -1, np.int32)
    for l in range(n_layers):
        for b in range(w.B):
            n = int(w.seq_ptr[b + 1] - w.seq_ptr[b])
            for g in range(w.Hkv):
                row = rng.integers(0, max(1, min(n, 9)), k)   # few distinct values: many repeats
                kind = rng.random(k)
                row[kind < 0.15] = -1
                row[(kind >= 0.15) & (kind < 0.25)] = n + rng.integers(0, 5)
                if (l + b + g) % 4 == 0:
                    row = np.sort(row)                         # ascending with repeats
                sel[l, b, g] = row
    votes = torch.empty(max(w.n_total, 1), dtype=torch.int32, device="cuda")
    cons = torch.empty((w.B, c), dtype=torch.int32, device="cuda")
    agree = torch.empty(w.B, dtype=torch.float32, device="cuda")
    st.consensus(_dev(sel), c, votes, cons, agree)
    torch.cuda.synchronize()
    v_ref, c_ref, a_ref = O.consensus(sel, w.seq_ptr, c)
    got = votes.cpu().numpy()[:w.n_total]
    say(f"[gpu] consensus with repeats, k={k}: max votes {int(v_ref.max())} "
        f"(rows {n_layers * w.Hkv}), entries listed {int((sel >= 0).sum())}")
    assert int(v_ref.max()) <= n_layers * w.Hkv
    assert np.array_equal(got, v_ref)
    assert np.array_equal(cons.cpu().numpy(), c_ref)
    assert np.max(np.abs(agree.cpu().numpy() - a_ref)) <= 1e-6


def test_zoom_attention_parity_and_cached_steps():
    w = _zoom_workload()
    T0 = (w.seq_lens - 5).astype(np.int32)
    n_prompt, c = w.extra["prompt"], w.extra["c"]
    st = zr.DeviceStep(w.q, w.k_pool, w.v_pool, w.block_table, T0, w.seq_ptr, w.th_start,
                       w.th_len, w.summary_keys, w.max_per_seq, w.k, w.window, w.scale,
                       int(w.seq_lens.max()))
    sel = _random_sels(w, 2, w.k, seed=5)
    v_ref, c_ref, _ = O.consensus(sel, w.seq_ptr, c)
    ss, sl = w.extra["sum_start"], w.extra["sum_len"]
    st.zoom_attn(_dev(ss), _dev(sl), _dev(v_ref), _dev(c_ref), c, n_prompt)
    torch.cuda.synchronize()
    h = P.host(w)
    ref = O.zoom_decode_step(h["q"], h["k_pool"], h["v_pool"], w.block_table, T0, w.seq_ptr,
                             w.th_start, w.th_len, ss, sl, v_ref, c_ref, n_prompt, w.window,
                             w.scale)
    err = np.max(np.abs(st.out.cpu().numpy() - ref["out"]))
    say(f"[gpu] zoom attention: |I_f| {ref['n_attended'].tolist()} max err {err:.3e}")
    assert err <= P.TOL[w.dtype]
    for i in range(1, 5):
        st.cached_attn(w.window + i, seq_lens=_dev(T0 + i))
        torch.cuda.synchronize()
        ref = O.zoom_decode_step(h["q"], h["k_pool"], h["v_pool"], w.block_table, T0 + i,
                                 w.seq_ptr, w.th_start, w.th_len, ss, sl, v_ref, c_ref, n_prompt,
                                 w.window + i, w.scale)
        err = np.max(np.abs(st.out.cpu().numpy() - ref["out"]))
        assert err <= P.TOL[w.dtype], i
    # the same steps on records made once at the boundary (zr_reuse_plan)
    st.reuse_plan(4, seq_lens=_dev(T0))
    for i in (0, 2, 4):
        st.reuse_attn(seq_lens=_dev(T0 + i))
        torch.cuda.synchronize()
        ref = O.zoom_decode_step(h["q"], h["k_pool"], h["v_pool"], w.block_table, T0 + i,
                                 w.seq_ptr, w.th_start, w.th_len, ss, sl, v_ref, c_ref, n_prompt,
                                 w.window + i, w.scale)
        err = np.max(np.abs(st.out.cpu().numpy() - ref["out"]))
        say(f"[gpu] zoom set on records, step {i}: max err {err:.3e}")
        assert err <= P.TOL[w.dtype], i


def test_zoom_pipeline_two_layers():
    """Two layers (same segment layout, their own K, V, summary keys and
    queries): scores and top-k per layer, consensus over both layers' sets,
    then each layer's attention over the shared multi-granularity set."""
    layers = [synth.make_workload(5, device="cuda", value_seed=50 + l,
                                  overrides=dict(B=2, seq_len=("uniform", 3000, 5000)))
              for l in range(2)]
    w0 = layers[0]
    steps = [zr.step_from_workload(w) for w in layers]
    for st in steps:
        st.coarse_score()
        st.select_topk()
    torch.cuda.synchronize()
    sel_stack = torch.stack([st.sel for st in steps])
    c, n_prompt = w0.extra["c"], w0.extra["prompt"]
    votes = torch.empty(w0.n_total, dtype=torch.int32, device="cuda")
    cons = torch.empty((w0.B, c), dtype=torch.int32, device="cuda")
    agree = torch.empty(w0.B, dtype=torch.float32, device="cuda")
    steps[0].consensus(sel_stack, c, votes, cons, agree)
    ss, sl = _dev(w0.extra["sum_start"]), _dev(w0.extra["sum_len"])
    outs = []
    for st in steps:
        st.zoom_attn(ss, sl, votes, cons, c, n_prompt)
        torch.cuda.synchronize()
        outs.append(st.out.cpu().numpy())
    # oracle pipeline (on the GPU's selections where a near-tie made them differ)
    sels = []
    hosts = [P.host(w) for w in layers]
    for w, h, st in zip(layers, hosts, steps):
        ref = P.oracle_step(w, h, pairs=[])
        events = P.compare_selection(st.sel.cpu().numpy(), ref["scores"], w.seq_ptr, w.k, w.Hkv)
        sels.append(st.sel.cpu().numpy() if events else ref["sel"])
    v_ref, c_ref, a_ref = O.consensus(np.stack(sels), w0.seq_ptr, c)
    assert np.array_equal(votes.cpu().numpy(), v_ref)
    assert np.array_equal(cons.cpu().numpy(), c_ref)
    assert np.max(np.abs(agree.cpu().numpy() - a_ref)) <= 1e-6
    # the set is the same for every layer: layer 1 attending on layer 0's
    # block lists gives layer 1's own result, bit for bit
    steps[1].cached_attn(w0.window, workspace=steps[0].workspace)
    torch.cuda.synchronize()
    assert np.array_equal(steps[1].out.cpu().numpy(), outs[1])
    for w, h, got in zip(layers, hosts, outs):
        ref = O.zoom_decode_step(h["q"], h["k_pool"], h["v_pool"], w.block_table, w.seq_lens,
                                 w.seq_ptr, w.th_start, w.th_len, w.extra["sum_start"],
                                 w.extra["sum_len"], v_ref, c_ref, n_prompt, w.window, w.scale)
        err = np.max(np.abs(got - ref["out"]))
        say(f"[gpu] zoom pipeline layer: AG {agree.cpu().numpy().round(3).tolist()} err {err:.3e}")
        assert err <= P.TOL[w.dtype]
