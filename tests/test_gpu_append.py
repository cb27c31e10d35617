"""GPU parity of the append path (zr_append_kv, zr_summary_keys) against the
CPU oracle. The oracle allocates blocks to sequences in index order; on the
GPU sequences pop the free stack concurrently, so the tests compare what is
unique (the logical cache every sequence reads back, lengths, statuses, the
set of blocks taken) and check that the rest is valid (each popped block used
once, old table entries untouched)."""
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


def _grow_workload(dtype="bf16", d=128, extra=40, spare=None, B=4, seq_len=("uniform", 1, 200)):
    over = dict(B=B, dtype=dtype, d=d, Hq=8, Hkv=4 if d == 128 else 2,
                seq_len=seq_len, thought=("uniform", 8, 60), extra_tokens=extra)
    nb_new = B * ((extra + 15) // 16 + 1)
    over["spare_blocks"] = nb_new if spare is None else spare
    return synth.make_workload(1, device="cuda", overrides=over)


def _append_run(w, steps, seed=0):
    st = zr.step_from_workload(w)
    free_np = w.extra["free_blocks"]
    free = torch.as_tensor(np.concatenate([free_np, [0]]).astype(np.int32), device="cuda")
    count = torch.tensor([len(free_np)], dtype=torch.int32, device="cuda")
    status = torch.empty(w.B, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(seed)
    shape = (w.B, w.Hkv, w.d)
    news = []
    statuses = []
    for _ in range(steps):
        kn = torch.randn(shape, generator=gen, device="cuda").to(w.k_pool.dtype)
        vn = torch.randn(shape, generator=gen, device="cuda").to(w.k_pool.dtype)
        st.append(kn, vn, free, count, status)
        news.append((kn, vn))
        statuses.append(status.clone())
    torch.cuda.synchronize()
    return st, news, [s.cpu().numpy() for s in statuses], int(count.item())


def _oracle_run(w, news):
    k = synth.to_numpy_f32(w.k_pool)
    v = synth.to_numpy_f32(w.v_pool)
    table, lens = w.block_table.copy(), w.seq_lens.copy()
    free = w.extra["free_blocks"]
    top = len(free)
    sts = []
    for kn, vn in news:
        k, v, table, lens, top, st = O.append_kv(k, v, table, lens, synth.to_numpy_f32(kn),
                                                 synth.to_numpy_f32(vn), free, top)
        sts.append(st)
    return k, v, table, lens, top, sts


def _check_views(w, st, k_ref, v_ref, table_ref, lens_ref, ok_rows=None):
    k = synth.to_numpy_f32(st.k_pool)
    v = synth.to_numpy_f32(st.v_pool)
    table = st.block_table.cpu().numpy()
    lens = st.seq_lens.cpu().numpy()
    for b in range(w.B):
        if ok_rows is not None and not ok_rows[b]:
            continue
        assert lens[b] == lens_ref[b], b
        T = int(lens[b])
        assert np.array_equal(O.gather_keys(k, table[b], T), O.gather_keys(k_ref, table_ref[b], T))
        assert np.array_equal(O.gather_values(v, table[b], T),
                              O.gather_values(v_ref, table_ref[b], T))
        old = (int(w.seq_lens[b]) + 15) // 16
        assert np.array_equal(table[b, :old], w.block_table[b, :old]), b
    return table, lens


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_append_parity(dtype, d):
    w = _grow_workload(dtype, d)
    say(f"[gpu] append {dtype} d{d}: B={w.B} lens={w.seq_lens.tolist()}")
    st, news, sts, top = _append_run(w, 40)
    k_ref, v_ref, table_ref, lens_ref, top_ref, sts_ref = _oracle_run(w, news)
    assert all(np.all(s == 0) for s in sts) and all(np.all(s == 0) for s in sts_ref)
    assert top == top_ref
    table, lens = _check_views(w, st, k_ref, v_ref, table_ref, lens_ref)
    # the popped blocks are exactly the stack's top entries, each used once
    free = w.extra["free_blocks"]
    taken = []
    for b in range(w.B):
        old = (int(w.seq_lens[b]) + 15) // 16
        taken += table[b, old:(int(lens[b]) + 15) // 16].tolist()
    assert sorted(taken) == sorted(free[top:].tolist())


def test_append_exhausts_the_free_stack():
    """Fewer spare blocks than the sequences need: as many appends fail as in
    the oracle, failing sequences are untouched, the others are exact."""
    w = _grow_workload(extra=16, spare=2, B=6, seq_len=("fixed", 32))
    # every sequence needs a block on its first append
    st, news, sts, top = _append_run(w, 1)
    k_ref, v_ref, table_ref, lens_ref, top_ref, sts_ref = _oracle_run(w, news)
    got = sts[0]
    say(f"[gpu] exhaustion: gpu status {got.tolist()}, oracle {sts_ref[0].tolist()}")
    assert top == top_ref == 0
    assert np.sum(got == zr.ZR_APPEND_NO_FREE_BLOCK) == np.sum(sts_ref[0] == 1) == w.B - 2
    assert set(np.unique(got)) <= {0, zr.ZR_APPEND_NO_FREE_BLOCK}
    lens = st.seq_lens.cpu().numpy()
    assert np.array_equal(lens, np.where(got == 0, 33, 32))
    # successful sequences hold the token; their blocks are the two spare ones
    table = st.block_table.cpu().numpy()
    k = synth.to_numpy_f32(st.k_pool)
    kn = synth.to_numpy_f32(news[0][0])
    assert sorted(table[got == 0, 2].tolist()) == sorted(w.extra["free_blocks"].tolist())
    for b in np.nonzero(got == 0)[0]:
        assert np.array_equal(O.gather_keys(k, table[b], 33)[32], kn[b].astype(np.float64))
    assert np.all(table[got != 0, 2] == -1)


def test_append_table_full():
    w = _grow_workload(extra=0, spare=4, B=3)
    w.seq_lens[:] = w.block_table.shape[1] * 16  # no column left
    st, news, sts, top = _append_run(w, 1)
    assert np.all(sts[0] == zr.ZR_APPEND_TABLE_FULL)
    assert top == 4
    assert np.array_equal(st.seq_lens.cpu().numpy(), w.seq_lens)


@pytest.mark.parametrize("dtype,d,seq_len,thought", [
    ("bf16", 128, ("uniform", 100, 3000), ("uniform", 1, 700)),
    ("bf16", 64, ("uniform", 100, 3000), ("uniform", 1, 700)),
    ("f32", 128, ("uniform", 100, 3000), ("uniform", 1, 700)),
    # thoughts longer than one LDS window of block ids (8176 tokens)
    ("bf16", 128, ("fixed", 40000), ("uniform", 8000, 20000))])
def test_summary_keys_parity(dtype, d, seq_len, thought):
    w = synth.make_workload(1, device="cuda", overrides=dict(
        B=3, dtype=dtype, d=d, Hq=8, Hkv=2, seq_len=seq_len, thought=thought))
    st = zr.step_from_workload(w)
    out = torch.full_like(st.summary_keys, 7.0)
    which_np = np.concatenate([np.arange(w.n_total), [-1, w.n_total, 0]]).astype(np.int32)
    which = torch.as_tensor(which_np, device="cuda")
    st.compute_summary_keys(which, out=out)
    torch.cuda.synchronize()
    ref = O.summary_keys(synth.to_numpy_f32(w.k_pool), w.block_table, w.seq_ptr, w.th_start,
                         w.th_len, range(w.n_total), dtype)
    got = synth.to_numpy_f32(out)
    say(f"[gpu] summary keys {dtype} d{d}: {w.n_total} thoughts")
    if dtype == "bf16":
        assert np.array_equal(got, ref)
    else:
        ulp = np.spacing(np.abs(ref).astype(np.float32))
        assert np.all(np.abs(got - ref) <= ulp)
    # rows not listed stay as they were
    part = torch.full_like(st.summary_keys, 7.0)
    st.compute_summary_keys(torch.as_tensor([1], dtype=torch.int32, device="cuda"), out=part)
    torch.cuda.synchronize()
    p = synth.to_numpy_f32(part)
    assert np.all(p[0] == 7.0) and np.all(p[2:] == 7.0)
    assert np.array_equal(p[1], got[1])


def test_decode_steps_with_append():
    """Append tokens for a few steps, refresh the summary key of each
    sequence's last thought, then run the sparse step: it matches the oracle
    on the oracle's own appended cache and summary keys."""
    w = _grow_workload(extra=24)
    st, news, sts, top = _append_run(w, 20)
    k_ref, v_ref, table_ref, lens_ref, _, _ = _oracle_run(w, news)
    # the last thought of every sequence grows with the appended tokens
    th_len = w.th_len.copy()
    for b in range(w.B):
        last = int(w.seq_ptr[b + 1]) - 1
        if last >= int(w.seq_ptr[b]):
            th_len[last] += 20
    st2 = zr.DeviceStep(w.q, st.k_pool, st.v_pool, st.block_table, st.seq_lens, w.seq_ptr,
                        w.th_start, th_len, w.summary_keys, w.max_per_seq, w.k, w.window,
                        w.scale, int(lens_ref.max()))
    lasts = torch.as_tensor([int(w.seq_ptr[b + 1]) - 1 for b in range(w.B)
                             if w.seq_ptr[b + 1] > w.seq_ptr[b]], dtype=torch.int32, device="cuda")
    st2.compute_summary_keys(lasts)
    st2.step()
    torch.cuda.synchronize()
    kbar = synth.to_numpy_f32(w.summary_keys)
    kbar[lasts.cpu().numpy()] = O.summary_keys(k_ref, table_ref, w.seq_ptr, w.th_start, th_len,
                                               lasts.cpu().numpy(), w.dtype)
    assert np.array_equal(synth.to_numpy_f32(st2.summary_keys), kbar)
    ref = O.sparse_decode_step(synth.to_numpy_f32(w.q), k_ref, v_ref, table_ref, lens_ref,
                               w.seq_ptr, w.th_start, th_len, kbar, w.k, w.window, w.scale)
    events = P.compare_selection(st2.sel.cpu().numpy(), ref["scores"], w.seq_ptr, w.k, w.Hkv)
    if events:
        ref = O.sparse_decode_step(synth.to_numpy_f32(w.q), k_ref, v_ref, table_ref, lens_ref,
                                   w.seq_ptr, w.th_start, th_len, kbar, w.k, w.window, w.scale,
                                   sel=st2.sel.cpu().numpy())
    err = np.max(np.abs(st2.out.cpu().numpy() - ref["out"]))
    say(f"[gpu] decode with append: max|out-oracle| = {err:.3e}")
    assert err <= P.TOL[w.dtype]
