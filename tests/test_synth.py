"""Properties of the seeded workload generators (CPU)."""
import numpy as np
import pytest
import torch

from hierarchical_sparse_kv_amd import synth
from oracle import zr_oracle as O

SMALL = {  # shrunken versions of the workloads: same recipe, CPU-sized
    0: {},
    1: dict(B=2, seq_len=("fixed", 2048)),
    3: dict(B=4, seq_len=("uniform", 256, 1500), thought=("uniform", 32, 300)),
    4: dict(B=1, seq_len=("fixed", 4096), thought=("loguniform", 32, 512)),
}


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_structure_tiles_and_pages(cfg):
    w = synth.make_workload(cfg, overrides=SMALL[cfg])
    spec = {**synth.CONFIGS[cfg], **SMALL[cfg]}["thought"]
    for b in range(w.B):
        lo, hi = w.seq_ptr[b], w.seq_ptr[b + 1]
        st, ln = w.th_start[lo:hi], w.th_len[lo:hi]
        assert st[0] == 0 and np.all(st[1:] == st[:-1] + ln[:-1])
        assert st[-1] + ln[-1] == w.seq_lens[b]
        assert np.all(ln >= 1)
        lo_b, hi_b = (spec[1], spec[1]) if spec[0] == "fixed" else (spec[1], spec[2])
        assert np.all(ln[:-1] >= lo_b) and np.all(ln <= hi_b)
    used = []
    for b in range(w.B):
        nb = (int(w.seq_lens[b]) + 15) // 16
        assert np.all(w.block_table[b, :nb] >= 0) and np.all(w.block_table[b, nb:] == -1)
        used.extend(w.block_table[b, :nb].tolist())
    assert sorted(used) == list(range(w.num_blocks))
    assert tuple(w.k_pool.shape) == (w.num_blocks, w.Hkv, 16, w.d)
    assert tuple(w.v_pool.shape) == (w.num_blocks, w.Hkv, w.d, 16)
    assert w.k_pool.dtype == synth.TORCH_DTYPE[w.dtype]


def test_interleaved_paging_is_lockstep():
    w = synth.make_workload(3, overrides=SMALL[3])
    # block j of every live sequence is allocated before block j+1 of any
    first_of_round = [min(w.block_table[b, j] for b in range(w.B) if w.block_table[b, j] >= 0)
                      for j in range(w.max_blocks) if np.any(w.block_table[:, j] >= 0)]
    assert first_of_round == sorted(first_of_round)
    live = [int(np.sum(w.block_table[:, j] >= 0)) for j in range(w.max_blocks)]
    for j in range(w.max_blocks - 1):
        if live[j + 1]:
            assert first_of_round[j + 1] - first_of_round[j] == live[j]


def test_seeded_and_deterministic():
    a = synth.make_workload(0)
    b = synth.make_workload(0)
    c = synth.make_workload(0, seed=5)
    assert torch.equal(a.k_pool, b.k_pool) and torch.equal(a.q, b.q)
    assert np.array_equal(a.block_table, b.block_table)
    assert not torch.equal(a.k_pool, c.k_pool)


def test_summary_keys_are_noisy_thought_means():
    w = synth.make_workload(0)
    K = O.gather_logical(synth.to_numpy_f32(w.k_pool), w.block_table[0], int(w.seq_lens[0]))
    kb = synth.to_numpy_f32(w.summary_keys)
    resid = []
    for i in range(w.n_total):
        s, ln = w.th_start[i], w.th_len[i]
        resid.append(kb[i] - K[s:s + ln].mean(0))
    r = np.array(resid)
    assert abs(r.std() - 0.1) < 0.01 and abs(r.mean()) < 0.01


@pytest.mark.parametrize("cfg", [0, 1, 3, 4])
def test_planted_thoughts_are_selected(cfg):
    """The query is built from the planted thoughts' summary keys, so the
    oracle's top-k must contain them."""
    w = synth.make_workload(cfg, overrides=SMALL[cfg])
    s = O.coarse_scores(synth.to_numpy_f32(w.q), synth.to_numpy_f32(w.summary_keys),
                        w.seq_ptr, w.Hkv)
    sel = O.select_topk(s, w.seq_ptr, w.k, w.Hkv)
    for b in range(w.B):
        for g in range(w.Hkv):
            for i in w.planted[b, g]:
                if i >= 0:
                    assert i in sel[b, g], (cfg, b, g, i, sel[b, g])


def test_dense_config_uses_every_thought():
    w = synth.make_workload(2, overrides=SMALL[1])
    assert w.k == w.max_per_seq
