"""The benchmark's byte accounting (bench.attended_counts) against the
oracle's attended set (CPU). The count of gathered tokens per (sequence, KV
head) is what the roofline figure multiplies by 2 d s bytes, so it must equal
|A(b, g)| as the oracle builds it: the window united with the selected
thoughts' spans, each token once (ZoomR Sec. 3.3, eq. I_f restricted to the
window and the regular segments)."""
import numpy as np
import pytest

import bench
from hierarchical_sparse_kv_amd import synth
from oracle import zr_oracle as O


def _random_sel(rng, seq_ptr, Hkv, k):
    """Selections in [-1, N_b): ascending distinct rows, plus messy rows with
    repeats, holes and any order."""
    B = len(seq_ptr) - 1
    sel = np.full((B, Hkv, k), -1, np.int32)
    for b in range(B):
        n = int(seq_ptr[b + 1] - seq_ptr[b])
        for g in range(Hkv):
            if n == 0:
                continue
            m = min(k, n)
            if (b + g) % 3 == 0:
                sel[b, g] = rng.integers(-1, n, k)
            else:
                sel[b, g, :m] = np.sort(rng.choice(n, size=m, replace=False))
    return sel


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5])
def test_counts_equal_the_oracle_attended_set(cfg):
    """Full-size integer structure of every workload (no tensors), random
    selections: the count equals the size of the oracle's attended set."""
    spec = synth.CONFIGS[cfg]
    st = synth.make_structure(spec, spec.get("seed", cfg))
    rng = np.random.default_rng(cfg)
    ptr = st["seq_ptr"]
    k = spec["k"] if spec["k"] is not None else int(np.max(np.diff(ptr)))
    sel = _random_sel(rng, ptr, spec["Hkv"], k)
    got = bench.attended_counts(sel, st["seq_lens"], ptr, st["th_start"], st["th_len"],
                                spec["window"])
    B = len(ptr) - 1
    pairs = [(b, g) for b in range(B) for g in range(spec["Hkv"])]
    if len(pairs) > 64:  # the ragged batch: every pair of a quarter of the sequences
        pairs = [(b, g) for b, g in pairs if b % 4 == 0]
    for b, g in pairs:
        lo, hi = int(ptr[b]), int(ptr[b + 1])
        toks = O.attended_tokens(sel[b, g], st["th_start"][lo:hi], st["th_len"][lo:hi],
                                 int(st["seq_lens"][b]), spec["window"])
        assert got[b, g] == len(toks), (cfg, b, g)


def test_counts_equal_the_oracle_step_on_cpu_workloads():
    """The oracle's own decode step (scores, top-k, attended set) on CPU
    workloads: its n_attended equals the count from its selection."""
    for cfg, over in ((0, {}), (1, dict(B=2, seq_len=("fixed", 3000))),
                      (4, dict(B=1, seq_len=("fixed", 6000)))):
        w = synth.make_workload(cfg, overrides=over)
        f = synth.to_numpy_f32
        ref = O.sparse_decode_step(f(w.q), f(w.k_pool), f(w.v_pool), w.block_table, w.seq_lens,
                                   w.seq_ptr, w.th_start, w.th_len, f(w.summary_keys), w.k,
                                   w.window, w.scale)
        got = bench.attended_counts(ref["sel"], w.seq_lens, w.seq_ptr, w.th_start, w.th_len,
                                    w.window)
        assert np.array_equal(got, ref["n_attended"]), cfg
