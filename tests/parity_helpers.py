"""Shared helpers of the GPU parity tests: oracle runs on host copies of a
workload, the selection comparison with the near-tie rule, and the planting
of near-tied distractor summary keys (built with the oracle's scores only)."""
from __future__ import annotations

import math

import numpy as np
import torch

from hierarchical_sparse_kv_amd import synth, zr
from oracle import zr_oracle as O

TOL = {"f32": 1e-5, "bf16": 2e-3}
NEAR_TIE_REL = 1e-5


def host(w):
    """float32 host copies (bf16 -> f32 exact) of a workload's tensors."""
    return dict(q=synth.to_numpy_f32(w.q), k_pool=synth.to_numpy_f32(w.k_pool),
                v_pool=synth.to_numpy_f32(w.v_pool), kbar=synth.to_numpy_f32(w.summary_keys))


def oracle_step(w, h, sel=None, k=None, pairs=None):
    k = w.k if k is None else k
    return O.sparse_decode_step(h["q"], h["k_pool"], h["v_pool"], w.block_table, w.seq_lens,
                                w.seq_ptr, w.th_start, w.th_len, h["kbar"], k, w.window,
                                w.scale, sel=sel, pairs=pairs)


def rank_order(s):
    """Thought indices in the selection order of the oracle (shared rule:
    larger first, NaN last, ties to the lower index)."""
    return sorted(range(len(s)), key=lambda i: O._rank_key(s[i], i))


def compare_selection(sel_gpu, ref_scores, seq_ptr, k, Hkv):
    """Selected sets must be identical, except where the oracle's k-th and
    (k+1)-th scores differ by less than 1e-5 relative; there the sets may
    differ only by thoughts whose oracle score is within 1e-5 |s_k| of s_k.
    Returns the list of near-tie events (logged by the caller)."""
    events = []
    B = len(seq_ptr) - 1
    for b in range(B):
        lo, hi = int(seq_ptr[b]), int(seq_ptr[b + 1])
        for g in range(Hkv):
            s = ref_scores[lo:hi, g]
            order = rank_order(s)
            ref = sorted(order[:min(k, hi - lo)])
            got_row = sel_gpu[b, g]
            got = [int(x) for x in got_row if x >= 0]
            assert all(x == -1 for x in got_row[len(got):]), (b, g, got_row)
            if got == ref:
                continue
            assert len(order) > k, (b, g, got, ref)
            sk, sk1 = float(s[order[k - 1]]), float(s[order[k]])
            rel = abs(sk - sk1) / max(abs(sk), abs(sk1), 1e-30)
            assert rel < NEAR_TIE_REL, f"selection differs at ({b},{g}) with gap {rel:.3e}: {got} vs {ref}"
            for i in set(got) ^ set(ref):
                assert abs(float(s[i]) - sk) <= NEAR_TIE_REL * abs(sk), (b, g, i, s[i], sk)
            events.append(dict(b=b, g=g, s_k=sk, s_k1=sk1, rel_gap=rel, gpu=got, oracle=ref))
    return events


def _bf16_step(x: float, up: bool) -> float:
    bits = int(np.array([x], np.float32).view(np.uint32)[0]) >> 16
    neg = bits & 0x8000
    if x == 0.0:
        nb = 0x0001 if up else 0x8001
    elif (not neg) == up:
        nb = bits + 1
    else:
        nb = bits - 1
    return float(np.array([nb << 16], np.uint32).view(np.float32)[0])


def plant_near_ties(w, per_pair=(1, 2, 2), seed=0):
    """For every (b, g): copy the summary key of the oracle's k-th thought
    into one distractor (an exact tie), and into further distractors with one
    element moved by one bf16 step, chosen so the oracle's score gap to the
    k-th score is below 1e-5 relative ("tiny", exempt) or in [1e-5, 1e-4)
    ("small", must match exactly). Modifies w.summary_keys in place and
    returns counts of the realised ties."""
    rng = np.random.default_rng(seed)
    h = host(w)
    kbar = h["kbar"].copy()
    q = h["q"]
    scores = O.coarse_scores(q, kbar, w.seq_ptr, w.Hkv)
    counts = {"exact": 0, "tiny": 0, "small": 0}
    n_exact, n_tiny, n_small = per_pair
    for b in range(w.B):
        lo, hi = int(w.seq_ptr[b]), int(w.seq_ptr[b + 1])
        for g in range(w.Hkv):
            s = scores[lo:hi, g]
            order = rank_order(s)
            if len(order) <= w.k + n_exact + n_tiny + n_small:
                continue
            kth = order[w.k - 1]
            sk = float(s[kth])
            planted = set(int(x) for x in w.planted[b, g] if x >= 0)
            pool = [i for i in order[w.k:] if i not in planted]
            rng.shuffle(pool)
            it = iter(pool)
            base = kbar[lo + kth, g].copy()
            for _ in range(n_exact):
                d = next(it)
                kbar[lo + d, g] = base
                counts["exact"] += 1

            def candidates():
                # every single-element bf16 step of the k-th key, with the
                # oracle's relative score gap to s_k
                for e in rng.permutation(w.d):
                    for up in (True, False):
                        row = base.copy()
                        row[e] = _bf16_step(float(base[e]), up)
                        keys = np.zeros((1, w.Hkv, w.d), np.float32)
                        keys[0, g] = row
                        sc = O.coarse_scores(q[b:b + 1], keys, np.array([0, 1], np.int32),
                                             w.Hkv)[0, g]
                        rel = abs(float(sc) - sk) / max(abs(sk), 1e-30)
                        yield row, rel

            want = [("tiny", lambda r: 0 < r < 1e-5)] * n_tiny + \
                   [("small", lambda r: 1e-5 <= r < 1e-4)] * n_small
            cands = list(candidates())
            used = set()
            for name, ok in want:
                for ci, (row, rel) in enumerate(cands):
                    if ci not in used and ok(rel):
                        d = next(it)
                        kbar[lo + d, g] = row
                        used.add(ci)
                        counts[name] += 1
                        break
    w.summary_keys.copy_(torch.as_tensor(kbar).to(w.summary_keys.dtype))
    return counts


def prefetch_hits(st, w):
    """Number of sequences whose thought range lies inside the summary-key
    rows the scorer loads ahead of it, under the rule the library reports
    (zr_summary_prefetch_rule); 0 when the rule is off."""
    status, rows, per, margin = zr.zr_summary_prefetch_rule(st.geom, w.n_total, w.max_per_seq)
    assert status == zr.ZR_OK
    if rows == 0:
        return 0
    sp = np.asarray(w.seq_ptr)
    hits = 0
    for b in range(w.B):
        g0 = max(0, int(np.float32(b) * np.float32(per)) - margin)
        n = min(int(sp[b + 1] - sp[b]), w.max_per_seq)
        hits += int(sp[b] >= g0 and sp[b] + n <= g0 + rows)
    return hits
