"""Pins of the CPU oracle against things fixed outside it: printed figures of
the pages, closed forms, brute force over subsets, a library attention routine
and invariants of the method. None of these re-runs the oracle's own formula."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import zr_oracle as O


# ---------------------------------------------------------------- accounting
def test_memory_savings_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "zoomr_memory_savings.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ms = O.memory_savings(c["n_prompt"], c["n_gen"], c["n_window"], c["c"],
                              c["len_regular"], c["len_summary"], c["n_all"])
        assert round(ms, c["decimals"]) == pytest.approx(c["ms"], abs=1e-9), c


def test_dense_kv_bytes_printed_figures(golden_dir):
    with open(os.path.join(golden_dir, "kv_cache_sizes.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        n = O.dense_kv_bytes(c["n_layers"], c["n_tokens"], c["n_kv_heads"], c["head_dim"],
                             c["bytes_per_elem"], c["batch"])
        if "expect_bytes" in c:
            assert n == c["expect_bytes"]
            assert n / 1024 == 800
        if "expect_gib_rounded_1" in c:
            assert round(n / 2**30, 1) == c["expect_gib_rounded_1"]
        if "expect_more_than_bytes" in c:
            assert n > c["expect_more_than_bytes"]


# ---------------------------------------------------------------- scorer
def _one_thought_per_seq_ptr(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def test_scores_one_hot_keys_pick_query_elements():
    """With one-hot summary keys c * e_p the score is c times the sum over the
    group's query heads of element p: catches transposed or mis-indexed
    operands (thought vs head vs dimension)."""
    rng = np.random.default_rng(0)
    B, Hq, Hkv, d = 2, 6, 3, 7
    G = Hq // Hkv
    counts = [4, 3]
    ptr = _one_thought_per_seq_ptr(counts)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    n = ptr[-1]
    kbar = np.zeros((n, Hkv, d), np.float32)
    expect = np.zeros((n, Hkv))
    for b in range(B):
        for i in range(ptr[b], ptr[b + 1]):
            for g in range(Hkv):
                p = int(rng.integers(d))
                c = float(rng.integers(1, 5))
                kbar[i, g, p] = c
                expect[i, g] = c * sum(float(q[b, h, p]) for h in range(g * G, (g + 1) * G))
    got = O.coarse_scores(q, kbar, ptr, Hkv)
    np.testing.assert_allclose(got, expect.astype(np.float32), rtol=1e-6, atol=0)


def test_scores_group_mapping_contiguous():
    """Query head h belongs to KV head h // G (reading R1): a query that is
    non-zero in one head only scores against that head's KV group only."""
    B, Hq, Hkv, d = 1, 8, 2, 4
    q = np.zeros((B, Hq, d), np.float32)
    q[0, 5] = [1, 2, 3, 4]
    kbar = np.ones((3, Hkv, d), np.float32)
    s = O.coarse_scores(q, kbar, np.array([0, 3], np.int32), Hkv)
    assert np.all(s[:, 0] == 0) and np.all(s[:, 1] == 10)


def test_scores_integer_closed_form_g1():
    """G = 1 reduces to the per-head inner product of ZoomR's eq. alpha:
    (1,2,3).(4,5,6) = 32 and (1,2,3).(-1,0,1) = 2."""
    q = np.array([[[1, 2, 3]]], np.float32)
    kbar = np.array([[[4, 5, 6]], [[-1, 0, 1]]], np.float32)
    s = O.coarse_scores(q, kbar, np.array([0, 2], np.int32), 1)
    assert s[0, 0] == 32 and s[1, 0] == 2


def test_scores_accumulate_in_float64_round_once():
    """2^30 + 1 - 2^30 = 1 exactly in float64; a float32 running sum gives 0.
    Pins the reading 'accumulate in float64, round once to float32'."""
    q = np.array([[[2.0**30, 1.0, -(2.0**30)]]], np.float32)
    kbar = np.array([[[1.0, 1.0, 1.0]]], np.float32)
    s = O.coarse_scores(q, kbar, np.array([0, 1], np.int32), 1)
    assert s.dtype == np.float32 and s[0, 0] == 1.0
    # the same across heads of a group
    q2 = np.zeros((1, 3, 1), np.float32)
    q2[0, :, 0] = [2.0**30, 1.0, -(2.0**30)]
    s2 = O.coarse_scores(q2, np.ones((1, 1, 1), np.float32), np.array([0, 1], np.int32), 1)
    assert s2[0, 0] == 1.0


# ---------------------------------------------------------------- selector
def _beats(s, i, j):
    """i is preferred to j: a number beats NaN; larger beats smaller; equal
    values (including -0 == +0, NaN with NaN) go to the lower index."""
    a, b = float(s[i]), float(s[j])
    if math.isnan(a) and math.isnan(b):
        return i < j
    if math.isnan(a):
        return False
    if math.isnan(b):
        return True
    return a > b or (a == b and i < j)


@pytest.mark.parametrize("seed", range(40))
def test_topk_brute_force_over_subsets(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 8))
    pool = np.array([0.0, -0.0, 1.0, 2.0, -1.5, np.nan, 2.0, 1e-30], np.float32)
    s = rng.choice(pool, size=n).astype(np.float32) if n else np.zeros(0, np.float32)
    for k in range(0, n + 3):
        sel = O.select_topk(s[:, None], np.array([0, n], np.int32), k, 1)[0, 0]
        m = min(k, n)
        winners = [set(c) for c in itertools.combinations(range(n), m)
                   if all(_beats(s, i, j) for i in c for j in range(n) if j not in c)]
        assert len(winners) == 1
        assert list(sel[:m]) == sorted(winners[0])
        assert np.all(sel[m:] == -1)


def test_topk_per_head_and_sequence_independent():
    scores = np.array([[3, 0], [1, 5], [2, 4],   # seq 0: thoughts 0..2
                       [7, 1], [6, 2]], np.float32)  # seq 1: thoughts 0..1
    sel = O.select_topk(scores, np.array([0, 3, 5], np.int32), 2, 2)
    assert sel.tolist() == [[[0, 2], [1, 2]], [[0, 1], [0, 1]]]
    assert O.select_topk(scores, np.array([0, 3, 5], np.int32), 0, 2).shape == (2, 2, 0)


# ---------------------------------------------------------------- attended set
def test_attended_all_thoughts_tiling_gives_every_token():
    starts = np.array([0, 5, 9, 20]); lens = np.array([5, 4, 11, 3])
    assert O.attended_tokens(np.arange(4), starts, lens, 23, 4).tolist() == list(range(23))


def test_attended_window_only_and_edges():
    starts = np.array([0, 10]); lens = np.array([10, 10])
    assert O.attended_tokens(np.array([-1, -1]), starts, lens, 20, 6).tolist() == list(range(14, 20))
    assert O.attended_tokens(np.array([], np.int32), starts, lens, 20, 50).tolist() == list(range(20))
    assert O.attended_tokens(np.array([], np.int32), starts, lens, 20, 0).tolist() == []
    # a selected thought inside the window adds nothing new
    assert O.attended_tokens(np.array([1]), starts, lens, 20, 12).tolist() == list(range(8, 20))


@pytest.mark.parametrize("seed", range(10))
def test_attended_count_matches_clipped_sum(seed):
    """|A| = min(W, T) + sum of the selected spans' lengths clipped below T - W
    (the kept-token count of ZoomR Sec. 3.5 with no prompt and no summary
    spans), counted arithmetically instead of as a set."""
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 300))
    ls, s = [], 0
    while s < T:
        ln = int(min(rng.integers(1, 40), T - s)); ls.append(ln); s += ln
    starts = np.concatenate([[0], np.cumsum(ls)[:-1]]); lens = np.array(ls)
    W = int(rng.integers(0, 60))
    k = int(rng.integers(0, len(ls) + 1))
    sel = np.sort(rng.choice(len(ls), size=k, replace=False))
    toks = O.attended_tokens(sel, starts, lens, T, W)
    tw = max(0, T - W)
    count = min(W, T) + sum(max(0, min(starts[i] + lens[i], tw) - starts[i]) for i in sel)
    assert len(toks) == count
    assert np.all(np.diff(toks) > 0)


# ---------------------------------------------------------------- attention
def _sdpa64(q, k, v, scale, mask=None):
    """torch's scaled_dot_product_attention on the CPU in float64."""
    t = lambda x: torch.as_tensor(np.asarray(x, np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q)[None], t(k)[None], t(v)[None],
        attn_mask=None if mask is None else torch.as_tensor(mask)[None], scale=scale)
    return out[0].numpy()


@pytest.mark.parametrize("seed", range(5))
def test_attend_matches_library_sdpa(seed):
    rng = np.random.default_rng(seed)
    G, n, d = 4, 37, 8
    q, k, v = (rng.standard_normal(s) for s in [(G, d), (n, d), (n, d)])
    np.testing.assert_allclose(O.attend(q, k, v, 0.3), _sdpa64(q, k, v, 0.3), rtol=0, atol=1e-12)


def test_attend_closed_forms():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((5, 3))
    k = rng.standard_normal((5, 3))
    # a single token gets weight 1: out = v exactly
    q = rng.standard_normal((2, 3))
    assert np.array_equal(O.attend(q, k[:1], v[:1], 0.7), np.repeat(v[:1], 2, axis=0))
    # equal logits: out = mean of V
    np.testing.assert_allclose(O.attend(np.zeros((1, 3)), k, v, 1.0)[0], v.mean(0), atol=1e-15)
    # two tokens: logistic weights
    z1, z2 = float(q[0] @ k[0]) * 0.5, float(q[0] @ k[1]) * 0.5
    w = 1.0 / (1.0 + math.exp(z2 - z1))
    np.testing.assert_allclose(O.attend(q[:1], k[:2], v[:2], 0.5)[0], w * v[0] + (1 - w) * v[1],
                               atol=1e-14)
    # weights are a probability vector
    _, p = O.attend(q, k, v, 2.0, return_weights=True)
    assert np.all(p >= 0) and np.allclose(p.sum(1), 1.0, atol=1e-14)
    # empty set -> zero output
    assert np.array_equal(O.attend(q, k[:0], v[:0], 1.0), np.zeros((2, 3)))


# ---------------------------------------------------------------- paging
def _scatter_to_pool(K, perm_seed, extra_blocks=3, slot_axis=2):
    """Write a contiguous [T][Hkv][d] cache into a pool at random physical
    blocks, one row per slot (slot_axis 2) or dimension-major (slot_axis 3)."""
    T, Hkv, d = K.shape
    nb = (T + 15) // 16
    rng = np.random.default_rng(perm_seed)
    ids = rng.permutation(nb + extra_blocks)[:nb]
    shape = (nb + extra_blocks, Hkv, 16, d) if slot_axis == 2 else (nb + extra_blocks, Hkv, d, 16)
    pool = rng.standard_normal(shape)
    for j in range(T):
        if slot_axis == 2:
            pool[ids[j // 16], :, j % 16, :] = K[j]
        else:
            pool[ids[j // 16], :, :, j % 16] = K[j]
    return pool, ids.astype(np.int32)


def test_paged_equals_contiguous():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((53, 2, 4))
    pool, table = _scatter_to_pool(K, 11)
    assert np.array_equal(O.gather_keys(pool, table, 53), K)
    vpool, vtable = _scatter_to_pool(K, 12, slot_axis=3)
    assert np.array_equal(O.gather_values(vpool, vtable, 53), K)
    # one element placed by hand: token 37, head 1, dim 2
    assert O.gather_values(vpool, vtable, 53)[37, 1, 2] == vpool[vtable[2], 1, 2, 5]


def _tiny_case(seed, T=77, Hq=4, Hkv=2, d=8, W=9):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((T, Hkv, d)); V = rng.standard_normal((T, Hkv, d))
    ls, s = [], 0
    while s < T:
        ln = int(min(rng.integers(3, 20), T - s)); ls.append(ln); s += ln
    starts = np.concatenate([[0], np.cumsum(ls)[:-1]]).astype(np.int32)
    lens = np.array(ls, np.int32)
    kbar = rng.standard_normal((len(ls), Hkv, d))
    q = rng.standard_normal((1, Hq, d))
    return K, V, starts, lens, kbar, q, W


@pytest.mark.parametrize("seed", range(4))
def test_sparse_step_invariant_under_block_permutation(seed):
    K, V, starts, lens, kbar, q, W = _tiny_case(seed)
    T = K.shape[0]
    ptr = np.array([0, len(starts)], np.int32)
    outs = []
    for perm_seed in (1, 2, 3):
        kp, table = _scatter_to_pool(K, perm_seed)
        vp, _ = _scatter_to_pool(V, perm_seed, slot_axis=3)  # same seed -> same block ids
        r = O.sparse_decode_step(q, kp, vp, table[None], np.array([T]), ptr, starts, lens,
                                 kbar, 3, W, 0.35)
        outs.append(r["out"])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("seed", range(4))
def test_sparse_all_thoughts_equals_dense_sdpa(seed):
    """k = every thought (thoughts tile the cache) must be full attention."""
    K, V, starts, lens, kbar, q, W = _tiny_case(seed)
    T, Hkv, d = K.shape
    G = q.shape[1] // Hkv
    kp, table = _scatter_to_pool(K, 5)
    vp, _ = _scatter_to_pool(V, 5, slot_axis=3)
    ptr = np.array([0, len(starts)], np.int32)
    r = O.sparse_decode_step(q, kp, vp, table[None], np.array([T]), ptr, starts, lens, kbar,
                             len(starts), W, 0.35)
    dense = O.dense_decode_step(q, kp, vp, table[None], np.array([T]), 0.35)
    for g in range(Hkv):
        ref = _sdpa64(q[0, g * G:(g + 1) * G], K[:, g], V[:, g], 0.35)
        np.testing.assert_allclose(r["out"][0, g * G:(g + 1) * G], ref, atol=1e-12)
        np.testing.assert_allclose(dense[0, g * G:(g + 1) * G], ref, atol=1e-12)
    assert np.all(r["n_attended"] == T)


@pytest.mark.parametrize("seed", range(6))
def test_sparse_step_equals_masked_sdpa(seed):
    """The sparse step equals library attention over the whole cache with a
    boolean mask: token j is visible iff it is in the last W positions or
    lies inside a thought the selector kept (per-token membership test)."""
    K, V, starts, lens, kbar, q, W = _tiny_case(seed)
    T, Hkv, d = K.shape
    G = q.shape[1] // Hkv
    kp, table = _scatter_to_pool(K, 9)
    vp, _ = _scatter_to_pool(V, 9, slot_axis=3)
    ptr = np.array([0, len(starts)], np.int32)
    k = 2
    r = O.sparse_decode_step(q, kp, vp, table[None], np.array([T]), ptr, starts, lens, kbar,
                             k, W, 0.35)
    for g in range(Hkv):
        chosen = [i for i in r["sel"][0, g] if i >= 0]
        assert len(chosen) == k
        mask = np.array([j >= T - W or any(starts[i] <= j < starts[i] + lens[i] for i in chosen)
                         for j in range(T)])
        ref = _sdpa64(q[0, g * G:(g + 1) * G], K[:, g], V[:, g], 0.35,
                      mask=np.broadcast_to(mask, (G, T)).copy())
        np.testing.assert_allclose(r["out"][0, g * G:(g + 1) * G], ref, atol=1e-12)
        # the selection is the top-k of the group-summed score
        sc = np.array([sum(float(q[0, h] @ kbar[i, g]) for h in range(g * G, (g + 1) * G))
                       for i in range(len(starts))])
        best = sorted(range(len(sc)), key=lambda i: (-sc[i], i))[:k]
        assert sorted(best) == chosen


# --------------------------------------------------------------------------
# Append path: append_kv and summary_keys
# --------------------------------------------------------------------------
def test_round_bf16_matches_torch():
    """float32 -> bf16 nearest-even, against torch's conversion (a library
    routine), on random values, exact halfway cases and both signs."""
    import torch
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(size=4000).astype(np.float32) * 10,
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8,
                                  0.0, -0.0, 65504.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O._round_bf16(x).view(np.uint32), ref.view(np.uint32))


def _tiny_cache(n_blocks=12, Hkv=2, d=4, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.normal(size=(n_blocks, Hkv, 16, d)).astype(np.float32)
    v = rng.normal(size=(n_blocks, Hkv, d, 16)).astype(np.float32)
    return k, v


def test_append_builds_the_logical_sequence():
    """Appending tokens one by one to sequences of lengths 0, 5, 16 and 31
    gives, read back through the table, the old tokens followed by the new
    ones in order; blocks are taken from the top of the stack only when a
    length is a multiple of 16."""
    k, v = _tiny_cache(n_blocks=16)
    lens0 = np.array([0, 5, 16, 31], np.int32)
    table = np.full((4, 5), -1, np.int32)
    table[1, 0] = 0
    table[2, 0] = 1
    table[3, :2] = [2, 3]
    free = np.arange(15, 3, -1, dtype=np.int32)  # top = last entry (4)
    top = len(free)
    old = [O.gather_keys(k, table[b], int(lens0[b])) for b in range(4)]
    rng = np.random.default_rng(9)
    new_k = rng.normal(size=(20, 4, 2, 4)).astype(np.float32)
    new_v = rng.normal(size=(20, 4, 2, 4)).astype(np.float32)
    lens = lens0
    pops = 0
    for step in range(20):
        need = int(np.sum(lens % 16 == 0))
        k, v, table, lens, top2, st = O.append_kv(k, v, table, lens, new_k[step], new_v[step],
                                                  free, top)
        assert np.all(st == 0)
        assert top2 == top - need
        pops += need
        top = top2
    assert np.array_equal(lens, lens0 + 20)
    for b in range(4):
        got_k = O.gather_keys(k, table[b], int(lens[b]))
        got_v = O.gather_values(v, table[b], int(lens[b]))
        assert np.array_equal(got_k[:lens0[b]], old[b])
        assert np.array_equal(got_k[lens0[b]:], new_k[:, b].astype(np.float64))
        assert np.array_equal(got_v[lens0[b]:], new_v[:, b].astype(np.float64))
    # blocks 0..3 were in use; the pops took the stack's top entries in order
    used = set(table[table >= 0].tolist())
    assert used == set(range(4)) | set(free[len(free) - pops:].tolist())
    # ceil((T + 20) / 16) - ceil(T / 16) new blocks per sequence: 2 + 1 + 2 + 2
    assert pops == 7


def test_append_failures_change_nothing():
    k, v = _tiny_cache(n_blocks=4)
    table = np.array([[0, -1], [1, 2]], np.int32)
    lens = np.array([16, 32], np.int32)          # both need a block; sequence 1's table is full
    kn = np.ones((2, 2, 4), np.float32)
    free = np.array([3], np.int32)
    k2, v2, t2, l2, top, st = O.append_kv(k, v, table, lens, kn, kn, free, 0)  # empty stack
    assert list(st) == [O.APPEND_NO_FREE_BLOCK, O.APPEND_TABLE_FULL]
    assert np.array_equal(k2, k) and np.array_equal(t2, table) and np.array_equal(l2, lens)
    k2, v2, t2, l2, top, st = O.append_kv(k, v, table, lens, kn, kn, free, 1)
    assert list(st) == [0, O.APPEND_TABLE_FULL] and top == 0 and t2[0, 1] == 3
    assert list(l2) == [17, 32]


def test_summary_keys_closed_forms():
    """Constant keys average to the constant; keys equal to the token index
    average to start + (len - 1) / 2; a one-token thought returns its key;
    the result does not depend on where the blocks sit in the pool."""
    n_blocks, Hkv, d = 8, 2, 4
    table = np.array([[5, 2, 7, 0], [1, 3, 4, 6]], np.int32)
    seq_ptr = np.array([0, 3, 5], np.int32)
    starts = np.array([0, 10, 40, 0, 63], np.int32)
    lens = np.array([10, 30, 1, 63, 1], np.int32)
    k = np.zeros((n_blocks, Hkv, 16, d), np.float32)
    for b in range(2):
        for j in range(64):
            k[table[b, j // 16], :, j % 16, :] = j
    got = O.summary_keys(k, table, seq_ptr, starts, lens, range(5), "f32")
    want = starts + (lens - 1) / 2.0
    assert np.array_equal(got, np.broadcast_to(want[:, None, None], got.shape).astype(np.float32))
    k.fill(0.375)
    assert np.all(O.summary_keys(k, table, seq_ptr, starts, lens, [1, 3], "bf16") == 0.375)
    rng = np.random.default_rng(1)
    k = rng.normal(size=k.shape).astype(np.float32)
    one = O.summary_keys(k, table, seq_ptr, starts, lens, [2], "f32")
    assert np.array_equal(one[0], k[table[0, 40 // 16], :, 40 % 16, :])
    perm = rng.permutation(n_blocks)
    k2 = np.empty_like(k)
    k2[perm] = k
    a = O.summary_keys(k, table, seq_ptr, starts, lens, range(5), "bf16")
    b = O.summary_keys(k2, perm[table], seq_ptr, starts, lens, range(5), "bf16")
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# Consensus and the multi-granularity set
# --------------------------------------------------------------------------
def test_consensus_hand_example():
    """2 layers x 2 KV heads, k = 2 over 5 thoughts: votes are counted per
    set (a repeated index counts once), the consensus set takes the most
    voted thoughts with ties to the lower index, AG is the consensus share of
    all votes."""
    sel = np.array([[[[0, 1], [1, 2]]], [[[1, 3], [3, 4]]]], np.int32)   # [L][B][Hkv][k]
    ptr = np.array([0, 5], np.int32)
    votes, cons, ag = O.consensus(sel, ptr, 2)
    assert votes.tolist() == [1, 3, 1, 2, 1]
    assert cons.tolist() == [[1, 3]] and ag[0] == 5 / 8
    votes, cons, ag = O.consensus(sel, ptr, 3)
    assert cons.tolist() == [[0, 1, 3]] and ag[0] == 6 / 8
    dup = sel.copy()
    dup[0, 0, 0] = [1, 1]
    votes, _, _ = O.consensus(dup, ptr, 2)
    assert votes.tolist() == [0, 3, 1, 2, 1]
    # every voted thought in the consensus set: AG = 1; no votes: AG = 0
    assert O.consensus(sel, ptr, 8)[2][0] == 1.0
    v, c, a = O.consensus(np.full_like(sel, -1), ptr, 2)
    assert v.sum() == 0 and c.tolist() == [[-1, -1]] and a[0] == 0.0


def test_consensus_votes_are_row_memberships():
    """Random rows: votes sum to the number of distinct valid entries per
    row, and each thought's votes equal the number of rows holding it."""
    rng = np.random.default_rng(4)
    L_, B, Hkv, k = 3, 2, 4, 5
    ptr = np.array([0, 9, 12], np.int32)
    sel = np.full((L_, B, Hkv, k), -1, np.int32)
    for l in range(L_):
        for b in range(B):
            n = ptr[b + 1] - ptr[b]
            for g in range(Hkv):
                m = min(k, n)
                sel[l, b, g, :m] = np.sort(rng.choice(n, size=m, replace=False))
    votes, cons, ag = O.consensus(sel, ptr, 2)
    for b in range(B):
        rows = sel[:, b].reshape(-1, k)
        assert votes[ptr[b]:ptr[b + 1]].sum() == (rows >= 0).sum()
        for i in range(ptr[b + 1] - ptr[b]):
            assert votes[ptr[b] + i] == sum(int(i in r) for r in rows.tolist())


def test_zoom_set_size_matches_memory_formula():
    """A layout of prompt + 100 thoughts (regular 250 tokens, summary 20) and
    an 80-thought candidate set with c = 2 consensus thoughts, away from the
    512-token window: |I_f| equals the denominator of ZoomR Sec. 3.5's memory
    savings, and N/|I_f| equals the savings helper pinned to the printed 5.48x."""
    n_p, n_w, L_R, L_S, n_th = 512, 512, 250, 20, 100
    starts = n_p + (L_R + L_S) * np.arange(n_th)
    lens = np.full(n_th, L_R)
    sstarts = starts + L_R
    slens = np.full(n_th, L_S)
    T = n_p + n_th * (L_R + L_S)
    votes = np.zeros(n_th, np.int32)
    votes[:80] = 1
    votes[[7, 40]] = 5
    cons = np.array([7, 40], np.int32)
    toks = O.zoom_attended_tokens(votes, cons, starts, lens, sstarts, slens, n_p, T, n_w)
    assert len(toks) == n_p + 2 * L_R + (80 - 2) * L_S + n_w
    ms = O.memory_savings(n_p, T - n_p, n_w, 2, L_R, L_S, 80)
    assert abs(ms - T / len(toks)) < 1e-12


def test_zoom_equals_per_head_path_when_heads_agree():
    """With summary segments equal to the regular ones, no prompt, and every
    KV head selecting the same thoughts, the multi-granularity set is the
    window plus those thoughts' spans whatever c is, so the zoom attention
    equals the per-head sparse step on that selection."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, d, nb = 2, 4, 2, 8, 12
    k_pool = rng.normal(size=(nb, Hkv, 16, d))
    v_pool = rng.normal(size=(nb, Hkv, d, 16))
    table = np.array([[3, 0, 7, 9, 1, 11], [2, 4, 5, 6, 8, 10]], np.int32)
    lens_seq = np.array([90, 77], np.int32)
    seq_ptr = np.array([0, 4, 7], np.int32)
    starts = np.array([0, 20, 45, 60, 0, 30, 50], np.int32)
    lens = np.array([20, 25, 15, 30, 30, 20, 27], np.int32)
    q = rng.normal(size=(B, Hq, d))
    kbar = rng.normal(size=(7, Hkv, d))
    sel = np.array([[[0, 2], [0, 2]], [[1, -1], [1, -1]]], np.int32)
    ref = O.sparse_decode_step(q, k_pool, v_pool, table, lens_seq, seq_ptr, starts, lens, kbar,
                               2, 16, 0.3, sel=sel)
    votes, cons, _ = O.consensus(sel[None], seq_ptr, 1)
    got = O.zoom_decode_step(q, k_pool, v_pool, table, lens_seq, seq_ptr, starts, lens, starts,
                             lens, votes, cons, 0, 16, 0.3)
    assert np.allclose(got["out"], ref["out"], rtol=0, atol=1e-12)
