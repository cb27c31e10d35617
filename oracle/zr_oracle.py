"""CPU oracle for one hierarchical-sparse-KV decode step (TEST INFRASTRUCTURE).

This module is the parity reference, not part of the product. Only the test
suite, the package's ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it. It shares no code with the HIP library and
imports nothing from the product package; callers hand it plain numpy arrays.

What it computes, step by step, in float64 (inputs are fp32 or bf16 values,
which convert to float64 exactly):

1. ``gather_keys`` / ``gather_values`` - the paged cache read: logical token
   j of a sequence lives in physical block ``block_table[j // 16]`` at slot
   ``j % 16`` (KV-cache management page, "Paged KV cache (PagedAttention)":
   block table per sequence, attention as a sum over blocks fetched through
   the table). Key blocks hold one row per slot; value blocks are stored
   dimension-major (each dimension's 16 slots contiguous).
2. ``coarse_scores``   - approximate attention score of the decode query
   against every mean summary key (ZoomR, Sec. 3.3 "Per-Head Importance
   Scoring and Voting", eq. for alpha_i). With grouped-query attention one
   score is kept per (sequence, KV head): the scores of the query heads that
   share that KV head are added (reading R1). Accumulated in float64 and
   rounded once to float32, the precision the selection is decided in.
3. ``select_topk``     - arg-top-k over the thoughts of one sequence and one
   KV head (ZoomR, Sec. 3.3, eq. for I_top-k). Ties go to the lower thought
   index, NaN ranks below every number, -0 equals +0 (reading R3).
4. ``attended_tokens`` - the zoomed-in token set: the recent window united
   with the full-resolution segments R_i of the selected thoughts (ZoomR,
   Sec. 3.3 eq. for I_f, restricted to I_w and the R_i; Appendix A.2,
   Algorithm 1, recent-window step). Window = the last W cached positions
   (reading R6). Written as a set union, so overlap is counted once.
5. ``attend``          - softmax(q K^T * scale) V over exactly those tokens
   (ZoomR, Sec. 2, eq. for A), two passes: max, then exp / sum / weighted V.

The append path (before a step's attention):

6. ``append_kv``       - write one new token's key and value per sequence
   into its paged cache, taking a fresh physical block from a free stack
   when the last block is full or the sequence has none (KV-cache
   management page, "Paged KV cache (PagedAttention)": allocation on demand,
   a new block only when the last one fills; ZoomR Algorithm 1, the append
   of k_t and v_t before scoring).
7. ``summary_keys``    - mean key of a completed thought per KV head
   (ZoomR, Sec. 3.3, eq. for the mean summary key; here the mean runs over
   the thought's own cached keys, reading R11), float64, rounded to float32
   and then to the cache dtype (bf16: round to nearest even).

The full multi-granularity set (ZoomR's consensus):

8. ``consensus``       - votes v_i = number of (layer, KV head) top-k sets that
   contain thought i, I_all = thoughts with a vote, consensus set I_c = the c
   thoughts with the most votes (ties to the lower index, reading R25), the
   agreement AG = sum of I_c's votes over all votes (ZoomR, Sec. 3.3 "Global
   Aggregation and Consensus", eqs. for I_all and v_i; Sec. 4, the AG metric).
9. ``zoom_attended_tokens`` - I_f = I_p U I_w U (R_i, i in I_c) U (S_i, i in
   I_s), I_s = I_all minus I_c (ZoomR, Sec. 3.3 "Constructing the Final
   Multi-Granularity Context", eq. for I_f), shared by every head.
10. ``zoom_decode_step`` - attention of every query head over I_f.

Accounting helpers pinned to printed figures:
``memory_savings`` (ZoomR, Sec. 3.5, eq. MS) and ``dense_kv_bytes`` (the
dense-cache sizing formula on the KV-cache management page, "Sizing the dense
cache").

Every function here has at least one pin in tests/test_oracle_pins.py that does
not re-run the function's own formula (worked figures from the pages, closed
forms, brute force over subsets, a library attention routine, invariants).
"""
from __future__ import annotations

import math

import numpy as np

BLOCK_SIZE = 16


# --------------------------------------------------------------------------
# 1. Paged cache read
# --------------------------------------------------------------------------
def gather_logical(pool: np.ndarray, table_row: np.ndarray, n_tokens: int,
                   slot_axis: int = 2) -> np.ndarray:
    """Logical view of one sequence's keys or values: float64 [n_tokens][Hkv][d].

    Token j is in physical block ``table_row[j // BLOCK_SIZE]`` at slot
    ``j % BLOCK_SIZE`` (paged KV cache, KV-cache management page, "Paged KV
    cache (PagedAttention)"). The page leaves the layout inside a block open;
    keys are [num_blocks][Hkv][16][d] (``slot_axis=2``, one row per slot) and
    values are [num_blocks][Hkv][d][16] (``slot_axis=3``, dimension-major).
    """
    j = np.arange(n_tokens)
    blocks = np.asarray(table_row)[j // BLOCK_SIZE]
    slots = j % BLOCK_SIZE
    pool = np.asarray(pool)
    if slot_axis == 2:
        # pool[blocks[t], :, slots[t], :] for every t -> [n_tokens][Hkv][d]
        return pool[blocks, :, slots, :].astype(np.float64)
    if slot_axis == 3:
        # pool[blocks[t], :, :, slots[t]] for every t -> [n_tokens][Hkv][d]
        return pool[blocks, :, :, slots].astype(np.float64)
    raise ValueError(slot_axis)


def gather_keys(k_pool, table_row, n_tokens):
    """Keys of one sequence in logical order (block layout [Hkv][16][d])."""
    return gather_logical(k_pool, table_row, n_tokens, slot_axis=2)


def gather_values(v_pool, table_row, n_tokens):
    """Values of one sequence in logical order (block layout [Hkv][d][16])."""
    return gather_logical(v_pool, table_row, n_tokens, slot_axis=3)


# --------------------------------------------------------------------------
# 2. Coarse scorer
# --------------------------------------------------------------------------
def coarse_scores(q: np.ndarray, summary_keys: np.ndarray, seq_ptr: np.ndarray,
                  n_kv_heads: int) -> np.ndarray:
    """alpha[i, g] for every thought i (rows of ``summary_keys``) and KV head g.

    q: [B][Hq][d]; summary_keys: [n_total][Hkv][d]; thoughts of sequence b are
    rows seq_ptr[b] .. seq_ptr[b+1]-1. Query head h belongs to KV head
    h // (Hq / Hkv). The score is sum over the group's query heads of the inner
    product q_h . kbar_i (ZoomR Sec. 3.3, eq. alpha; grouping per the GQA
    section of the KV-cache management page). Summed in float64 (the inner
    product of each head, then the heads in order) and rounded once to float32.
    """
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(summary_keys, dtype=np.float64)
    B, Hq, d = q64.shape
    G = Hq // n_kv_heads
    out = np.empty((k64.shape[0], n_kv_heads), dtype=np.float32)
    for b in range(B):
        lo, hi = int(seq_ptr[b]), int(seq_ptr[b + 1])
        for g in range(n_kv_heads):
            acc = np.zeros(hi - lo, dtype=np.float64)
            for h in range(g * G, (g + 1) * G):
                # inner products of query head h with every thought's key of head g
                acc = acc + k64[lo:hi, g, :] @ q64[b, h, :]
            out[lo:hi, g] = acc.astype(np.float32)
    return out


# --------------------------------------------------------------------------
# 3. Top-k selector
# --------------------------------------------------------------------------
def _rank_key(score: float, index: int):
    """Total order of the selection: larger score first; NaN after every number;
    among equal scores the lower thought index first (-0 == +0 as floats)."""
    s = float(score)
    if math.isnan(s):
        return (1, 0.0, index)
    return (0, -s, index)


def select_topk(scores: np.ndarray, seq_ptr: np.ndarray, k: int,
                n_kv_heads: int) -> np.ndarray:
    """sel[b, g, :]: the first min(k, N_b) thoughts of sequence b under the
    selection order for KV head g, listed in ascending thought index (local to
    the sequence), padded with -1 (ZoomR Sec. 3.3, eq. I_top-k; reading R4:
    k >= N_b keeps every thought, k = 0 keeps none)."""
    B = len(seq_ptr) - 1
    sel = np.full((B, n_kv_heads, k), -1, dtype=np.int32)
    for b in range(B):
        lo, hi = int(seq_ptr[b]), int(seq_ptr[b + 1])
        for g in range(n_kv_heads):
            s = scores[lo:hi, g]
            order = sorted(range(hi - lo), key=lambda i: _rank_key(s[i], i))
            chosen = sorted(order[:min(k, hi - lo)])
            sel[b, g, :len(chosen)] = chosen
    return sel


# --------------------------------------------------------------------------
# 4. Attended token set
# --------------------------------------------------------------------------
def attended_tokens(sel_row: np.ndarray, starts: np.ndarray, lens: np.ndarray,
                    n_cached: int, window: int) -> np.ndarray:
    """Ascending logical token indices attended for one (sequence, KV head).

    I = I_w  union  (union over selected i of R_i), with I_w the last ``window``
    cached positions [T - W, T) and R_i = [start_i, start_i + len_i)
    (ZoomR Sec. 3.3 eq. I_f without prompt sink and summary spans; Algorithm 1
    window step, read as the last W positions). ``starts``/``lens`` are the
    thought spans of this sequence indexed by local thought index.
    """
    tokens = set(range(max(0, n_cached - window), n_cached))
    for i in np.asarray(sel_row).tolist():
        if i < 0:
            continue
        s, ln = int(starts[i]), int(lens[i])
        tokens |= set(range(s, s + ln))
    return np.array(sorted(t for t in tokens if 0 <= t < n_cached), dtype=np.int64)


# --------------------------------------------------------------------------
# 5. Exact attention over a token set
# --------------------------------------------------------------------------
def attend(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float,
           return_weights: bool = False):
    """softmax(q K^T * scale) V for each query row (ZoomR Sec. 2, eq. A).

    q_rows: [G][d]; k_rows, v_rows: [n][d]. Float64, two passes: the logit
    maximum first, then p = exp(z - max), l = sum p, out = (p V) / l.
    An empty token set (n = 0) gives a zero output (reading R19).
    """
    q64 = np.asarray(q_rows, dtype=np.float64)
    k64 = np.asarray(k_rows, dtype=np.float64)
    v64 = np.asarray(v_rows, dtype=np.float64)
    G, d = q64.shape
    n = k64.shape[0]
    if n == 0:
        out = np.zeros((G, v64.shape[1] if v64.ndim == 2 else d))
        return (out, np.zeros((G, 0))) if return_weights else out
    z = (q64 @ k64.T) * float(scale)
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ v64) / l
    if return_weights:
        return out, p / l
    return out


# --------------------------------------------------------------------------
# Whole steps
# --------------------------------------------------------------------------
def sparse_decode_step(q, k_pool, v_pool, block_table, seq_lens, seq_ptr, starts, lens,
                       summary_keys, k, window, scale, sel=None, pairs=None):
    """One sparse decode step for a batch: scores -> top-k -> zoomed attention.

    Returns dict with ``scores`` [n_total][Hkv] f32, ``sel`` [B][Hkv][k] i32,
    ``out`` [B][Hq][d] f64 and ``n_attended`` [B][Hkv] i64. When ``sel`` is
    given it is used instead of the oracle's own selection (the near-tie rule
    compares outputs on the GPU's selected set). ``pairs`` restricts the
    attention to a list of (b, g); other output rows stay NaN.
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scores = coarse_scores(q, summary_keys, seq_ptr, Hkv)
    own_sel = select_topk(scores, seq_ptr, k, Hkv)
    use_sel = own_sel if sel is None else np.asarray(sel)
    out = np.full((B, Hq, d), np.nan)
    n_att = np.zeros((B, Hkv), dtype=np.int64)
    todo = pairs if pairs is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    cache = {}
    for b, g in todo:
        T = int(seq_lens[b])
        if b not in cache:
            cache = {b: (gather_keys(k_pool, block_table[b], T),
                         gather_values(v_pool, block_table[b], T))}
        K, V = cache[b]
        lo, hi = int(seq_ptr[b]), int(seq_ptr[b + 1])
        toks = attended_tokens(use_sel[b, g], starts[lo:hi], lens[lo:hi], T, window)
        n_att[b, g] = len(toks)
        out[b, g * G:(g + 1) * G] = attend(q[b, g * G:(g + 1) * G], K[toks, g], V[toks, g], scale)
    return {"scores": scores, "sel": own_sel, "out": out, "n_attended": n_att}


def consensus(sel_layers, seq_ptr, c):
    """Votes, consensus set and agreement per sequence.

    ``sel_layers`` [n_layers][B][Hkv][k] holds every (layer, KV head) top-k
    set (local thought indices, -1 = none). v_i counts the sets containing
    thought i (an indicator per set: a repeated index counts once); I_all is
    the thoughts with v_i > 0; I_c the min(c, |I_all|) of them with the most
    votes, ties to the lower index; AG = sum_{I_c} v_i / sum_{I_all} v_i (0
    with no votes). Returns votes [n_total] int32, cons [B][c] int32 (ascending,
    -1 padded) and agree [B] float64.
    """
    sel_layers = np.asarray(sel_layers)
    seq_ptr = np.asarray(seq_ptr)
    B = len(seq_ptr) - 1
    n_total = int(seq_ptr[-1])
    votes = np.zeros(n_total, dtype=np.int32)
    cons = np.full((B, max(c, 0)), -1, dtype=np.int32)
    agree = np.zeros(B, dtype=np.float64)
    for b in range(B):
        lo, hi = int(seq_ptr[b]), int(seq_ptr[b + 1])
        n = hi - lo
        for row in sel_layers[:, b].reshape(-1, sel_layers.shape[-1]):
            for i in set(int(x) for x in row if 0 <= x < n):
                votes[lo + i] += 1
        members = [i for i in range(n) if votes[lo + i] > 0]
        ranked = sorted(members, key=lambda i: (-int(votes[lo + i]), i))
        chosen = sorted(ranked[:max(c, 0)])
        cons[b, :len(chosen)] = chosen
        total = sum(int(votes[lo + i]) for i in members)
        agree[b] = sum(int(votes[lo + i]) for i in chosen) / total if total else 0.0
    return votes, cons, agree


def zoom_attended_tokens(votes_b, cons_row, starts, lens, sum_starts, sum_lens, n_prompt,
                         n_cached, window):
    """Ascending token indices of I_f for one sequence: the prompt [0, N_p),
    the window [T - W, T), the regular segment R_i of every consensus thought
    and the summary segment S_i of every other voted thought, as a set union
    inside [0, T). ``votes_b`` and the spans are indexed by local thought."""
    T = int(n_cached)
    tokens = set(range(0, min(int(n_prompt), T))) | set(range(max(0, T - window), T))
    cons = set(int(i) for i in cons_row if i >= 0)
    for i, v in enumerate(np.asarray(votes_b).tolist()):
        if v <= 0:
            continue
        if i in cons:
            s, ln = int(starts[i]), int(lens[i])
        else:
            s, ln = int(sum_starts[i]), int(sum_lens[i])
        tokens |= set(range(s, s + ln))
    return np.array(sorted(t for t in tokens if 0 <= t < T), dtype=np.int64)


def zoom_decode_step(q, k_pool, v_pool, block_table, seq_lens, seq_ptr, starts, lens,
                     sum_starts, sum_lens, votes, cons, n_prompt, window, scale):
    """Attention of every query head over its sequence's I_f (shared by all
    heads). Returns dict with ``out`` [B][Hq][d] f64 and ``n_attended`` [B]."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    n_att = np.zeros(B, dtype=np.int64)
    for b in range(B):
        T = int(seq_lens[b])
        K = gather_keys(k_pool, block_table[b], T)
        V = gather_values(v_pool, block_table[b], T)
        lo, hi = int(seq_ptr[b]), int(seq_ptr[b + 1])
        toks = zoom_attended_tokens(votes[lo:hi], cons[b], starts[lo:hi], lens[lo:hi],
                                    sum_starts[lo:hi], sum_lens[lo:hi], n_prompt, T, window)
        n_att[b] = len(toks)
        for g in range(Hkv):
            out[b, g * G:(g + 1) * G] = attend(q[b, g * G:(g + 1) * G], K[toks, g], V[toks, g],
                                               scale)
    return {"out": out, "n_attended": n_att}


def dense_decode_step(q, k_pool, v_pool, block_table, seq_lens, scale, pairs=None):
    """Full paged decode attention over every cached token (ZoomR Sec. 2 eq. A
    over the paged cache, KV-cache management page eq. 4 sum over blocks)."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    todo = pairs if pairs is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    cache = {}
    for b, g in todo:
        T = int(seq_lens[b])
        if b not in cache:
            cache = {b: (gather_keys(k_pool, block_table[b], T),
                         gather_values(v_pool, block_table[b], T))}
        K, V = cache[b]
        out[b, g * G:(g + 1) * G] = attend(q[b, g * G:(g + 1) * G], K[:, g], V[:, g], scale)
    return out


# --------------------------------------------------------------------------
# Accounting
# --------------------------------------------------------------------------
# --------------------------------------------------------------------------
# 6-7. Append path
# --------------------------------------------------------------------------
APPEND_OK, APPEND_NO_FREE_BLOCK, APPEND_TABLE_FULL = 0, 1, 2


def append_kv(k_pool, v_pool, block_table, seq_lens, k_new, v_new, free_blocks, free_count):
    """Append token T_b = seq_lens[b] of every sequence b, in order b = 0, 1, ...

    Before the write, a sequence whose cached length is a multiple of 16 (its
    last block is full, or it has none) pops the top of the free stack
    ``free_blocks[:free_count]`` into block_table[b][T_b // 16] (allocation
    on demand, KV-cache management page, paged KV cache). Then key row
    k_new[b][g] goes to k_pool[block][g][T_b % 16] and value v_new[b][g] to
    v_pool[block][g][:, T_b % 16] (dimension-major values), and seq_lens[b]
    grows by one. A sequence that needs a block when the stack is empty gets
    status 1, one whose table has no column left status 2; nothing of it
    changes. Works on copies; returns (k_pool, v_pool, block_table, seq_lens,
    free_count, status).
    """
    k_pool = np.array(k_pool, copy=True)
    v_pool = np.array(v_pool, copy=True)
    table = np.array(block_table, copy=True)
    lens = np.array(seq_lens, copy=True)
    status = np.zeros(len(lens), dtype=np.int32)
    top = int(free_count)
    for b in range(len(lens)):
        T = int(lens[b])
        col = T // BLOCK_SIZE
        if col >= table.shape[1]:
            status[b] = APPEND_TABLE_FULL
            continue
        if T % BLOCK_SIZE == 0:
            if top == 0:
                status[b] = APPEND_NO_FREE_BLOCK
                continue
            top -= 1
            table[b, col] = free_blocks[top]
        blk, slot = int(table[b, col]), T % BLOCK_SIZE
        k_pool[blk, :, slot, :] = k_new[b]
        v_pool[blk, :, :, slot] = v_new[b]
        lens[b] = T + 1
    return k_pool, v_pool, table, lens, top, status


def _round_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def summary_keys(k_pool, block_table, seq_ptr, starts, lens, which, dtype):
    """Mean summary key of each thought in ``which`` (global indices): for
    every KV head g, the mean of the thought's cached keys K[b, g, j] over
    j in [start, start + len) (ZoomR, Sec. 3.3, eq. for the mean summary key,
    over the thought's own keys: reading R11). float64 mean, rounded to
    float32, then to ``dtype`` ("bf16": nearest even). Returns
    float32 [len(which)][Hkv][d] holding the rounded values."""
    seq_ptr = np.asarray(seq_ptr)
    out = []
    for i in which:
        i = int(i)
        b = int(np.searchsorted(seq_ptr, i, side="right") - 1)
        s, n = int(starts[i]), int(lens[i])
        rows = gather_keys(k_pool, block_table[b], s + n)[s:s + n]
        m = rows.mean(axis=0).astype(np.float32)
        out.append(_round_bf16(m) if dtype == "bf16" else m)
    return np.array(out, dtype=np.float32).reshape(len(out), *np.asarray(k_pool).shape[1:2],
                                                   np.asarray(k_pool).shape[3])


def memory_savings(n_prompt, n_gen, n_window, c, len_regular, len_summary, n_all):
    """ZoomR Sec. 3.5, eq. MS: full-cache tokens over the tokens the selection
    keeps (prompt + c full segments + the other candidates' summaries + window)."""
    kept = n_prompt + c * len_regular + (n_all - c) * len_summary + n_window
    return (n_prompt + n_gen) / kept


def dense_kv_bytes(n_layers, n_tokens, n_kv_heads, head_dim, bytes_per_elem, batch=1):
    """Dense KV size: layers x 2 (K and V) x tokens x KV heads x head dim x bytes,
    times the number of sequences (KV-cache management page, "Sizing the dense
    cache", eq. 15)."""
    return n_layers * 2 * n_tokens * n_kv_heads * head_dim * bytes_per_elem * batch
