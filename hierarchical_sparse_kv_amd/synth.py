"""Seeded synthetic workloads for the sparse decode step.

These generators are the only code shared by the HIP path's tests, the CPU
oracle's tests and the benchmark. They draw inputs; they compute none of the
decode step (no scoring, selection, attention or output arithmetic).

Workload recipes (shapes follow the pages' setting: Llama-3.1-8B-shaped GQA
heads, 16K+ token reasoning outputs at batch 8, paragraph "thoughts" of a few
hundred tokens as in ZoomR Sec. 3.5's worked example):

* K, V ~ N(0, 1), rounded to the workload dtype, written straight into the
  paged pools, keys [num_blocks][Hkv][16][d] and values [num_blocks][Hkv][d][16]
  (the values are i.i.d., so drawing them in physical order is the same
  distribution as drawing them in logical order).
* Thought lengths are integers drawn until they cover the sequence; the last
  thought is cut to end at the last cached token.
* Summary key of a thought (per KV head) = mean of that thought's cached keys
  (float64, from the rounded keys) + N(0, 0.1^2) noise, rounded to dtype. This
  is an input recipe: the decode step consumes summary keys, it does not build
  them.
* Query: per (sequence, KV head) a few "planted" thoughts are drawn without
  replacement; every query head of the group gets
  q_scale * (sum of the planted summary keys) + its own N(0, q_noise^2) noise.
* Paging: "permuted" = one seeded permutation of every physical block id;
  "interleaved" = sequences allocate blocks in lockstep, one block per
  sequence per round, so consecutive blocks of a sequence are far apart.
* Multi-granularity layout (``summary`` spec set): ``prompt`` tokens first,
  then each thought's regular segment R_i followed by its summary segment S_i
  (lengths drawn from ``thought`` and ``summary``), until the next pair would
  pass the sequence end; the remaining tokens are the thought still being
  written (no summary yet, not a candidate). Summary keys then average the
  summary segment's keys (ZoomR's mean summary key) plus the same noise.
* Room to grow (append tests): ``extra_tokens`` widens the block table by that
  many tokens per sequence and ``spare_blocks`` adds unused physical blocks,
  returned as a free stack (``free_blocks``, top = last entry).

Large random tensors are drawn with a torch.Generator on the target device;
integer structure (lengths, tables, planted choices) with numpy from the same
seed, so it is identical on every device.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK_SIZE = 16

# Workload table. "k": None means every thought of the sequence (the dense
# case through the sparse path).
CONFIGS = {
    0: dict(name="tiny-fp32", B=1, Hq=8, Hkv=2, d=64, dtype="f32",
            seq_len=("fixed", 1024), thought=("fixed", 64), k=4, window=64,
            planted=2, q_scale=1.0, q_noise=0.5, kbar_noise=0.1, paging="permuted"),
    1: dict(name="llama8b-16k-b8", B=8, Hq=32, Hkv=8, d=128, dtype="bf16",
            seq_len=("fixed", 16384), thought=("uniform", 64, 512), k=8, window=128,
            planted=2, q_scale=1.0, q_noise=0.5, kbar_noise=0.1, paging="permuted"),
    2: dict(name="llama8b-16k-b8-dense", seed=1, B=8, Hq=32, Hkv=8, d=128, dtype="bf16",
            seq_len=("fixed", 16384), thought=("uniform", 64, 512), k=None, window=128,
            planted=2, q_scale=1.0, q_noise=0.5, kbar_noise=0.1, paging="permuted"),
    3: dict(name="ragged-b32", B=32, Hq=32, Hkv=8, d=128, dtype="bf16",
            seq_len=("uniform", 4096, 32768), thought=("uniform", 32, 1024), k=8, window=128,
            planted=2, q_scale=1.0, q_noise=0.5, kbar_noise=0.1, paging="interleaved"),
    4: dict(name="long-64k-b4", B=4, Hq=32, Hkv=8, d=128, dtype="bf16",
            seq_len=("fixed", 65536), thought=("loguniform", 32, 2048), k=16, window=256,
            planted=3, q_scale=3.0, q_noise=1.0, kbar_noise=0.1, paging="permuted"),
    # multi-granularity workload: prompt, regular + summary segments, sizes of
    # ZoomR Sec. 3.5's worked example (N_p 512, N_w 512, c 2, mean L_R 250,
    # mean L_S 20) on config 1's shapes
    5: dict(name="zoomr-16k-b8", B=8, Hq=32, Hkv=8, d=128, dtype="bf16",
            seq_len=("fixed", 16384), prompt=512, thought=("uniform", 100, 400),
            summary=("uniform", 10, 30), k=8, c=2, window=512,
            planted=2, q_scale=1.0, q_noise=0.5, kbar_noise=0.1, paging="permuted"),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "bf16": 2}


@dataclass
class Workload:
    """One decode step's inputs. Integer structure is numpy (host); the big
    tensors live on ``device``."""
    name: str
    seed: int
    dtype: str
    B: int
    Hq: int
    Hkv: int
    d: int
    k: int
    window: int
    seq_lens: np.ndarray          # int32 [B]
    block_table: np.ndarray       # int32 [B][max_blocks]; -1 = unused entry
    num_blocks: int
    seq_ptr: np.ndarray           # int32 [B+1]
    th_start: np.ndarray          # int32 [n_total]
    th_len: np.ndarray            # int32 [n_total]
    planted: np.ndarray           # int32 [B][Hkv][n_planted] (local thought index)
    k_pool: torch.Tensor          # [num_blocks][Hkv][16][d]
    v_pool: torch.Tensor          # [num_blocks][Hkv][d][16]
    summary_keys: torch.Tensor    # [n_total][Hkv][d]
    q: torch.Tensor               # [B][Hq][d]
    extra: dict = field(default_factory=dict)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def max_blocks(self):
        return self.block_table.shape[1]

    @property
    def n_total(self):
        return int(self.seq_ptr[-1])

    @property
    def max_per_seq(self):
        return int(np.max(np.diff(self.seq_ptr)))

    @property
    def scale(self):
        return float(np.float32(1.0 / math.sqrt(self.d)))


def _draw_one(rng, spec):
    """One integer length from a length spec."""
    kind = spec[0]
    if kind == "fixed":
        return int(spec[1])
    if kind == "uniform":
        return int(rng.integers(spec[1], spec[2] + 1))
    if kind == "loguniform":
        ln = int(math.floor(math.exp(rng.uniform(math.log(spec[1]), math.log(spec[2] + 1)))))
        return min(max(ln, spec[1]), spec[2])
    raise ValueError(kind)


def _draw_lengths(rng, spec, total):
    """Integer thought lengths covering ``total`` tokens; the last one is cut."""
    out = []
    acc = 0
    while acc < total:
        ln = min(_draw_one(rng, spec), total - acc)
        out.append(ln)
        acc += ln
    return out


def make_structure(cfg: dict, seed: int, seq_lens=None):
    """Integer structure only: sequence lengths, thought spans, block table,
    planted thoughts. Deterministic in ``seed`` on every device."""
    rng = np.random.default_rng(seed)
    B = cfg["B"]
    if seq_lens is None:
        kind = cfg["seq_len"]
        if kind[0] == "fixed":
            seq_lens = np.full(B, kind[1], dtype=np.int32)
        else:
            seq_lens = rng.integers(kind[1], kind[2] + 1, size=B).astype(np.int32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    starts, lens, ptr = [], [], [0]
    sstarts, slens = [], []
    for b in range(B):
        if cfg.get("summary") is None:
            ls = _draw_lengths(rng, cfg["thought"], int(seq_lens[b])) if seq_lens[b] > 0 else []
            s = 0
            for ln in ls:
                starts.append(s)
                lens.append(ln)
                s += ln
        else:
            T = int(seq_lens[b])
            s = min(int(cfg.get("prompt", 0)), T)
            while True:
                lr = _draw_one(rng, cfg["thought"])
                ls_ = _draw_one(rng, cfg["summary"])
                if s + lr + ls_ > T:
                    break
                starts.append(s)
                lens.append(lr)
                sstarts.append(s + lr)
                slens.append(ls_)
                s += lr + ls_
        ptr.append(len(starts))
    nblk = [(int(t) + BLOCK_SIZE - 1) // BLOCK_SIZE for t in seq_lens]
    extra = int(cfg.get("extra_tokens", 0))
    spare = int(cfg.get("spare_blocks", 0))
    max_blocks = max(1, max((int(t) + extra + BLOCK_SIZE - 1) // BLOCK_SIZE for t in seq_lens))
    num_blocks = max(1, sum(nblk) + spare)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    if cfg["paging"] == "permuted":
        perm = rng.permutation(num_blocks).astype(np.int32)
        pos = 0
        for b in range(B):
            table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
            pos += nblk[b]
        free_blocks = perm[pos:].copy()
    elif cfg["paging"] == "interleaved":
        nxt = 0
        for j in range(max_blocks):
            for b in range(B):
                if j < nblk[b]:
                    table[b, j] = nxt
                    nxt += 1
        free_blocks = np.arange(nxt, num_blocks, dtype=np.int32)
    else:
        raise ValueError(cfg["paging"])
    if spare == 0:
        free_blocks = np.zeros(0, dtype=np.int32)
    n_pl = cfg["planted"]
    planted = np.full((B, cfg["Hkv"], n_pl), -1, dtype=np.int32)
    for b in range(B):
        n_b = ptr[b + 1] - ptr[b]
        for g in range(cfg["Hkv"]):
            if n_b > 0:
                m = min(n_pl, n_b)
                planted[b, g, :m] = np.sort(rng.choice(n_b, size=m, replace=False))
    if not sstarts:
        sstarts, slens = list(starts), list(lens)
    return dict(seq_lens=seq_lens, block_table=table, num_blocks=num_blocks,
                free_blocks=free_blocks.astype(np.int32),
                sum_start=np.array(sstarts, dtype=np.int32),
                sum_len=np.array(slens, dtype=np.int32),
                seq_ptr=np.array(ptr, dtype=np.int32),
                th_start=np.array(starts, dtype=np.int32),
                th_len=np.array(lens, dtype=np.int32), planted=planted)


def _summary_keys(k_pool, st, cfg, gen, device):
    """mean of each thought's cached keys (float64) + noise, per KV head."""
    Hkv, d = cfg["Hkv"], cfg["d"]
    n_total = int(st["seq_ptr"][-1])
    out = torch.zeros((n_total, Hkv, d), dtype=torch.float64, device=device)
    table = torch.as_tensor(st["block_table"], device=device, dtype=torch.int64)
    for b in range(cfg["B"]):
        T = int(st["seq_lens"][b])
        lo, hi = int(st["seq_ptr"][b]), int(st["seq_ptr"][b + 1])
        if T == 0 or hi == lo:
            continue
        j = torch.arange(T, device=device)
        rows = k_pool[table[b, j // BLOCK_SIZE], :, j % BLOCK_SIZE, :].to(torch.float64)
        csum = torch.cat([torch.zeros((1, Hkv, d), dtype=torch.float64, device=device),
                          rows.cumsum(0)])
        s = torch.as_tensor(st["sum_start"][lo:hi], device=device, dtype=torch.int64)
        ln = torch.as_tensor(st["sum_len"][lo:hi], device=device, dtype=torch.int64)
        out[lo:hi] = (csum[s + ln] - csum[s]) / ln.to(torch.float64)[:, None, None]
        del rows, csum
    noise = torch.randn((n_total, Hkv, d), generator=gen, device=device, dtype=torch.float32)
    out = out + cfg["kbar_noise"] * noise.to(torch.float64)
    return out.to(TORCH_DTYPE[cfg["dtype"]])


def make_workload(cfg_id, seed=None, device="cpu", overrides=None, seq_lens=None,
                  value_seed=None) -> Workload:
    """Build workload ``cfg_id`` (a key of CONFIGS, or a dict) with ``seed``.

    ``overrides`` replaces entries of the recipe (used by the tests to shrink a
    workload while keeping its structure). ``value_seed`` (default ``seed``)
    seeds the tensor values only, so several layers can share one structure
    (lengths, thoughts, block table, planted thoughts) with their own K, V,
    summary keys and queries."""
    cfg = dict(CONFIGS[cfg_id]) if not isinstance(cfg_id, dict) else dict(cfg_id)
    if overrides:
        cfg.update(overrides)
    if seed is None:
        seed = cfg.get("seed", cfg_id if isinstance(cfg_id, int) else 0)
    st = make_structure(cfg, seed, seq_lens=seq_lens)
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed if value_seed is None else value_seed) * 7919 + 17)
    dt = TORCH_DTYPE[cfg["dtype"]]
    k_shape = (st["num_blocks"], cfg["Hkv"], BLOCK_SIZE, cfg["d"])   # one row per slot
    v_shape = (st["num_blocks"], cfg["Hkv"], cfg["d"], BLOCK_SIZE)   # dimension-major
    k_pool = torch.randn(k_shape, generator=gen, device=device, dtype=torch.float32).to(dt)
    v_pool = torch.randn(v_shape, generator=gen, device=device, dtype=torch.float32).to(dt)
    kbar = _summary_keys(k_pool, st, cfg, gen, device)
    B, Hq, Hkv, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    G = Hq // Hkv
    q = torch.randn((B, Hq, d), generator=gen, device=device, dtype=torch.float32) * cfg["q_noise"]
    kbar32 = kbar.to(torch.float32)
    for b in range(B):
        lo = int(st["seq_ptr"][b])
        for g in range(Hkv):
            base = torch.zeros(d, dtype=torch.float32, device=device)
            for i in st["planted"][b, g]:
                if i >= 0:
                    base = base + kbar32[lo + int(i), g]
            q[b, g * G:(g + 1) * G] += cfg["q_scale"] * base
    q = q.to(dt)
    n_max = int(np.max(np.diff(st["seq_ptr"]))) if B > 0 else 0
    k = cfg["k"] if cfg["k"] is not None else max(1, n_max)
    extra = {"cfg": cfg, "free_blocks": st["free_blocks"], "sum_start": st["sum_start"],
             "sum_len": st["sum_len"], "prompt": int(cfg.get("prompt", 0)),
             "c": int(cfg.get("c", 0))}
    return Workload(name=cfg["name"], seed=int(seed), dtype=cfg["dtype"], B=B, Hq=Hq, Hkv=Hkv,
                    d=d, k=int(k), window=int(cfg["window"]), seq_lens=st["seq_lens"],
                    block_table=st["block_table"], num_blocks=st["num_blocks"],
                    seq_ptr=st["seq_ptr"], th_start=st["th_start"], th_len=st["th_len"],
                    planted=st["planted"], k_pool=k_pool, v_pool=v_pool, summary_keys=kbar,
                    q=q, extra=extra)


def to_numpy_f32(t: torch.Tensor) -> np.ndarray:
    """Host float32 copy of a tensor (bf16 -> f32 is exact)."""
    return t.detach().to(torch.float32).cpu().numpy()
