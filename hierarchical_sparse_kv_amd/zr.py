"""ctypes binding of libzr (C ABI in include/zr.h).

The functions named like the C entry points (``zr_coarse_score`` ...) only
marshal arguments: device pointers come from ``torch.Tensor.data_ptr()``, the
stream from ``torch.cuda.current_stream()``; every step of the decode path
runs in the library's HIP kernels. There is no fallback: if libzr.so is
missing or fails to load, ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libzr.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "zr.h")

(ZR_OK, ZR_E_NULL, ZR_E_SHAPE, ZR_E_UNSUPPORTED, ZR_E_WORKSPACE, ZR_E_LAUNCH, ZR_E_ALIGN,
 ZR_E_SCRATCH) = range(8)
ZR_NOALLOC_SCRATCH_BYTES = 16 << 20
ZR_BLOCK_SIZE, ZR_MAX_K, ZR_MAX_THOUGHTS_PER_SEQ, ZR_MAX_PAIRS = 16, 1024, 8192, 4096
ZR_APPEND_OK, ZR_APPEND_NO_FREE_BLOCK, ZR_APPEND_TABLE_FULL, ZR_APPEND_BAD_BLOCK = range(4)
ZR_F32, ZR_BF16 = 0, 1
DTYPE_CODE = {torch.float32: ZR_F32, torch.bfloat16: ZR_BF16}


class ZrError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} -> {status} ({status_string(status)})")


class zr_geom(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class zr_thoughts(ctypes.Structure):
    _fields_ = [("seq_ptr", ctypes.c_void_p), ("start", ctypes.c_void_p),
                ("len", ctypes.c_void_p), ("summary_keys", ctypes.c_void_p),
                ("n_total", ctypes.c_int32), ("max_per_seq", ctypes.c_int32)]


_P = ctypes.c_void_p
_G = ctypes.POINTER(zr_geom)
_T = ctypes.POINTER(zr_thoughts)
_SIGS = {
    "zr_coarse_score": (ctypes.c_int, [_G, _P, _T, _P, _P]),
    "zr_select_topk": (ctypes.c_int, [_G, _T, _P, ctypes.c_int32, _P, _P]),
    "zr_score_topk": (ctypes.c_int, [_G, _P, _T, ctypes.c_int32, _P, _P, _P]),
    "zr_sparse_decode_attn": (ctypes.c_int, [_G, _P, _P, _P, _P, _P, _T, _P, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                             _P, _P, ctypes.c_size_t, _P]),
    "zr_sparse_decode_step": (ctypes.c_int, [_G, _P, _P, _P, _P, _P, _T, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                             _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "zr_sparse_decode_step_noalloc": (ctypes.c_int, [_G, _P, _P, _P, _P, _P, _T, ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.c_float,
                                                     ctypes.c_int32, _P, _P, _P, _P]),
    "zr_stage_selected": (ctypes.c_int, [_G, _P, _P, _P, _P, _T, _P, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_size_t,
                                         ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "zr_reuse_plan": (ctypes.c_int, [_G, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     _P, ctypes.c_size_t, _P]),
    "zr_sparse_decode_attn_reuse": (ctypes.c_int, [_G, _P, _P, _P, _P, _P, ctypes.c_float,
                                                   ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
    "zr_sparse_decode_attn_cached": (ctypes.c_int, [_G, _P, _P, _P, _P, _P, ctypes.c_int32,
                                                    ctypes.c_float, ctypes.c_int32, _P, _P,
                                                    ctypes.c_size_t, _P]),
    "zr_sparse_decode_attn_partials": (ctypes.c_int, [_G, _P, _P, _P, _P, _P, ctypes.c_int32,
                                                      ctypes.c_float, ctypes.c_int32, _P,
                                                      ctypes.c_size_t, _P]),
    "zr_attn_combine": (ctypes.c_int, [_G, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
    "zr_consensus": (ctypes.c_int, [_G, _T, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    _P, _P, _P, _P]),
    "zr_zoom_decode_attn": (ctypes.c_int, [_G, _P, _P, _P, _P, _P, _T, _P, _P, _P, _P,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_float, ctypes.c_int32, _P, _P,
                                           ctypes.c_size_t, _P]),
    "zr_append_kv": (ctypes.c_int, [_G, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "zr_summary_keys": (ctypes.c_int, [_G, _P, _P, _T, _P, ctypes.c_int32, _P, _P]),
    "zr_dense_paged_decode_attn": (ctypes.c_int, [_G, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                                  ctypes.c_size_t, _P]),
    "zr_workspace_bytes": (ctypes.c_size_t, [_G, ctypes.c_int32]),
    "zr_summary_prefetch_rule": (ctypes.c_int, [_G, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "zr_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libzr.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m hierarchical_sparse_kv_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def header_symbols() -> list[str]:
    """Entry points declared in include/zr.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:zr_status|size_t|const char\*)\s+(zr_\w+)\s*\(",
                                 text, flags=re.M)))


def status_string(status: int) -> str:
    return lib().zr_status_string(int(status)).decode()


# --------------------------------------------------------------------------
# The entry points, same names as the C ABI. Pointer arguments are ints
# (device addresses) or None; geom/thoughts are the ctypes structs.
# --------------------------------------------------------------------------
def zr_coarse_score(geom, q, th, scores, stream=None) -> int:
    return lib().zr_coarse_score(ctypes.byref(geom), q, ctypes.byref(th), scores, stream)


def zr_select_topk(geom, th, scores, k, sel, stream=None) -> int:
    return lib().zr_select_topk(ctypes.byref(geom), ctypes.byref(th), scores, int(k), sel, stream)


def zr_score_topk(geom, q, th, k, scores, sel, stream=None) -> int:
    return lib().zr_score_topk(ctypes.byref(geom), q, ctypes.byref(th), int(k), scores, sel,
                               stream)


def zr_sparse_decode_attn(geom, q, k_pool, v_pool, block_table, seq_lens, th, sel, k, window,
                          scale, max_attended, out, workspace, ws_bytes, stream=None) -> int:
    return lib().zr_sparse_decode_attn(ctypes.byref(geom), q, k_pool, v_pool, block_table,
                                       seq_lens, ctypes.byref(th), sel, int(k), int(window),
                                       float(scale), int(max_attended), out, workspace,
                                       int(ws_bytes), stream)


def zr_sparse_decode_step(geom, q, k_pool, v_pool, block_table, seq_lens, th, k, window, scale,
                          max_attended, scores, sel, out, workspace, ws_bytes, stream=None) -> int:
    return lib().zr_sparse_decode_step(ctypes.byref(geom), q, k_pool, v_pool, block_table,
                                       seq_lens, ctypes.byref(th), int(k), int(window),
                                       float(scale), int(max_attended), scores, sel, out,
                                       workspace, int(ws_bytes), stream)


def zr_sparse_decode_step_noalloc(geom, q, k_pool, v_pool, block_table, seq_lens, th, k, window,
                                  scale, max_attended, scores, sel, out, stream=None) -> int:
    return lib().zr_sparse_decode_step_noalloc(ctypes.byref(geom), q, k_pool, v_pool,
                                               block_table, seq_lens, ctypes.byref(th), int(k),
                                               int(window), float(scale), int(max_attended),
                                               scores, sel, out, stream)


def zr_stage_selected(geom, k_pool, v_pool, block_table, seq_lens, th, sel, k, window,
                      max_attended, workspace, ws_bytes, stage_blocks, k_stage, v_stage,
                      stage_workspace, stage_ws_bytes, dropped, stream=None) -> int:
    return lib().zr_stage_selected(ctypes.byref(geom), k_pool, v_pool, block_table, seq_lens,
                                   ctypes.byref(th), sel, int(k), int(window), int(max_attended),
                                   workspace, int(ws_bytes), int(stage_blocks), k_stage, v_stage,
                                   stage_workspace, int(stage_ws_bytes), dropped, stream)


def zr_reuse_plan(geom, block_table, seq_lens, window, horizon, max_attended, workspace, ws_bytes,
                  stream=None) -> int:
    return lib().zr_reuse_plan(ctypes.byref(geom), block_table, seq_lens, int(window), int(horizon),
                               int(max_attended), workspace, int(ws_bytes), stream)


def zr_sparse_decode_attn_reuse(geom, q, k_pool, v_pool, block_table, seq_lens, scale,
                                max_attended, out, workspace, ws_bytes, stream=None) -> int:
    return lib().zr_sparse_decode_attn_reuse(ctypes.byref(geom), q, k_pool, v_pool, block_table,
                                             seq_lens, float(scale), int(max_attended), out,
                                             workspace, int(ws_bytes), stream)


def zr_sparse_decode_attn_cached(geom, q, k_pool, v_pool, block_table, seq_lens, window, scale,
                                 max_attended, out, workspace, ws_bytes, stream=None) -> int:
    return lib().zr_sparse_decode_attn_cached(ctypes.byref(geom), q, k_pool, v_pool, block_table,
                                              seq_lens, int(window), float(scale),
                                              int(max_attended), out, workspace, int(ws_bytes),
                                              stream)


def zr_sparse_decode_attn_partials(geom, q, k_pool, v_pool, block_table, seq_lens, window,
                                   scale, max_attended, workspace, ws_bytes, stream=None) -> int:
    return lib().zr_sparse_decode_attn_partials(ctypes.byref(geom), q, k_pool, v_pool,
                                                block_table, seq_lens, int(window), float(scale),
                                                int(max_attended), workspace, int(ws_bytes),
                                                stream)


def zr_attn_combine(geom, max_attended, out, workspace, ws_bytes, stream=None) -> int:
    return lib().zr_attn_combine(ctypes.byref(geom), int(max_attended), out, workspace,
                                 int(ws_bytes), stream)


def zr_consensus(geom, th, sel, n_layers, k, c, votes, cons, agree, stream=None) -> int:
    return lib().zr_consensus(ctypes.byref(geom), ctypes.byref(th), sel, int(n_layers), int(k),
                              int(c), votes, cons, agree, stream)


def zr_zoom_decode_attn(geom, q, k_pool, v_pool, block_table, seq_lens, th, sum_start, sum_len,
                        votes, cons, c, n_prompt, window, scale, max_attended, out, workspace,
                        ws_bytes, stream=None) -> int:
    return lib().zr_zoom_decode_attn(ctypes.byref(geom), q, k_pool, v_pool, block_table,
                                     seq_lens, ctypes.byref(th), sum_start, sum_len, votes, cons,
                                     int(c), int(n_prompt), int(window), float(scale),
                                     int(max_attended), out, workspace, int(ws_bytes), stream)


def zr_append_kv(geom, k_pool, v_pool, block_table, seq_lens, k_new, v_new, free_blocks,
                 free_count, status, stream=None) -> int:
    return lib().zr_append_kv(ctypes.byref(geom), k_pool, v_pool, block_table, seq_lens, k_new,
                              v_new, free_blocks, free_count, status, stream)


def zr_summary_keys(geom, k_pool, block_table, th, which, n_which, summary_keys,
                    stream=None) -> int:
    return lib().zr_summary_keys(ctypes.byref(geom), k_pool, block_table, ctypes.byref(th),
                                 which, int(n_which), summary_keys, stream)


def zr_dense_paged_decode_attn(geom, q, k_pool, v_pool, block_table, seq_lens, scale, out,
                               workspace, ws_bytes, stream=None) -> int:
    return lib().zr_dense_paged_decode_attn(ctypes.byref(geom), q, k_pool, v_pool, block_table,
                                            seq_lens, float(scale), out, workspace,
                                            int(ws_bytes), stream)


def zr_workspace_bytes(geom, max_attended) -> int:
    return int(lib().zr_workspace_bytes(ctypes.byref(geom), int(max_attended)))


def zr_summary_prefetch_rule(geom, n_total, max_per_seq):
    """(status, rows, per_seq, margin) of the scorer's summary-key prefetch
    rule for this geometry and thought counts (host values)."""
    rows, margin = ctypes.c_int32(), ctypes.c_int32()
    per_seq = ctypes.c_float()
    st = lib().zr_summary_prefetch_rule(ctypes.byref(geom), int(n_total), int(max_per_seq),
                                        ctypes.addressof(rows), ctypes.addressof(per_seq),
                                        ctypes.addressof(margin))
    return st, rows.value, per_seq.value, margin.value


# --------------------------------------------------------------------------
# Torch-side marshalling helpers
# --------------------------------------------------------------------------
def _ptr(t):
    return None if t is None else t.data_ptr()


_hip = None


def pinned_device_ptr(t: torch.Tensor) -> int:
    """Device address of a pinned host tensor (hipHostGetDevicePointer), for
    pools kept in host memory and read by the kernels over PCIe. Raises if
    the tensor is not pinned or the runtime reports no device mapping."""
    global _hip
    if not (t.device.type == "cpu" and t.is_pinned()):
        raise ValueError("expected a pinned host tensor")
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipHostGetDevicePointer.restype = ctypes.c_int
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                 ctypes.c_void_p, ctypes.c_uint]
    dev = ctypes.c_void_p()
    err = _hip.hipHostGetDevicePointer(ctypes.byref(dev), ctypes.c_void_p(t.data_ptr()), 0)
    if err != 0 or not dev.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({err})")
    return int(dev.value)


def _pool_ptr(t):
    """Device address of a K/V pool: device memory, or pinned host memory."""
    return pinned_device_ptr(t) if t.device.type == "cpu" else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def check(fn, status):
    if status != ZR_OK:
        raise ZrError(fn, status)


class DeviceStep:
    """Device-resident inputs of one decode step plus the structs the C ABI
    takes. Holds references to every tensor whose address is passed."""

    def __init__(self, q, k_pool, v_pool, block_table, seq_lens, seq_ptr, th_start, th_len,
                 summary_keys, max_per_seq, k, window, scale, max_attended):
        dev = q.device
        i32 = lambda x: torch.as_tensor(np.asarray(x, np.int32) if not torch.is_tensor(x) else x,
                                        dtype=torch.int32, device=dev).contiguous()
        self.q = q.contiguous()
        self.k_pool, self.v_pool = k_pool.contiguous(), v_pool.contiguous()
        # pools may live in pinned host memory (read over PCIe)
        self.kp, self.vp = _pool_ptr(self.k_pool), _pool_ptr(self.v_pool)
        self.block_table = i32(block_table)
        self.seq_lens = i32(seq_lens)
        n_total = int(np.asarray(seq_ptr)[-1]) if not torch.is_tensor(seq_ptr) else int(seq_ptr[-1])
        pad1 = lambda t: t if t.numel() > 0 else torch.zeros(1, dtype=t.dtype, device=dev)
        self.seq_ptr = i32(seq_ptr)
        self.th_start, self.th_len = pad1(i32(th_start)), pad1(i32(th_len))
        self.summary_keys = summary_keys.contiguous()
        if self.summary_keys.numel() == 0:  # no thoughts at all: a valid, unread buffer
            self.summary_keys = torch.zeros(16, dtype=summary_keys.dtype, device=dev)
        B, Hq, d = self.q.shape
        nb, Hkv = self.k_pool.shape[0], self.k_pool.shape[1]
        self.geom = zr_geom(B, Hq, Hkv, d, 16, self.block_table.shape[1], nb,
                            DTYPE_CODE[self.q.dtype])
        self.th = zr_thoughts(_ptr(self.seq_ptr), _ptr(self.th_start), _ptr(self.th_len),
                              _ptr(self.summary_keys), n_total, int(max_per_seq))
        self.k, self.window, self.scale = int(k), int(window), float(scale)
        self.max_attended = int(max_attended)
        self.n_total = n_total
        self.scores = torch.empty((max(self.n_total, 1), Hkv), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, Hkv, max(self.k, 0)), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        ws = max(zr_workspace_bytes(self.geom, self.max_attended),
                 zr_workspace_bytes(self.geom, self.geom.max_blocks_per_seq * 16))
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)

    # one call per entry point; all on the current stream
    def coarse_score(self):
        check("zr_coarse_score", zr_coarse_score(self.geom, _ptr(self.q), self.th,
                                                 _ptr(self.scores), _stream()))

    def select_topk(self):
        check("zr_select_topk", zr_select_topk(self.geom, self.th, _ptr(self.scores), self.k,
                                               _ptr(self.sel) if self.k else None, _stream()))

    def score_topk(self, sel=None):
        """Scores and top-k in one call (zr_score_topk); sel defaults to self.sel."""
        sel = self.sel if sel is None else sel
        check("zr_score_topk", zr_score_topk(self.geom, _ptr(self.q), self.th, self.k,
                                             _ptr(self.scores), _ptr(sel) if self.k else None,
                                             _stream()))

    def sparse_attn(self, sel=None, out=None):
        sel = self.sel if sel is None else sel
        out = self.out if out is None else out
        check("zr_sparse_decode_attn", zr_sparse_decode_attn(
            self.geom, _ptr(self.q), self.kp, self.vp,
            _ptr(self.block_table), _ptr(self.seq_lens), self.th,
            _ptr(sel) if self.k else None, self.k, self.window, self.scale, self.max_attended,
            _ptr(out), _ptr(self.workspace), self.workspace.numel(), _stream()))

    def cached_attn(self, window, seq_lens=None, q=None, out=None, workspace=None):
        """Attention on the selection cached in the workspace by the last
        sparse_attn / step / zoom_attn call, with window `window` over
        `seq_lens`. `workspace`: another step's (same geometry), e.g. the
        multi-granularity set that every layer shares."""
        seq_lens = self.seq_lens if seq_lens is None else seq_lens
        q = self.q if q is None else q
        out = self.out if out is None else out
        ws = self.workspace if workspace is None else workspace
        check("zr_sparse_decode_attn_cached", zr_sparse_decode_attn_cached(
            self.geom, _ptr(q), self.kp, self.vp, _ptr(self.block_table),
            _ptr(seq_lens), int(window), self.scale, self.max_attended, _ptr(out),
            _ptr(ws), ws.numel(), _stream()))

    def reuse_plan(self, horizon, window=None, seq_lens=None, workspace=None):
        """Records of the split for the steps until the next semantic
        boundary (zr_reuse_plan) on the lists the last boundary call left in
        `workspace` (default: this step's)."""
        window = self.window if window is None else int(window)
        seq_lens = self.seq_lens if seq_lens is None else seq_lens
        ws = self.workspace if workspace is None else workspace
        check("zr_reuse_plan", zr_reuse_plan(
            self.geom, _ptr(self.block_table), _ptr(seq_lens), window, int(horizon),
            self.max_attended, _ptr(ws), ws.numel(), _stream()))

    def reuse_attn(self, seq_lens=None, q=None, out=None, partials=False, workspace=None):
        """Attention on the records of reuse_plan at the current lengths
        (zr_sparse_decode_attn_reuse); partials=True: the attention pass only.
        `workspace`: another step's (same geometry), e.g. the
        multi-granularity set that every layer shares."""
        seq_lens = self.seq_lens if seq_lens is None else seq_lens
        q = self.q if q is None else q
        out = self.out if out is None else out
        ws = self.workspace if workspace is None else workspace
        check("zr_sparse_decode_attn_reuse", zr_sparse_decode_attn_reuse(
            self.geom, _ptr(q), self.kp, self.vp, _ptr(self.block_table), _ptr(seq_lens),
            self.scale, self.max_attended, None if partials else _ptr(out),
            _ptr(ws), ws.numel(), _stream()))

    def cached_partials(self, window, seq_lens=None, q=None, workspace=None):
        """The attention pass of cached_attn alone: partial softmax states
        stay in the workspace for combine()."""
        seq_lens = self.seq_lens if seq_lens is None else seq_lens
        q = self.q if q is None else q
        ws = self.workspace if workspace is None else workspace
        check("zr_sparse_decode_attn_partials", zr_sparse_decode_attn_partials(
            self.geom, _ptr(q), self.kp, self.vp, _ptr(self.block_table),
            _ptr(seq_lens), int(window), self.scale, self.max_attended,
            _ptr(ws), ws.numel(), _stream()))

    def combine(self, out=None, workspace=None):
        """Merge the partial states the last attention call left in the
        workspace into `out`."""
        out = self.out if out is None else out
        ws = self.workspace if workspace is None else workspace
        check("zr_attn_combine", zr_attn_combine(
            self.geom, self.max_attended, _ptr(out), _ptr(ws), ws.numel(), _stream()))

    def append(self, k_new, v_new, free_blocks, free_count, status):
        """Append one token per sequence (zr_append_kv); updates this step's
        block table and sequence lengths in place."""
        check("zr_append_kv", zr_append_kv(
            self.geom, self.kp, self.vp, _ptr(self.block_table),
            _ptr(self.seq_lens), _ptr(k_new.contiguous()), _ptr(v_new.contiguous()),
            _ptr(free_blocks), _ptr(free_count), _ptr(status), _stream()))

    def compute_summary_keys(self, which, out=None):
        """Mean summary keys of the thoughts `which` (zr_summary_keys), written
        into `out` (default: this step's summary keys)."""
        out = self.summary_keys if out is None else out
        check("zr_summary_keys", zr_summary_keys(
            self.geom, self.kp, _ptr(self.block_table), self.th, _ptr(which),
            which.numel(), _ptr(out), _stream()))

    def consensus(self, sel_stack, c, votes, cons, agree):
        """Votes, consensus set and agreement over stacked selections
        [n_layers][B][Hkv][k] (zr_consensus)."""
        sel_stack = sel_stack.contiguous()
        n_layers, k = sel_stack.shape[0], sel_stack.shape[-1]
        check("zr_consensus", zr_consensus(
            self.geom, self.th, _ptr(sel_stack), n_layers, k, int(c), _ptr(votes),
            _ptr(cons) if c else None, _ptr(agree), _stream()))

    def zoom_attn(self, sum_start, sum_len, votes, cons, c, n_prompt, window=None, out=None):
        """Attention over the multi-granularity set (zr_zoom_decode_attn)."""
        window = self.window if window is None else int(window)
        out = self.out if out is None else out
        check("zr_zoom_decode_attn", zr_zoom_decode_attn(
            self.geom, _ptr(self.q), self.kp, self.vp,
            _ptr(self.block_table), _ptr(self.seq_lens), self.th, _ptr(sum_start),
            _ptr(sum_len), _ptr(votes), _ptr(cons) if c else None, int(c), int(n_prompt), window,
            self.scale, self.max_attended, _ptr(out), _ptr(self.workspace),
            self.workspace.numel(), _stream()))

    def dense_attn(self, out=None):
        out = self.out if out is None else out
        check("zr_dense_paged_decode_attn", zr_dense_paged_decode_attn(
            self.geom, _ptr(self.q), self.kp, self.vp,
            _ptr(self.block_table), _ptr(self.seq_lens), self.scale, _ptr(out),
            _ptr(self.workspace), self.workspace.numel(), _stream()))

    def step(self, scores=None, sel=None, out=None, seq_lens=None):
        """One sparse decode step as one call (zr_sparse_decode_step)."""
        seq_lens = self.seq_lens if seq_lens is None else seq_lens
        scores = self.scores if scores is None else scores
        sel = self.sel if sel is None else sel
        out = self.out if out is None else out
        check("zr_sparse_decode_step", zr_sparse_decode_step(
            self.geom, _ptr(self.q), self.kp, self.vp,
            _ptr(self.block_table), _ptr(seq_lens), self.th, self.k, self.window,
            self.scale, self.max_attended, _ptr(scores), _ptr(sel) if self.k else None,
            _ptr(out), _ptr(self.workspace), self.workspace.numel(), _stream()))

    def step_noalloc(self, scores=None, sel=None, out=None):
        """The same step through zr_sparse_decode_step_noalloc (no workspace:
        the library's built-in device scratch)."""
        scores = self.scores if scores is None else scores
        sel = self.sel if sel is None else sel
        out = self.out if out is None else out
        check("zr_sparse_decode_step_noalloc", zr_sparse_decode_step_noalloc(
            self.geom, _ptr(self.q), self.kp, self.vp, _ptr(self.block_table),
            _ptr(self.seq_lens), self.th, self.k, self.window, self.scale, self.max_attended,
            _ptr(scores), _ptr(sel) if self.k else None, _ptr(out), _stream()))

    def stage(self, staging, sel=None, window=None):
        """Build this step's block lists from `sel` and copy the listed K/V
        tiles (and the window's) from the pools, which may be in pinned host
        memory, into `staging` (zr_stage_selected)."""
        sel = self.sel if sel is None else sel
        window = self.window if window is None else int(window)
        check("zr_stage_selected", zr_stage_selected(
            self.geom, self.kp, self.vp, _ptr(self.block_table), _ptr(self.seq_lens), self.th,
            _ptr(sel) if self.k else None, self.k, window, self.max_attended,
            _ptr(self.workspace), self.workspace.numel(), staging.stage_blocks,
            _ptr(staging.k_stage), _ptr(staging.v_stage), _ptr(staging.workspace),
            staging.workspace.numel(), _ptr(staging.dropped), _stream()))

    def attend_staged(self, staging, out=None, q=None):
        """Attention over what the last stage() call moved into `staging`
        (zr_sparse_decode_attn_cached on the staging pools, no window)."""
        out = self.out if out is None else out
        q = self.q if q is None else q
        check("zr_sparse_decode_attn_cached", zr_sparse_decode_attn_cached(
            staging.geom, _ptr(q), _ptr(staging.k_stage), _ptr(staging.v_stage),
            _ptr(self.block_table), _ptr(self.seq_lens), 0, self.scale, self.max_attended,
            _ptr(out), _ptr(staging.workspace), staging.workspace.numel(), _stream()))

    def step_calls(self):
        """The same step as three calls: score, select, attend."""
        self.coarse_score()
        self.select_topk()
        self.sparse_attn()


class Staging:
    """Device buffers that receive a step's attended K/V tiles
    (zr_stage_selected): staging pools for `stage_blocks` blocks per
    sequence, their block lists and the per-pair count of entries that did
    not fit. `geom` is the staged geometry (num_blocks = batch *
    stage_blocks, lists one entry longer than a block-table row)."""

    def __init__(self, step: "DeviceStep", stage_blocks: int):
        g = step.geom
        self.stage_blocks = int(stage_blocks)
        dev = step.q.device
        nb = max(g.batch * self.stage_blocks, 1)
        dt = step.q.dtype
        self.k_stage = torch.empty((nb, g.n_kv_heads, 16, g.head_dim), dtype=dt, device=dev)
        self.v_stage = torch.empty((nb, g.n_kv_heads, g.head_dim, 16), dtype=dt, device=dev)
        self.geom = zr_geom(g.batch, g.n_q_heads, g.n_kv_heads, g.head_dim, 16,
                            g.max_blocks_per_seq + 1, nb, g.dtype)
        ws = zr_workspace_bytes(self.geom, step.max_attended)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.dropped = torch.empty(max(g.batch * g.n_kv_heads, 1), dtype=torch.int32, device=dev)


def max_attended_bound(seq_lens, seq_ptr, th_len, k, window):
    """Upper bound on attended tokens per (sequence, KV head): the window plus
    the k longest thoughts of the sequence, at most the sequence length."""
    best = 0
    for b in range(len(seq_lens)):
        lens = np.sort(np.asarray(th_len[seq_ptr[b]:seq_ptr[b + 1]]))[::-1]
        best = max(best, min(int(seq_lens[b]), int(window) + int(lens[:k].sum())))
    return best


def step_from_workload(w, k=None, meta=None):
    """DeviceStep for a synth.Workload (tensors already on the GPU). `meta`: a
    DeviceStep whose per-sequence tensors (block table, lengths, thought spans)
    this one shares, as the layers of one model share them (each layer has
    its own pools, summary keys and queries); the workload must have the same
    structure."""
    k = w.k if k is None else k
    bt, lens, ptr, ts, tl = (w.block_table, w.seq_lens, w.seq_ptr, w.th_start, w.th_len)
    if meta is not None:
        assert np.array_equal(meta.block_table.cpu().numpy(), w.block_table)
        assert np.array_equal(meta.seq_lens.cpu().numpy(), w.seq_lens)
        bt, lens, ptr, ts, tl = (meta.block_table, meta.seq_lens, meta.seq_ptr, meta.th_start,
                                 meta.th_len)
    return DeviceStep(w.q, w.k_pool, w.v_pool, bt, lens, ptr, ts, tl, w.summary_keys,
                      max(w.max_per_seq, 1), k, w.window, w.scale,
                      max_attended_bound(w.seq_lens, w.seq_ptr, w.th_len, k, w.window))
