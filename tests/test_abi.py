"""The C-ABI library loads, exports every entry point include/zr.h declares,
and rejects bad host-side arguments before enqueuing anything (these calls
return during validation, so they need no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from hierarchical_sparse_kv_amd import zr

FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced on error paths


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(zr.LIB_PATH):
        from hierarchical_sparse_kv_amd import build
        build.build()
    return zr.lib()


def test_exports_every_declared_symbol(L):
    declared = zr.header_symbols()
    assert declared == sorted(["zr_coarse_score", "zr_select_topk", "zr_score_topk",
                               "zr_sparse_decode_attn",
                               "zr_sparse_decode_attn_cached", "zr_sparse_decode_step",
                               "zr_sparse_decode_step_noalloc",
                               "zr_sparse_decode_attn_partials", "zr_attn_combine",
                               "zr_dense_paged_decode_attn", "zr_append_kv", "zr_summary_keys",
                               "zr_consensus", "zr_zoom_decode_attn",
                               "zr_summary_prefetch_rule", "zr_stage_selected",
                               "zr_reuse_plan", "zr_sparse_decode_attn_reuse",
                               "zr_workspace_bytes", "zr_status_string"])
    out = subprocess.run(["nm", "-D", "--defined-only", zr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if l.split()[-2] == "T")
    assert exported == declared
    for name in declared:
        assert hasattr(L, name)


def test_header_constants_match_the_binding():
    """Every #define ZR_* of include/zr.h that the binding mirrors has its value."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hdr = open(os.path.join(root, "include", "zr.h")).read()
    defs = {}
    for name, val, shift in re.findall(r"#define (ZR_[A-Z_0-9]+) \(?(\d+)u?(?: << (\d+))?", hdr):
        defs[name] = int(val) << (int(shift) if shift else 0)
    mirrored = [n for n in defs if hasattr(zr, n)]
    assert {"ZR_BLOCK_SIZE", "ZR_MAX_K", "ZR_MAX_THOUGHTS_PER_SEQ", "ZR_MAX_PAIRS",
            "ZR_NOALLOC_SCRATCH_BYTES", "ZR_APPEND_BAD_BLOCK"} <= set(mirrored)
    for n in mirrored:
        assert getattr(zr, n) == defs[n], n


def test_status_strings(L):
    for s in range(8):
        assert zr.status_string(s)
    assert zr.status_string(99) == "unknown zr_status"


def _geom(**kw):
    d = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
             max_blocks_per_seq=4, num_blocks=8, dtype=zr.ZR_BF16)
    d.update(kw)
    return zr.zr_geom(**d)


def _th(**kw):
    d = dict(seq_ptr=FAKE, start=FAKE, len=FAKE, summary_keys=FAKE, n_total=5, max_per_seq=3)
    d.update(kw)
    return zr.zr_thoughts(**d)


def test_workspace_bytes(L):
    g = _geom()
    n = zr.zr_workspace_bytes(g, 1000)
    # 4 (sequence, KV head) pairs of at most ceil(1000/16) + 2 blocks, 8 blocks
    # per workgroup -> 33 workgroups; partial slots = workgroups + pairs.
    # Regions, each 16-byte aligned: first workgroup per pair [pairs + 1],
    # list length per pair [pairs], the window start each pair's list was
    # clipped at [pairs], block lists [pairs][max_blocks] (8 bytes each), m
    # and l [slots][G], acc [slots][G][128], then for the calls
    # between semantic boundaries one 1616-byte segment record per workgroup,
    # the boundary's lengths [batch] and 16 bytes of settings
    up16 = lambda x: (x + 15) // 16 * 16
    nwg = -(-4 * (-(-1000 // 16) + 2) // 8)
    slots = nwg + 4
    lists = up16(5 * 4) + 2 * up16(4 * 4) + 4 * 4 * 8
    reuse = lambda nwg: nwg * 1616 + up16(2 * 4) + up16(5 * 4) + 16
    assert n == lists + 2 * up16(slots * 4 * 4) + slots * 4 * 128 * 4 + reuse(nwg)
    # the grid is capped at 512 workgroups
    big = zr.zr_workspace_bytes(g, 10 ** 6)
    assert big == lists + 2 * up16(516 * 16) + 516 * 4 * 128 * 4 + reuse(512)
    assert zr.zr_workspace_bytes(_geom(head_dim=96), 10) == 0
    assert zr.zr_workspace_bytes(g, -1) == 0
    assert zr.zr_workspace_bytes(_geom(batch=1024, n_q_heads=32, n_kv_heads=8), 10) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=6, n_kv_heads=4), zr.ZR_E_SHAPE),
    (dict(n_q_heads=48, n_kv_heads=2), zr.ZR_E_UNSUPPORTED),
    (dict(n_q_heads=64, n_kv_heads=2, dtype=zr.ZR_F32), zr.ZR_E_UNSUPPORTED),
    (dict(head_dim=96), zr.ZR_E_UNSUPPORTED),
    (dict(block_size=32), zr.ZR_E_UNSUPPORTED),
    (dict(dtype=7), zr.ZR_E_UNSUPPORTED),
    (dict(batch=-1), zr.ZR_E_SHAPE),
    (dict(num_blocks=0), zr.ZR_E_SHAPE),
])
def test_geometry_rejected(L, kw, code):
    g = _geom(**kw)
    assert zr.zr_coarse_score(g, FAKE, _th(), FAKE) == code
    assert zr.zr_sparse_decode_attn(g, FAKE, FAKE, FAKE, FAKE, FAKE, _th(), FAKE, 2, 16, 0.1,
                                    100, FAKE, FAKE, 1 << 20) == code
    assert zr.zr_dense_paged_decode_attn(g, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE,
                                         1 << 20) == code
    assert zr.zr_sparse_decode_step(g, FAKE, FAKE, FAKE, FAKE, FAKE, _th(), 2, 16, 0.1, 100,
                                    FAKE, FAKE, FAKE, FAKE, 1 << 20) == code
    assert zr.zr_sparse_decode_attn_cached(g, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 0.1, 100, FAKE,
                                           FAKE, 1 << 20) == code


def test_null_and_range_errors(L):
    g = _geom()
    assert zr.lib().zr_coarse_score(None, FAKE, ctypes.byref(_th()), FAKE, None) == zr.ZR_E_NULL
    assert zr.zr_coarse_score(g, None, _th(), FAKE) == zr.ZR_E_NULL
    assert zr.zr_coarse_score(g, FAKE, _th(summary_keys=None), FAKE) == zr.ZR_E_NULL
    assert zr.zr_coarse_score(g, FAKE + 4, _th(), FAKE) == zr.ZR_E_ALIGN
    assert zr.zr_coarse_score(g, FAKE, _th(max_per_seq=100000), FAKE) == zr.ZR_E_UNSUPPORTED
    assert zr.zr_select_topk(g, _th(), FAKE, -1, FAKE) == zr.ZR_E_SHAPE
    assert zr.zr_select_topk(g, _th(), FAKE, 1025, FAKE) == zr.ZR_E_SHAPE
    assert zr.zr_select_topk(g, _th(), FAKE, 3, None) == zr.ZR_E_NULL
    assert zr.zr_select_topk(g, _th(seq_ptr=None), FAKE, 3, FAKE) == zr.ZR_E_NULL
    st = lambda **kw: zr.zr_score_topk(**dict(dict(geom=g, q=FAKE, th=_th(), k=3, scores=FAKE,
                                                    sel=FAKE), **kw))
    assert st(k=-1) == zr.ZR_E_SHAPE
    assert st(k=1025) == zr.ZR_E_SHAPE
    assert st(sel=None) == zr.ZR_E_NULL
    assert st(scores=None) == zr.ZR_E_NULL
    assert st(q=None) == zr.ZR_E_NULL
    assert st(th=_th(summary_keys=None)) == zr.ZR_E_NULL
    assert st(q=FAKE + 4) == zr.ZR_E_ALIGN
    assert st(th=_th(max_per_seq=100000)) == zr.ZR_E_UNSUPPORTED
    args = lambda **kw: dict(dict(geom=g, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_table=FAKE,
                                  seq_lens=FAKE, th=_th(), sel=FAKE, k=2, window=16, scale=0.1,
                                  max_attended=100, out=FAKE, workspace=FAKE,
                                  ws_bytes=1 << 20), **kw)
    sp = lambda **kw: zr.zr_sparse_decode_attn(**args(**kw))
    assert sp(k=-1) == zr.ZR_E_SHAPE
    assert sp(window=-1) == zr.ZR_E_SHAPE
    assert sp(max_attended=-5) == zr.ZR_E_SHAPE
    assert sp(scale=float("nan")) == zr.ZR_E_SHAPE
    assert sp(sel=None) == zr.ZR_E_NULL
    assert sp(out=None) == zr.ZR_E_NULL
    assert sp(v_pool=FAKE + 8) == zr.ZR_E_ALIGN
    assert sp(out=FAKE + 4) == zr.ZR_E_ALIGN
    assert sp(workspace=None) == zr.ZR_E_WORKSPACE
    assert sp(ws_bytes=16) == zr.ZR_E_WORKSPACE
    need = zr.zr_workspace_bytes(g, 100)
    assert sp(ws_bytes=need - 1) == zr.ZR_E_WORKSPACE
    assert zr.zr_dense_paged_decode_attn(g, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, 64) \
        == zr.ZR_E_WORKSPACE
    # all pairs' list entries must be countable in int32 (4096 pairs x 2 x 300000 blocks)
    big = _geom(batch=512, n_kv_heads=8, n_q_heads=32, max_blocks_per_seq=300000)
    assert zr.zr_dense_paged_decode_attn(big, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE,
                                         1 << 40) == zr.ZR_E_UNSUPPORTED


def test_step_errors(L):
    g = _geom()
    args = lambda **kw: dict(dict(geom=g, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_table=FAKE,
                                  seq_lens=FAKE, th=_th(), k=2, window=16, scale=0.1,
                                  max_attended=100, scores=FAKE, sel=FAKE, out=FAKE,
                                  workspace=FAKE, ws_bytes=1 << 20), **kw)
    st = lambda **kw: zr.zr_sparse_decode_step(**args(**kw))
    assert st(k=-1) == zr.ZR_E_SHAPE
    assert st(k=2000) == zr.ZR_E_SHAPE
    assert st(window=-3) == zr.ZR_E_SHAPE
    assert st(scores=None) == zr.ZR_E_NULL
    assert st(sel=None) == zr.ZR_E_NULL
    assert st(th=_th(summary_keys=None)) == zr.ZR_E_NULL
    assert st(th=_th(summary_keys=FAKE + 2)) == zr.ZR_E_ALIGN
    assert st(ws_bytes=zr.zr_workspace_bytes(g, 100) - 1) == zr.ZR_E_WORKSPACE
    # block lists too large for the pair kernel's on-chip memory
    assert st(geom=_geom(max_blocks_per_seq=60000, batch=1), ws_bytes=1 << 30) == zr.ZR_E_UNSUPPORTED


def test_cached_errors(L):
    g = _geom()
    c = lambda **kw: zr.zr_sparse_decode_attn_cached(**dict(dict(
        geom=g, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_table=FAKE, seq_lens=FAKE, window=16,
        scale=0.1, max_attended=100, out=FAKE, workspace=FAKE, ws_bytes=1 << 20), **kw))
    assert c(window=-1) == zr.ZR_E_SHAPE
    assert c(seq_lens=None) == zr.ZR_E_NULL
    assert c(q=FAKE + 2) == zr.ZR_E_ALIGN
    assert c(workspace=None) == zr.ZR_E_WORKSPACE
    assert c(scale=float("inf")) == zr.ZR_E_SHAPE


def test_partials_and_combine_errors(L):
    g = _geom()
    pt = lambda **kw: zr.zr_sparse_decode_attn_partials(**dict(dict(
        geom=g, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_table=FAKE, seq_lens=FAKE, window=16,
        scale=0.1, max_attended=100, workspace=FAKE, ws_bytes=1 << 20), **kw))
    assert pt(window=-1) == zr.ZR_E_SHAPE
    assert pt(q=None) == zr.ZR_E_NULL
    assert pt(v_pool=FAKE + 4) == zr.ZR_E_ALIGN
    assert pt(workspace=None) == zr.ZR_E_WORKSPACE
    assert pt(ws_bytes=16) == zr.ZR_E_WORKSPACE
    assert pt(max_attended=-1) == zr.ZR_E_SHAPE
    assert pt(geom=_geom(head_dim=96)) == zr.ZR_E_UNSUPPORTED
    cb = lambda **kw: zr.zr_attn_combine(**dict(dict(
        geom=g, max_attended=100, out=FAKE, workspace=FAKE, ws_bytes=1 << 20), **kw))
    assert cb(out=None) == zr.ZR_E_NULL
    assert cb(out=FAKE + 4) == zr.ZR_E_ALIGN
    assert cb(max_attended=-1) == zr.ZR_E_SHAPE
    assert cb(workspace=None) == zr.ZR_E_WORKSPACE
    assert cb(workspace=FAKE + 8) == zr.ZR_E_WORKSPACE
    # the layout grows with max_attended: a workspace sized for a small bound is too small
    small = zr.zr_workspace_bytes(g, 16)
    assert cb(max_attended=1 << 20, ws_bytes=small) == zr.ZR_E_WORKSPACE
    assert cb(geom=_geom(n_q_heads=12)) == zr.ZR_E_UNSUPPORTED
    assert cb(geom=_geom(batch=0), workspace=None) == zr.ZR_OK  # nothing to do


def test_append_and_summary_errors(L):
    g = _geom()
    ap = lambda **kw: zr.zr_append_kv(**dict(dict(
        geom=g, k_pool=FAKE, v_pool=FAKE, block_table=FAKE, seq_lens=FAKE, k_new=FAKE,
        v_new=FAKE, free_blocks=FAKE, free_count=FAKE, status=FAKE), **kw))
    assert ap(free_count=None) == zr.ZR_E_NULL
    assert ap(status=None) == zr.ZR_E_NULL
    assert ap(k_new=FAKE + 2) == zr.ZR_E_ALIGN
    assert ap(geom=_geom(head_dim=96)) == zr.ZR_E_UNSUPPORTED
    assert ap(geom=_geom(batch=0), k_pool=None) == zr.ZR_OK  # nothing to do
    sk = lambda **kw: zr.zr_summary_keys(**dict(dict(
        geom=g, k_pool=FAKE, block_table=FAKE, th=_th(), which=FAKE, n_which=3,
        summary_keys=FAKE), **kw))
    assert sk(n_which=-1) == zr.ZR_E_SHAPE
    assert sk(which=None) == zr.ZR_E_NULL
    assert sk(summary_keys=FAKE + 8) == zr.ZR_E_ALIGN
    assert sk(th=_th(len=None)) == zr.ZR_E_NULL
    assert sk(n_which=0, which=None) == zr.ZR_OK


def test_consensus_and_zoom_errors(L):
    g = _geom()
    cs = lambda **kw: zr.zr_consensus(**dict(dict(
        geom=g, th=_th(), sel=FAKE, n_layers=2, k=4, c=2, votes=FAKE, cons=FAKE, agree=FAKE),
        **kw))
    assert cs(c=-1) == zr.ZR_E_SHAPE
    assert cs(k=2000) == zr.ZR_E_SHAPE
    assert cs(n_layers=-1) == zr.ZR_E_SHAPE
    assert cs(votes=None) == zr.ZR_E_NULL
    assert cs(cons=None) == zr.ZR_E_NULL
    assert cs(sel=None) == zr.ZR_E_NULL
    assert cs(th=_th(max_per_seq=9000)) == zr.ZR_E_UNSUPPORTED
    zm = lambda **kw: zr.zr_zoom_decode_attn(**dict(dict(
        geom=g, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_table=FAKE, seq_lens=FAKE, th=_th(),
        sum_start=FAKE, sum_len=FAKE, votes=FAKE, cons=FAKE, c=2, n_prompt=16, window=16,
        scale=0.1, max_attended=100, out=FAKE, workspace=FAKE, ws_bytes=1 << 20), **kw))
    assert zm(n_prompt=-1) == zr.ZR_E_SHAPE
    assert zm(c=-2) == zr.ZR_E_SHAPE
    assert zm(sum_len=None) == zr.ZR_E_NULL
    assert zm(cons=None) == zr.ZR_E_NULL
    assert zm(out=FAKE + 4) == zr.ZR_E_ALIGN
    assert zm(ws_bytes=8) == zr.ZR_E_WORKSPACE


def test_summary_prefetch_rule(L):
    """The scorer's prefetch rule, read from the library (no GPU): on for even
    batches whose sequences fit one batch of rows, off otherwise; argument
    errors are reported."""
    g = _geom(batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype=zr.ZR_BF16)
    st, rows, per, margin = zr.zr_summary_prefetch_rule(g, 456, 64)
    assert st == zr.ZR_OK and rows == 64 and abs(per - 57.0) < 1e-6 and margin == 3
    # uneven (max per sequence above 1.25x the mean) or too many per sequence: off
    assert zr.zr_summary_prefetch_rule(g, 456, 80)[1:] == (0, 0.0, 0)
    assert zr.zr_summary_prefetch_rule(g, 8 * 100, 100)[1:] == (0, 0.0, 0)
    assert zr.zr_summary_prefetch_rule(g, 0, 0)[1:] == (0, 0.0, 0)
    # fp32, head_dim 128: 32 rows per batch
    g32 = _geom(batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype=zr.ZR_F32)
    assert zr.zr_summary_prefetch_rule(g32, 8 * 30, 32)[1] == 32
    assert zr.zr_summary_prefetch_rule(g, -1, 0)[0] == zr.ZR_E_SHAPE
    assert zr.zr_summary_prefetch_rule(_geom(head_dim=96), 10, 2)[0] == zr.ZR_E_UNSUPPORTED


def test_noalloc_step_errors(L):
    """Argument checks of zr_sparse_decode_step_noalloc that return before any
    device call: a workspace larger than the built scratch is ZR_E_SCRATCH."""
    g = _geom()
    f = lambda geom, **kw: zr.zr_sparse_decode_step_noalloc(**dict(dict(
        geom=geom, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_table=FAKE, seq_lens=FAKE, th=_th(),
        k=2, window=16, scale=0.1, max_attended=100, scores=FAKE, sel=FAKE, out=FAKE), **kw))
    big = _geom(batch=512, n_q_heads=32, n_kv_heads=8, max_blocks_per_seq=8192)
    assert zr.zr_workspace_bytes(big, 100) > zr.ZR_NOALLOC_SCRATCH_BYTES
    assert f(big) == zr.ZR_E_SCRATCH
    assert f(g, max_attended=-1) == zr.ZR_E_SHAPE
    assert f(_geom(head_dim=96)) == zr.ZR_E_UNSUPPORTED
    assert f(_geom(batch=0)) == zr.ZR_OK  # nothing to do, nothing touched


def test_stage_selected_errors(L):
    g = _geom()
    f = lambda **kw: zr.zr_stage_selected(**dict(dict(
        geom=g, k_pool=FAKE, v_pool=FAKE, block_table=FAKE, seq_lens=FAKE, th=_th(), sel=FAKE,
        k=2, window=16, max_attended=100, workspace=FAKE, ws_bytes=1 << 20, stage_blocks=4,
        k_stage=FAKE, v_stage=FAKE, stage_workspace=FAKE, stage_ws_bytes=1 << 20,
        dropped=FAKE), **kw))
    assert f(stage_blocks=0) == zr.ZR_E_SHAPE
    assert f(stage_blocks=6) == zr.ZR_E_SHAPE   # more than max_blocks_per_seq + 1
    assert f(k=-1) == zr.ZR_E_SHAPE
    assert f(window=-1) == zr.ZR_E_SHAPE
    assert f(sel=None) == zr.ZR_E_NULL
    assert f(dropped=None) == zr.ZR_E_NULL
    assert f(k_stage=None) == zr.ZR_E_NULL
    assert f(v_stage=FAKE + 8) == zr.ZR_E_ALIGN
    assert f(workspace=None) == zr.ZR_E_WORKSPACE
    assert f(stage_workspace=None) == zr.ZR_E_WORKSPACE
    assert f(stage_ws_bytes=16) == zr.ZR_E_WORKSPACE
    assert f(geom=_geom(head_dim=96)) == zr.ZR_E_UNSUPPORTED
    assert f(geom=_geom(batch=0)) == zr.ZR_OK


def test_reuse_errors(L):
    g = _geom()
    f = lambda **kw: zr.zr_reuse_plan(**dict(dict(geom=g, block_table=FAKE, seq_lens=FAKE,
                                                  window=16, horizon=32, max_attended=100,
                                                  workspace=FAKE, ws_bytes=1 << 20), **kw))
    assert f(window=-1) == zr.ZR_E_SHAPE
    assert f(horizon=-1) == zr.ZR_E_SHAPE
    # more than the table can hold: clamped to its capacity, not an error
    assert f(horizon=4 * 16 + 1, geom=_geom(batch=0)) == zr.ZR_OK
    assert f(horizon=2 ** 31 - 1, workspace=None) == zr.ZR_E_WORKSPACE
    assert f(max_attended=-1) == zr.ZR_E_SHAPE
    assert f(block_table=None) == zr.ZR_E_NULL
    assert f(workspace=None) == zr.ZR_E_WORKSPACE
    assert f(geom=_geom(batch=0)) == zr.ZR_OK
    r = lambda **kw: zr.zr_sparse_decode_attn_reuse(**dict(dict(
        geom=g, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_table=FAKE, seq_lens=FAKE, scale=0.1,
        max_attended=100, out=FAKE, workspace=FAKE, ws_bytes=1 << 20), **kw))
    assert r(q=None) == zr.ZR_E_NULL
    assert r(out=FAKE + 4) == zr.ZR_E_ALIGN
    assert r(ws_bytes=16) == zr.ZR_E_WORKSPACE
    assert r(scale=float("inf")) == zr.ZR_E_SHAPE
