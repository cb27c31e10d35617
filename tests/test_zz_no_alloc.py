"""zr_sparse_decode_step_noalloc (the step on the library's built-in device
scratch, for callers that cannot allocate) against zr_sparse_decode_step with
a workspace of its own, through the C ABI: scores, selection and output bit for
bit, on two calls in a row, the second with a smaller batch and shorter
sequences, and an oversized request rejected before anything is enqueued."""
import sys

import numpy as np
import pytest
import torch

from hierarchical_sparse_kv_amd import synth, zr
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


def _check(w, name):
    st = zr.step_from_workload(w)
    need = zr.zr_workspace_bytes(st.geom, st.max_attended)
    say(f"[gpu] no-alloc {name}: B={w.B} T<={int(w.seq_lens.max())} workspace {need} bytes "
        f"(scratch {zr.ZR_NOALLOC_SCRATCH_BYTES})")
    assert 0 < need <= zr.ZR_NOALLOC_SCRATCH_BYTES
    st.step()
    torch.cuda.synchronize()
    ref = (st.scores.clone(), st.sel.clone(), st.out.clone())
    st.scores.fill_(float("nan"))
    st.sel.fill_(-7)
    st.out.fill_(float("nan"))
    st.step_noalloc()
    torch.cuda.synchronize()
    n = w.n_total
    assert torch.equal(st.scores[:n], ref[0][:n]), name
    assert torch.equal(st.sel, ref[1]), name
    assert torch.equal(st.out, ref[2]), name
    return st


def test_noalloc_step_equals_step_twice_then_smaller():
    big = synth.make_workload(1, device="cuda")                 # 16K tokens x batch 8
    _check(big, "16k-b8")
    small = synth.make_workload(1, seed=3, device="cuda",
                                overrides=dict(B=3, seq_len=("uniform", 900, 3000)))
    st = _check(small, "small-b3")
    # the oracle on the smaller call's own output (it came from the scratch path)
    h = P.host(small)
    ref = P.oracle_step(small, h)
    events = P.compare_selection(st.sel.cpu().numpy(), ref["scores"], small.seq_ptr, small.k,
                                 small.Hkv)
    if events:
        ref = P.oracle_step(small, h, sel=st.sel.cpu().numpy())
    err = float(np.max(np.abs(st.out.cpu().numpy() - ref["out"])))
    say(f"[gpu] no-alloc small-b3: max|out - oracle| = {err:.3e}")
    assert err <= P.TOL[small.dtype]


def test_noalloc_step_in_a_graph():
    """The entry point's purpose: capture under a HIP graph. The captured call
    gives on every replay, with other eager work in between, the eager
    result bit for bit (the scratch is rewritten by every replay)."""
    w = synth.make_workload(1, seed=4, device="cuda",
                            overrides=dict(B=4, seq_len=("uniform", 1000, 4000)))
    other = synth.make_workload(3, device="cuda", overrides=dict(B=2, seq_len=("fixed", 1500)))
    st, st2 = zr.step_from_workload(w), zr.step_from_workload(other)
    st.step_noalloc()
    torch.cuda.synchronize()
    ref = (st.scores.clone(), st.sel.clone(), st.out.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            st.step_noalloc()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        st.out.fill_(float("nan"))
        st.sel.fill_(-7)
        st2.step()              # eager work between replays (its own workspace)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.sel, ref[1]), rep
        assert torch.equal(st.out, ref[2]), rep


def test_noalloc_rejects_requests_beyond_the_scratch():
    """A geometry whose workspace exceeds the scratch: ZR_E_SCRATCH, and the
    outputs are untouched."""
    w = synth.make_workload(1, device="cuda", overrides=dict(B=2, seq_len=("fixed", 2048)))
    st = zr.step_from_workload(w)
    st.out.fill_(7.0)
    big = zr.zr_geom(512, 32, 8, 128, 16, 8192, w.num_blocks, zr.ZR_BF16)
    s = zr.zr_sparse_decode_step_noalloc(big, zr._ptr(st.q), st.kp, st.vp,
                                         zr._ptr(st.block_table), zr._ptr(st.seq_lens), st.th,
                                         st.k, st.window, st.scale, st.max_attended,
                                         zr._ptr(st.scores), zr._ptr(st.sel), zr._ptr(st.out))
    torch.cuda.synchronize()
    assert s == zr.ZR_E_SCRATCH
    assert torch.all(st.out == 7.0)
