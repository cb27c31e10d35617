"""The decode step captured in a HIP graph gives, on every replay, exactly the
eager result (the benchmark times graph replays)."""
import pytest
import torch

from hierarchical_sparse_kv_amd import synth, zr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zr.lib()


@pytest.mark.parametrize("fused,dtype", [(True, "bf16"), (False, "bf16"), (True, "f32")])
def test_graph_replays_match_eager(fused, dtype):
    w = synth.make_workload(1, device="cuda", overrides=dict(B=4, seq_len=("fixed", 4096),
                                                             dtype=dtype))
    other = synth.make_workload(3, device="cuda",
                                overrides=dict(B=3, seq_len=("uniform", 500, 3000)))
    st, st2 = zr.step_from_workload(w), zr.step_from_workload(other)
    run = st.step if fused else st.step_calls
    run()
    torch.cuda.synchronize()
    ref = (st.scores.clone(), st.sel.clone(), st.out.clone())
    st.dense_attn(out=torch.empty_like(st.out))

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        st.out.fill_(float("nan"))
        st.sel.fill_(-7)
        st2.step()              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.scores, ref[0]), rep
        assert torch.equal(st.sel, ref[1]), rep
        assert torch.equal(st.out, ref[2]), rep



def test_graph_replays_of_cached_and_zoom_calls():
    """Cached-selection and multi-granularity attention captured in one graph:
    every replay equals the eager result."""
    import numpy as np
    w = synth.make_workload(5, device="cuda", overrides=dict(B=2, seq_len=("fixed", 3000)))
    st = zr.step_from_workload(w)
    ss = torch.as_tensor(w.extra["sum_start"], device="cuda")
    sl = torch.as_tensor(w.extra["sum_len"], device="cuda")
    st.coarse_score()
    st.select_topk()
    c = w.extra["c"]
    votes = torch.empty(w.n_total, dtype=torch.int32, device="cuda")
    cons = torch.empty((w.B, c), dtype=torch.int32, device="cuda")
    agree = torch.empty(w.B, dtype=torch.float32, device="cuda")
    outz = torch.empty_like(st.out)
    outc = torch.empty_like(st.out)

    def work():
        st.consensus(st.sel[None], c, votes, cons, agree)
        st.zoom_attn(ss, sl, votes, cons, c, w.extra["prompt"], out=outz)
        st.cached_attn(w.window + 3, out=outc)

    work()
    torch.cuda.synchronize()
    ref = (votes.clone(), cons.clone(), agree.clone(), outz.clone(), outc.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (votes, cons, outz, outc):
            t.fill_(-3)
        st.step()                # eager work between replays, same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((votes, cons, agree, outz, outc), ref):
            assert torch.equal(a, b), rep


def test_graph_replays_of_staging_from_host_pools():
    """zr_stage_selected and the attention on the staging pool, captured in a
    graph (as the bench runs them): every replay, with other eager work in
    between, gives the eager output bit for bit."""
    w = synth.make_workload(1, device="cuda", overrides=dict(B=3, seq_len=("uniform", 800, 3000)))
    other = synth.make_workload(3, device="cuda", overrides=dict(B=2, seq_len=("fixed", 1500)))
    st, st2 = zr.step_from_workload(w), zr.step_from_workload(other)
    st.step()
    torch.cuda.synchronize()
    kp, vp = w.k_pool.cpu().pin_memory(), w.v_pool.cpu().pin_memory()
    hs = zr.DeviceStep(w.q, kp, vp, w.block_table, w.seq_lens, w.seq_ptr, w.th_start, w.th_len,
                       w.summary_keys, w.max_per_seq, w.k, w.window, w.scale, st.max_attended)
    sg = zr.Staging(hs, w.max_blocks + 1)
    sel = st.sel.clone()

    def run():
        hs.stage(sg, sel=sel)
        hs.attend_staged(sg)

    run()
    torch.cuda.synchronize()
    ref = hs.out.clone()
    assert torch.equal(ref, st.out)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        hs.out.fill_(float("nan"))
        sg.k_stage.zero_()
        st2.step()              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(hs.out, ref), rep
        assert int(sg.dropped.sum().item()) == 0
