"""GPU: the fused decode step captured in a HIP graph replays to the eager result.

The benchmark times graph replays, so every replay has to compute what an eager call
computes.  Each case runs one eager step for the reference, captures one step, then
replays the graph five times.  Before each replay the outputs are poisoned and the
program does eager work of its own (a library call on another tensor and an eager step
of the same layer), with synchronisations in between.  Every replay must match the eager
outputs bit for bit: the step is deterministic, and a node that only works on the first
replay (a memset recorded into the graph, scratch left from the previous call) would
show here.
"""
import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

# eight sequences whose three local heads need 512-row window blocks (the heavy-window
# kernel), with full, partial and single-row windows
HEAVY_WINDOW_LENS = [9000, 1, 700, 5000, 8196, 8197, 20000, 8200]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def rtp():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import head_wise_sparse_rtp_amd as m
    m.lib()
    return m


def _outputs(st):
    """The step's outputs; of the exported sets, only the first sel_count entries of a row
    are written (the rest keep what they held), so the rest are masked to -1."""
    ts = [st.out, st.lse, st.thresh, st.count]
    if st.sel_idx is not None:
        cap = st.sel_idx.shape[-1]
        n = st.sel_count.clamp(min=0, max=cap).unsqueeze(-1)
        pos = torch.arange(cap, device=st.sel_idx.device)
        ts += [torch.where(pos < n, st.sel_idx, torch.full_like(st.sel_idx, -1)), st.sel_count]
    return [t for t in ts if t is not None]


def _poison(st, ret_q):
    # out and lse cover every query head; the threshold, count and set outputs cover the
    # retrieval query heads only, so only their rows are poisoned
    st.out.fill_(float("nan"))
    st.lse.fill_(float("nan"))
    for t in (st.thresh, st.count, st.sel_idx, st.sel_count):
        if t is not None:
            t[:, ret_q] = -7


def _ret_q(wl, layer):
    return [kh * wl.G + g for kh in layer.ret_heads for g in range(wl.G)]


def _case(name):
    dev = torch.device("cuda:0")
    if name == "ragged":
        wl = workloads.make_workload("t", 2, [20000, 9000], 32, 4, [[1, 0, 0, 1]], seed=81,
                                     p=0.9, dtype="f16", device=dev)
        return wl, None, 0
    if name == "heavy":
        wl = workloads.make_workload("t", 8, HEAVY_WINDOW_LENS, 32, 4, [[1, 0, 0, 0]], seed=82,
                                     p=0.9, dtype="f16", window=8192, sinks=4, device=dev)
        return wl, None, 0
    # the cache update fused into stage A, with the attended sets exported
    wl = workloads.make_workload("t", 2, [20000, 9000], 32, 4, [[1, 0, 0, 1]], seed=83, p=0.9,
                                 dtype="f16", device=dev)
    return wl, workloads.make_embedding_step_inputs(wl, device=dev), wl.Lmax


@pytest.mark.parametrize("name", ["ragged", "heavy", "append_sets"])
def test_decode_step_graph_replays_match_eager(rtp, name):
    say("graph replay", name)
    wl, app, want_sets = _case(name)
    layer = wl.layers[0]
    sl = torch.as_tensor(wl.seq_lens, dtype=torch.int32, device="cuda:0")
    st = rtp.DecodeStep(layer, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks, wl.p,
                        wl.bin_width, wl.scale_idx, wl.scale_attn, want_debug=True,
                        want_sets=want_sets, append=app)
    st()
    torch.cuda.synchronize()
    ref = [t.clone() for t in _outputs(st)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st()  # warm the capture stream once, as graph capture expects
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st()
    torch.cuda.synchronize()

    other = torch.randn(512, 512, device="cuda:0")
    ret_q = _ret_q(wl, layer)
    for rep in range(5):
        _poison(st, ret_q)
        other = torch.tanh(other @ other.t() * 1e-3)  # unrelated eager library work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(st), ref)):
            assert torch.equal(a, b), "%s: replay %d, output %d differs from eager" % (name, rep, i)
        st()  # an eager step of the same layer between replays
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(st), ref)):
            assert torch.equal(a, b), "%s: eager step after replay %d, output %d" % (name, rep, i)


def test_decode_step_noalloc_graph_replays_match_eager(rtp):
    """The no-allocation entry point (fixed library scratch) captured in a graph: every
    replay, and every eager no-allocation call between replays, matches the eager step on
    a caller workspace bit for bit."""
    say("graph replay, no-allocation entry point")
    wl, _, _ = _case("ragged")
    layer = wl.layers[0]
    sl = torch.as_tensor(wl.seq_lens, dtype=torch.int32, device="cuda:0")
    st = rtp.DecodeStep(layer, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks, wl.p,
                        wl.bin_width, wl.scale_idx, wl.scale_attn, want_debug=True)
    st()
    torch.cuda.synchronize()
    ref = [t.clone() for t in _outputs(st)]
    ret_q = _ret_q(wl, layer)
    _poison(st, ret_q)
    st.noalloc()  # resolves the scratch on this device outside the capture
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(_outputs(st), ref)):
        assert torch.equal(a, b), "eager no-allocation call, output %d" % i
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.noalloc()
    torch.cuda.synchronize()
    for rep in range(5):
        _poison(st, ret_q)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(st), ref)):
            assert torch.equal(a, b), "replay %d, output %d differs from eager" % (rep, i)
        _poison(st, ret_q)
        st.noalloc()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(st), ref)):
            assert torch.equal(a, b), "eager no-allocation call after replay %d, output %d" % (rep, i)
