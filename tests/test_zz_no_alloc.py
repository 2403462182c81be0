"""rtp_decode_step_noalloc: the decode step on the library's fixed scratch array, for
callers that cannot allocate.  Its outputs (out, lse, A and b*, set sizes, exported sets)
must equal rtp_decode_step's on a caller workspace bit for bit -- the same kernels -- on
two calls in a row, the second with a smaller input (the scratch keeps the first call's
contents), and on the single-purpose kernels' path."""
import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def rtp():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import head_wise_sparse_rtp_amd as m
    m.lib()
    return m


def _same_as_workspace_call(rtp, wl, label):
    dev = torch.device("cuda:0")
    layer = wl.layers[0]
    sl = torch.as_tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    st = rtp.DecodeStep(layer, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks, wl.p,
                        wl.bin_width, wl.scale_idx, wl.scale_attn, want_debug=True,
                        want_sets=wl.Lmax, topk=wl.topk, ret_window=wl.ret_window)
    outs = [st.out, st.lse, st.thresh, st.count, st.sel_idx, st.sel_count]
    st()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    # overwrite every output, so that each value compared below was written by the call
    for t in outs:
        t.fill_(float("nan") if t.is_floating_point() else -7)
    st.noalloc()
    torch.cuda.synchronize()
    # out and lse cover every query head; A and b*, the counts and the sets are written for
    # the retrieval query heads only (other rows are left as they are), and each set row up
    # to its size
    ret_q = [kh * wl.G + g for kh in layer.ret_heads for g in range(wl.G)]
    for i, (name, a, b) in enumerate(zip(["out", "lse", "thresh", "count"], ref, outs)):
        if i >= 2:
            a, b = a[:, ret_q], b[:, ret_q]
        assert torch.equal(a, b), "%s: %s differs from the workspace call" % (label, name)
    assert torch.equal(ref[5][:, ret_q], outs[5][:, ret_q]), "%s: sel_count differs" % label
    cnt = ref[5].cpu()
    for b_ in range(wl.B):
        for h in ret_q:
            n = min(int(cnt[b_, h]), wl.Lmax)
            assert torch.equal(ref[4][b_, h, :n], outs[4][b_, h, :n]), \
                "%s: the set of b %d head %d differs" % (label, b_, h)
    say(label, "bit-exact; ws %.1f MiB" % (st.ws_bytes / 2 ** 20))


def test_noalloc_matches_workspace_call_twice(rtp):
    """First the 1M-token layer (fused path, 14 MiB of scratch, exported sets 4 MiB more),
    then a small ragged batch on the same scratch."""
    say("noalloc c4 then small")
    _same_as_workspace_call(rtp, workloads.make_config("c4", device=torch.device("cuda:0")), "c4")
    wl = workloads.make_workload("t", 3, [3000, 1, 4099], 32, 4, [[1, 0, 1, 0]], seed=61,
                                 p=0.9, dtype="f16", window=256, sinks=4,
                                 device=torch.device("cuda:0"))
    _same_as_workspace_call(rtp, wl, "small-f16")


def test_noalloc_single_purpose_path(rtp):
    """fp32 caches run the single-purpose kernels on the same scratch."""
    say("noalloc f32")
    wl = workloads.make_workload("t", 2, [5000, 700], 16, 2, [[1, 0]], seed=62, p=0.9,
                                 dtype="f32", window=512, sinks=4, device=torch.device("cuda:0"))
    _same_as_workspace_call(rtp, wl, "small-f32")
