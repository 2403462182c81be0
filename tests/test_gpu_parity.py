"""GPU parity: every entry point of librtp.so against the CPU oracle.

Small ragged cases span several chunks/tiles and ragged tails; the full-size
configurations run in the launch configuration the benchmark times.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import (SelCheck, compare_count, compare_sets, expected_set, max_err,
                               out_tol)

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


def dev():
    return torch.device("cuda:0")


# ---------------------------------------------------------------------------
# rtp_index_score
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,G,lens", [("f16", 8, [5000, 1, 2049]), ("f32", 1, [4097]),
                                          ("f16", 3, [700, 3]), ("f32", 4, [2048, 2047]),
                                          ("bf16", 8, [5000, 1, 2049])])
def test_index_score_bit_exact(rtp, dtype, G, lens):
    say("index_score", dtype, G, lens)
    Hkv = 2
    wl = workloads.make_workload("t", len(lens), lens, G * Hkv, Hkv, [[1, 1]], seed=21,
                                 dtype=dtype, device=dev(), classes=lambda b, k, r: ["gaussian"] * G)
    lay = wl.layers[0]
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    z = torch.full((len(lens), 2 * G, wl.Lmax), 123.0, dtype=torch.float32, device=dev())
    rtp.rtp_index_score(lay.q_idx, lay.k_idx, sl, wl.scale_idx, z)
    zc = z.cpu().numpy()
    qi = oracle.np_of(lay.q_idx)
    for b, L in enumerate(lens):
        for h in range(2 * G):
            zo = oracle.index_score(qi[b, h], oracle.np_of(lay.k_idx[b, h // G, :L]), wl.scale_idx)
            assert np.array_equal(zc[b, h, :L], zo), (b, h)
            assert np.all(zc[b, h, L:] == 123.0)


# ---------------------------------------------------------------------------
# rtp_topp_select
# ---------------------------------------------------------------------------
def _logit_rows(seed, Lmax, lens):
    rng = np.random.default_rng(seed)
    rows = []
    kinds = ["gauss1", "gauss4", "spike", "broad", "edges", "allequal", "wide", "flat"]
    for i, L in enumerate(lens):
        k = kinds[i % len(kinds)]
        z = np.zeros(Lmax, dtype=np.float32)
        if k == "gauss1":
            v = rng.standard_normal(L)
        elif k == "gauss4":
            v = 4 * rng.standard_normal(L)
        elif k == "spike":
            v = rng.standard_normal(L)
            v[rng.choice(L, min(3, L), replace=False)] = 12.0
        elif k == "broad":
            v = rng.standard_normal(L) - 6
            v[rng.choice(L, max(1, L // 10), replace=False)] = 2 + 0.7 * rng.standard_normal(max(1, L // 10))
        elif k == "edges":
            v = rng.integers(-100, 50, L) * 0.125
        elif k == "allequal":
            v = np.full(L, -3.3)
        elif k == "wide":
            v = 25 * rng.standard_normal(L)
        else:
            v = 0.01 * rng.standard_normal(L)
        z[:L] = v.astype(np.float32)
        z[L:] = 1e6  # must never be read
        rows.append(z)
    return np.stack(rows)


@pytest.mark.parametrize("p", [0.5, 0.9, 0.95, 1.0])
@pytest.mark.parametrize("lens", [[9000, 1, 2, 4097, 2048, 12345, 3, 777], [70000, 70000]])
def test_topp_select_matches_oracle(rtp, p, lens):
    say("topp_select", p, lens)
    Lmax = max(lens)
    B, H = 1, len(lens)
    zr = _logit_rows(31 + len(lens), Lmax, lens)
    z = torch.from_numpy(zr).view(B, H, Lmax).to(dev())
    # each row is its own "sequence": use B = rows, H = 1 so seq_lens differ per row
    z = z.view(H, 1, Lmax).contiguous()
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    sel_idx, cnt, hist, thr = rtp.rtp_topp_select(z, sl, p)
    sel_idx, cnt, hist, thr = (t.cpu().numpy() for t in (sel_idx, cnt, hist, thr))
    st = SelCheck()
    for i, L in enumerate(lens):
        so = oracle.topp_select(zr[i, :L], p)
        where = "row %d L=%d p=%g" % (i, L, p)
        ex = expected_set(zr[i, :L], so, int(thr[i, 0, 0]), int(thr[i, 0, 1]), p, 0.125, st, where)
        n = int(cnt[i, 0])
        compare_sets(sel_idx[i, 0, :n], ex, zr[i, :L], 0.125, st, where)
        assert np.all(np.diff(sel_idx[i, 0, :n]) > 0)
        Z = so.hist.sum()
        assert np.max(np.abs(hist[i, 0] - so.hist)) <= 2e-6 * Z, where
    say("mass ties", st.mass_ties, "edge tokens", st.edge_tokens)


@pytest.mark.parametrize("p", [0.5, 0.9, 0.999])
def test_topp_select_smallest_bin_width(rtp, p):
    """w = 2^-10, the smallest accepted width: 256 bins then span a quarter of a nat, so
    chunks far below the top cell in cells still weigh in (one token at 0 and 8191 at -4.5
    put almost all the mass in the tail bin: b* = 255)."""
    w = 2.0 ** -10
    say("topp_select w=2^-10", p)
    rows = []
    z = np.full(8192, -4.5, dtype=np.float32)
    z[3000] = 0.0
    rows.append(z)
    rng = np.random.default_rng(17)
    rows.append((0.3 * rng.standard_normal(8192)).astype(np.float32))
    z = (rng.standard_normal(8192) - 3).astype(np.float32)
    z[rng.choice(8192, 40, replace=False)] = 0.1 * rng.standard_normal(40).astype(np.float32)
    rows.append(z)
    zr = np.stack(rows)
    H, Lmax = zr.shape
    zt = torch.from_numpy(zr).view(H, 1, Lmax).to(dev())
    sl = torch.tensor([Lmax] * H, dtype=torch.int32, device=dev())
    sel_idx, cnt, hist, thr = rtp.rtp_topp_select(zt, sl, p, bin_width=w)
    sel_idx, cnt, hist, thr = (t.cpu().numpy() for t in (sel_idx, cnt, hist, thr))
    st = SelCheck()
    for i in range(H):
        so = oracle.topp_select(zr[i], p, bin_width=w)
        where = "row %d p=%g w=2^-10" % (i, p)
        ex = expected_set(zr[i], so, int(thr[i, 0, 0]), int(thr[i, 0, 1]), p, w, st, where)
        n = int(cnt[i, 0])
        compare_sets(sel_idx[i, 0, :n], ex, zr[i], w, st, where)
        Z = so.hist.sum()
        assert np.max(np.abs(hist[i, 0] - so.hist)) <= 2e-6 * Z, where
    # the first row is the case a fixed cutoff of 4096 cells would get wrong
    assert oracle.topp_select(zr[0], 0.9, bin_width=w).bstar == 255


@pytest.mark.parametrize("p", [0.5, 0.9])
def test_decode_step_smallest_bin_width(rtp, p):
    """The fused step (f16) and the single-purpose kernels (f32) at w = 2^-10, with
    sequences long enough that chunk top cells lie thousands of cells below the head's."""
    say("decode_step w=2^-10", p)
    for dtype in ("f16", "f32"):
        wl = workloads.make_workload("t", 2, [20000, 5000], 32, 4, [[1, 0, 1, 0]], seed=67, p=p,
                                     dtype=dtype, window=256, sinks=4, device=dev(),
                                     bin_width=2.0 ** -10)
        check_decode(rtp, wl, label="w2^-10-%s-p%g" % (dtype, p))


@pytest.mark.parametrize("k", [1, 3, 100, 4096, 100000])
@pytest.mark.parametrize("lens", [[9000, 1, 2, 4097, 2048, 12345, 3, 777], [70000, 70000]])
def test_topk_select_bit_exact(rtp, k, lens):
    """Fixed top-k through the histogram: cells come from the same z on both sides and
    the counts are exact, so A, b*, the counts and the set must match exactly."""
    say("topk_select", k, lens)
    Lmax = max(lens)
    H = len(lens)
    zr = _logit_rows(71 + len(lens), Lmax, lens)
    z = torch.from_numpy(zr).view(H, 1, Lmax).to(dev())
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    sel_idx, cnt, hist, thr = rtp.rtp_topk_select(z, sl, k)
    sel_idx, cnt, hist, thr = (t.cpu().numpy() for t in (sel_idx, cnt, hist, thr))
    for i, L in enumerate(lens):
        so = oracle.topk_select(zr[i, :L], k)
        where = "row %d L=%d k=%d" % (i, L, k)
        assert int(thr[i, 0, 0]) == so.A and int(thr[i, 0, 1]) == so.bstar, where
        assert np.array_equal(hist[i, 0].astype(np.float64), so.hist), where
        n = int(cnt[i, 0])
        assert np.array_equal(sel_idx[i, 0, :n], so.idx), where


def test_topk_select_empty_and_capped(rtp):
    say("topk_select empty/capped")
    zr = _logit_rows(6, 5000, [1, 5000])
    z = torch.from_numpy(zr).view(2, 1, 5000).to(dev())
    sl = torch.tensor([0, 5000], dtype=torch.int32, device=dev())
    so = oracle.topk_select(zr[1], 1000)
    sel_idx, cnt, hist, thr = rtp.rtp_topk_select(z, sl, 1000, cap=100)
    cnt = cnt.cpu().numpy()
    assert cnt[0, 0] == 0 and cnt[1, 0] == so.count
    assert np.array_equal(sel_idx.cpu().numpy()[1, 0], so.idx[:100])
    assert np.all(hist.cpu().numpy()[0] == 0)


def test_topp_select_empty_and_capped(rtp):
    say("topp_select empty/capped")
    lens = [0, 5000]
    zr = _logit_rows(5, 5000, [1, 5000])
    z = torch.from_numpy(zr).view(2, 1, 5000).to(dev())
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    so = oracle.topp_select(zr[1], 1.0)
    sel_idx, cnt, hist, thr = rtp.rtp_topp_select(z, sl, 1.0, cap=100)
    cnt = cnt.cpu().numpy()
    assert cnt[0, 0] == 0 and cnt[1, 0] == 5000
    assert np.array_equal(sel_idx.cpu().numpy()[1, 0], np.arange(100))
    assert np.all(hist.cpu().numpy()[0] == 0)
    assert so.count == 5000


# ---------------------------------------------------------------------------
# rtp_sparse_decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f16", "f32", "bf16"])
def test_sparse_decode_matches_oracle(rtp, dtype):
    say("sparse_decode", dtype)
    lens = [6000, 300]
    G, Hr = 4, 2
    wl = workloads.make_workload("t", 2, lens, G * Hr, Hr, [[1, 1]], seed=41, dtype=dtype,
                                 device=dev())
    lay = wl.layers[0]
    rng = np.random.default_rng(3)
    cap = 6000
    sel = np.full((2, G * Hr, cap), -1, dtype=np.int32)
    cnt = np.zeros((2, G * Hr), dtype=np.int32)
    sets = {}
    sizes = [0, 1, 2, 63, 64, 65, 1000, 6000]
    for b in range(2):
        for h in range(G * Hr):
            n = min(sizes[(h + b) % len(sizes)], lens[b])
            s = np.sort(rng.choice(lens[b], n, replace=False)).astype(np.int32)
            sel[b, h, :n] = s
            cnt[b, h] = n
            sets[(b, h)] = s
    out, lse = rtp.rtp_sparse_decode(lay.q, lay.K_ret, lay.V_ret, torch.from_numpy(sel).to(dev()),
                                     torch.from_numpy(cnt).to(dev()), wl.scale_attn)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qn = oracle.np_of(lay.q)
    for b in range(2):
        for h in range(G * Hr):
            s = sets[(b, h)]
            if len(s) == 0:
                assert np.all(out[b, h] == 0) and lse[b, h] == -np.inf
                continue
            o, l = oracle.attention(qn[b, h], oracle.np_of(lay.K_ret[b, h // G]),
                                    oracle.np_of(lay.V_ret[b, h // G]), s, wl.scale_attn)
            assert max_err(out[b, h], o) <= out_tol(dtype), (b, h, len(s))
            assert abs(lse[b, h] - l) <= 1e-4 * max(1, abs(l))


# ---------------------------------------------------------------------------
# rtp_window_decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,window,sinks,lens", [
    ("f16", 64, 4, [1, 3, 4, 5, 67, 68, 69, 500]),
    ("f32", 64, 4, [2, 68, 1000]),
    ("f16", 100, 0, [50, 100, 101, 333]),
    ("f16", 8192, 4, [8196, 9000, 4000]),
    ("bf16", 64, 4, [1, 3, 4, 5, 67, 68, 69, 500]),
])
def test_window_decode_matches_oracle(rtp, dtype, window, sinks, lens):
    say("window_decode", dtype, window, sinks, lens)
    G, Hl = 8, 2
    wl = workloads.make_workload("t", len(lens), lens, G * Hl, Hl, [[0, 0]], seed=51, dtype=dtype,
                                 window=window, sinks=sinks, device=dev())
    lay = wl.layers[0]
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    out, lse = rtp.rtp_window_decode(lay.q, lay.K_loc, lay.V_loc, sl, window, sinks, wl.scale_attn)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qn = oracle.np_of(lay.q)
    for b, L in enumerate(lens):
        rows = oracle.ring_slot(oracle.window_positions(L, window, sinks), window, sinks)
        for h in range(G * Hl):
            o, l = oracle.attention(qn[b, h], oracle.np_of(lay.K_loc[b, h // G]),
                                    oracle.np_of(lay.V_loc[b, h // G]), rows, wl.scale_attn)
            assert max_err(out[b, h], o) <= out_tol(dtype), (b, h, L)
            assert abs(lse[b, h] - l) <= 1e-4 * max(1, abs(l))


# ---------------------------------------------------------------------------
# rtp_decode_step
# ---------------------------------------------------------------------------
# Beside the 2e-3 / 1e-5 bar of the outputs, the measured error of a correct step is far
# smaller (about 1e-7 with fp16 K/V): one token wrongly kept or dropped in a set of a few
# thousand moves an output by about 1e-4, so the tighter diagnostic bound below catches
# it even where the exported sets could not.
DIAG_TOL = {"f16": 1e-4, "bf16": 1e-4, "f32": 1e-5}


def check_decode(rtp, wl, local_sample=None, layers=None, label="", oracle_layers=None,
                 sets=True, appends=None):
    """Run every layer on the GPU and compare with the oracle (all retrieval heads; all
    local heads or the first `local_sample` of each layer).  `oracle_layers`, when given,
    are the oracle's own copies of the layers (after its own cache update).  With `sets`
    the step also exports the token set each retrieval query head attended to, and every
    set is compared with the oracle's element by element (up to edge-band tokens)."""
    res = rtp.decode_workload(wl, want_debug=True, want_sets=wl.Lmax if sets else 0,
                              appends=appends)
    torch.cuda.synchronize()
    st = SelCheck()
    tol = out_tol(wl.dtype)
    worst = 0.0
    nsets = 0
    for li, layer in enumerate(wl.layers):
        if layers is not None and li not in layers:
            continue
        if len(wl.layers) > 2:
            say(label, "layer", li)
        if oracle_layers is not None:
            layer = oracle_layers[li]
        out, lse, thr, cnt = (t.cpu().numpy() for t in res[li][:4])
        ret_q = [kh * wl.G + g for kh in layer.ret_heads for g in range(wl.G)]
        sidx = scnt = None
        if sets and ret_q:
            sidx = res[li][4][:, ret_q].cpu().numpy()   # retrieval rows only
            scnt = res[li][5].cpu().numpy()
        heads = None
        if local_sample is not None:
            loc_q = [kh * wl.G + g for kh in layer.loc_heads for g in range(wl.G)][:local_sample]
            heads = ret_q + loc_q
        orc = oracle.decode_layer(layer, wl.seq_lens, wl.Hq, wl.Hkv, wl.p, wl.bin_width,
                                  wl.scale_idx, wl.scale_attn, wl.window, wl.sinks, heads=heads,
                                  topk=wl.topk, ret_window=wl.ret_window)
        for (b, h), r in orc.items():
            where = "%s layer %d b %d head %d" % (label, li, b, h)
            o_ref = r.out
            if r.sel is not None:
                A, bs = int(thr[b, h, 0]), int(thr[b, h, 1])
                ex = expected_set(r.z, r.sel, A, bs, wl.p, wl.bin_width, st, where, wl.topk)
                same = ex is r.sel.idx
                if wl.ret_window:
                    win = oracle.window_positions(int(wl.seq_lens[b]), wl.window, wl.sinks)
                    ex = np.union1d(ex, win).astype(np.int64)
                compare_count(int(cnt[b, h]), ex, r.z, wl.bin_width, A, bs, st, where)
                if sidx is not None:
                    n = int(scnt[b, h])
                    assert n == int(cnt[b, h]), "%s: exported %d tokens, counted %d" % (
                        where, n, int(cnt[b, h]))
                    got = sidx[b, ret_q.index(h), :n]
                    assert np.all(np.diff(got) > 0), "%s: exported set not ascending" % where
                    compare_sets(got, ex, r.z, wl.bin_width, st, where)
                    nsets += 1
                    if not np.array_equal(got, ex):
                        # edge-band tokens differ (allowed): the arithmetic is compared on the
                        # set the step attended to
                        ex, same = got, False
                if not same:
                    kr = layer.ret_heads.index(h // wl.G)
                    o_ref, _ = oracle.attention(oracle.np_of(layer.q)[b, h],
                                                oracle.np_of(layer.K_ret[b, kr]),
                                                oracle.np_of(layer.V_ret[b, kr]), ex, wl.scale_attn)
            e = max_err(out[b, h], o_ref)
            worst = max(worst, e)
            assert e <= tol, "%s: max |dO| = %g > %g" % (where, e, tol)
            assert abs(lse[b, h] - r.lse) <= 1e-3 * max(1.0, abs(r.lse)), where
    say(label, "rows", st.rows, "sets compared", nsets, "mass ties", st.mass_ties,
        "edge tokens", st.edge_tokens, "worst |dO|", worst)
    assert worst <= DIAG_TOL[wl.dtype], "%s: worst |dO| = %g above the diagnostic bound %g" % (
        label, worst, DIAG_TOL[wl.dtype])
    return res


@pytest.mark.parametrize("dtype", ["f16", "f32", "bf16"])
@pytest.mark.parametrize("p", [0.5, 0.9, 1.0])
def test_decode_step_small_ragged(rtp, dtype, p):
    say("decode_step small", dtype, p)
    wl = workloads.make_workload("t", 3, [3000, 1, 4099], 32, 4, [[1, 0, 1, 0]], seed=61, p=p,
                                 dtype=dtype, window=256, sinks=4, device=dev())
    check_decode(rtp, wl, label="small-%s-p%g" % (dtype, p))


@pytest.mark.parametrize("G", [1, 2, 3, 5, 16, 20])
def test_decode_step_heads_per_kv(rtp, G):
    """Query heads per KV head: the fused path takes G <= 16 (one or two 8-head groups in
    the histogram kernel, 8- or 16-column selection tiles); G = 20 runs the single-purpose
    kernels."""
    say("decode_step G", G)
    wl = workloads.make_workload("t", 3, [5000, 1, 2300], 3 * G, 3, [[1, 0, 1]], seed=70 + G,
                                 p=0.9, dtype="f16", window=384, sinks=4, device=dev())
    check_decode(rtp, wl, label="G%d" % G)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("k", [1, 64, 3000, 5000])
def test_decode_step_topk_small_ragged(rtp, dtype, k):
    """Fixed top-k on the fused path (f16) and on the single-purpose kernels (f32); k =
    5000 exceeds every sequence, so every token is kept."""
    say("decode_step topk small", dtype, k)
    wl = workloads.make_workload("t", 3, [3000, 1, 4099], 32, 4, [[1, 0, 1, 0]], seed=65,
                                 dtype=dtype, window=256, sinks=4, device=dev())
    wl.topk = k
    res = check_decode(rtp, wl, label="topk-%s-k%d" % (dtype, k))
    cnt = res[0][3].cpu().numpy()
    for b, L in enumerate([3000, 1, 4099]):
        for h in list(range(8)) + list(range(16, 24)):
            assert cnt[b, h] >= min(k, L)
            if k >= L:
                assert cnt[b, h] == L


@pytest.mark.parametrize("name,k", [("c1", 2048), ("c4", 2048), ("c4", 16384)])
def test_decode_step_topk_config(rtp, name, k):
    say("config", name, "topk", k)
    wl = workloads.make_config(name, device=dev())
    wl.topk = k
    check_decode(rtp, wl, label="%s-topk%d" % (name, k))


# ---------------------------------------------------------------------------
# rtp_append_project: the step's cache update
# ---------------------------------------------------------------------------
def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a.view(np.uint32)


def _oracle_layer(lay, arrays):
    q_idx, k_idx, K_ret, V_ret, K_loc, V_loc = (torch.from_numpy(a) for a in arrays)
    return workloads.Layer(lay.kv_is_retrieval, lay.q.cpu(), q_idx, k_idx, K_ret, V_ret, K_loc,
                           V_loc)


@pytest.mark.parametrize("dtype", ["f16", "f32", "bf16"])
def test_append_project_bit_exact(rtp, dtype):
    """Projections are fp32 fma chains in input order on both sides and the rows are
    copies: every cache array must match bit for bit (ring wrap, a sink position, an
    empty sequence, L = 1)."""
    lens = [1, 5000, 0, 70, 3]
    say("append_project", dtype, lens)
    wl = workloads.make_workload("t", len(lens), lens, 32, 4, [[1, 0, 1, 0]], seed=81,
                                 dtype=dtype, window=64, sinks=4, device=dev(), Lmax=5000)
    lay = wl.layers[0]
    si = workloads.make_step_inputs(wl, seed=1, device=dev())
    want = oracle.append_project(lay, lens, si.q_pre, si.k_pre, si.k_new, si.v_new, si.Wq, si.Wk,
                                 wl.window, wl.sinks)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    rtp.rtp_append_project(lay, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks, si.q_pre,
                           si.k_pre, si.Wq, si.Wk, si.k_new, si.v_new)
    got = [oracle.np_of(t) for t in (lay.q_idx, lay.k_idx, lay.K_ret, lay.V_ret, lay.K_loc,
                                     lay.V_loc)]
    for name, g, w in zip(["q_idx", "k_idx", "K_ret", "V_ret", "K_loc", "V_loc"], got, want):
        assert np.array_equal(_bits(g), _bits(w)), name


def test_append_then_decode_c1(rtp):
    """A whole step at 64K context: the new token's cache update, then the layer step that
    attends over it; the oracle runs its own update and its own decode."""
    say("append + decode c1")
    wl = workloads.make_config("c1", device=dev())
    lay = wl.layers[0]
    si = workloads.make_step_inputs(wl, seed=2, device=dev())
    want = oracle.append_project(lay, wl.seq_lens, si.q_pre, si.k_pre, si.k_new, si.v_new, si.Wq,
                                 si.Wk, wl.window, wl.sinks)
    olay = _oracle_layer(lay, want)
    sl = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev())
    rtp.rtp_append_project(lay, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks, si.q_pre,
                           si.k_pre, si.Wq, si.Wk, si.k_new, si.v_new)
    assert np.array_equal(_bits(oracle.np_of(lay.k_idx)), _bits(want[1]))
    check_decode(rtp, wl, label="append-c1", oracle_layers=[olay])


def _check_caches(lay, want, label):
    got = [oracle.np_of(t) for t in (lay.q_idx, lay.k_idx, lay.K_ret, lay.V_ret, lay.K_loc,
                                     lay.V_loc)]
    for name, g, w in zip(["q_idx", "k_idx", "K_ret", "V_ret", "K_loc", "V_loc"], got, want):
        assert np.array_equal(_bits(g), _bits(w)), "%s: %s" % (label, name)


@pytest.mark.parametrize("dtype,mask,ret_window", [
    ("f16", [1, 0, 1, 0], False), ("bf16", [1, 0, 1, 0], False), ("f16", [1, 0, 1, 0], True),
    ("f32", [1, 0, 1, 0], False), ("f16", [0, 0, 0, 0], False), ("f16", [1, 1, 1, 1], False)])
def test_decode_step_fused_append_small_ragged(rtp, dtype, mask, ret_window):
    """The cache update fused into the step: stage A projects the group's q_idx and the new
    token's indexer key and copies the new K/V rows (the standalone update kernel runs first
    on the single-purpose path, fp32, and for layers without retrieval heads).  Every cache
    must equal the oracle's update bit for bit, and the outputs its decode over the updated
    caches; lengths put the new token on sinks, ring wraps, chunk and wave edges."""
    lens = [1, 5000, 70, 3, 4099, 2049]
    label = "fused-append-%s-%s%s" % (dtype, "".join(map(str, mask)), "-rw" if ret_window else "")
    say(label, lens)
    wl = workloads.make_workload("t", len(lens), lens, 32, 4, [mask], seed=83, dtype=dtype,
                                 window=64, sinks=4, device=dev(), Lmax=5000)
    wl.ret_window = ret_window
    lay = wl.layers[0]
    si = workloads.make_step_inputs(wl, seed=3, device=dev())
    want = oracle.append_project(lay, lens, si.q_pre, si.k_pre, si.k_new, si.v_new, si.Wq, si.Wk,
                                 wl.window, wl.sinks)
    olay = _oracle_layer(lay, want)
    check_decode(rtp, wl, label=label, oracle_layers=[olay], appends=[si])
    _check_caches(lay, want, label)


@pytest.mark.parametrize("Hq,Hkv,mask", [(32, 2, [1, 0]), (12, 4, [1, 0, 0, 1]), (10, 2, [1, 1]),
                                          (4, 4, [1, 0, 1, 1])])
def test_decode_step_fused_append_heads_per_kv(rtp, Hq, Hkv, mask):
    """The fused update with 16, 3, 5 and 1 query heads per KV head: two head groups per
    retrieval KV head (16), and groups whose chains leave lanes idle (3, 5, 1).  Every
    cache bit-exact, then the step's parity."""
    lens = [4099, 1, 2049, 300]
    label = "fused-append-G%d-%s" % (Hq // Hkv, "".join(map(str, mask)))
    say(label, lens)
    wl = workloads.make_workload("t", len(lens), lens, Hq, Hkv, [mask], seed=91, window=64,
                                 sinks=4, device=dev(), Lmax=4099)
    lay = wl.layers[0]
    si = workloads.make_step_inputs(wl, seed=5, device=dev())
    want = oracle.append_project(lay, lens, si.q_pre, si.k_pre, si.k_new, si.v_new, si.Wq, si.Wk,
                                 wl.window, wl.sinks)
    olay = _oracle_layer(lay, want)
    check_decode(rtp, wl, label=label, oracle_layers=[olay], appends=[si])
    _check_caches(lay, want, label)


def test_decode_step_fused_append_empty_sequence(rtp):
    """A sequence of length 0 takes no update and yields zeros; the others are updated."""
    lens = [0, 3000, 1]
    say("fused append with an empty sequence", lens)
    wl = workloads.make_workload("t", 3, lens, 32, 4, [[1, 0, 1, 0]], seed=84, dtype="f16",
                                 window=64, sinks=4, device=dev(), Lmax=3000)
    lay = wl.layers[0]
    si = workloads.make_step_inputs(wl, seed=4, device=dev())
    want = oracle.append_project(lay, lens, si.q_pre, si.k_pre, si.k_new, si.v_new, si.Wq, si.Wk,
                                 wl.window, wl.sinks)
    out, lse, _, _ = rtp.decode_workload(wl, want_debug=True, appends=[si])[0]
    torch.cuda.synchronize()
    _check_caches(lay, want, "empty")
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    olay = _oracle_layer(lay, want)
    orc = oracle.decode_layer(olay, lens, wl.Hq, wl.Hkv, wl.p, wl.bin_width, wl.scale_idx,
                              wl.scale_attn, wl.window, wl.sinks, batches=[1, 2])
    for (b, h), r in orc.items():
        assert max_err(out[b, h], r.out) <= 2e-3, (b, h)


@pytest.mark.parametrize("name", ["c1", "c2", "c4"])
def test_decode_step_fused_append_config(rtp, name):
    """The bench's `--with-append` step: the update fused into the step at 64K, 8 x 128K
    and 1M context (inputs that reproduce the workload's own last row and q_idx, so the
    selection stays the planted one); the oracle runs its own update and its own decode."""
    say("fused append + decode", name)
    wl = workloads.make_config(name, device=dev())
    lay = wl.layers[0]
    si = workloads.make_embedding_step_inputs(wl, device=dev())
    want = oracle.append_project(lay, wl.seq_lens, si.q_pre, si.k_pre, si.k_new, si.v_new, si.Wq,
                                 si.Wk, wl.window, wl.sinks)
    olay = _oracle_layer(lay, want)
    check_decode(rtp, wl, label="fused-append-" + name, oracle_layers=[olay], appends=[si])
    assert np.array_equal(_bits(oracle.np_of(lay.k_idx)), _bits(want[1]))
    assert np.array_equal(_bits(oracle.np_of(lay.q_idx)), _bits(want[0]))
    for b in range(wl.B):  # the new token's retrieval K/V rows of every sequence
        n = int(wl.seq_lens[b]) - 1
        if n >= 0:
            assert np.array_equal(_bits(oracle.np_of(lay.K_ret[b, :, n])), _bits(want[2][b, :, n]))
            assert np.array_equal(_bits(oracle.np_of(lay.V_ret[b, :, n])), _bits(want[3][b, :, n]))
    assert np.array_equal(_bits(oracle.np_of(lay.K_loc)), _bits(want[4]))
    assert np.array_equal(_bits(oracle.np_of(lay.V_loc)), _bits(want[5]))


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("p", [0.5, 0.9])
def test_decode_step_retrieval_window_small_ragged(rtp, dtype, p):
    """Retrieval heads that also attend to the sinks and the window (fused path f16,
    single-purpose kernels f32); lengths below, at and above window + sinks."""
    say("decode_step retrieval+window", dtype, p)
    wl = workloads.make_workload("t", 4, [3000, 1, 4099, 200], 32, 4, [[1, 0, 1, 0]], seed=66,
                                 p=p, dtype=dtype, window=256, sinks=4, device=dev())
    wl.ret_window = True
    check_decode(rtp, wl, label="retwin-%s-p%g" % (dtype, p))


def test_append_then_decode_c4(rtp):
    """The bench's `--with-append` step at 1M context: the cache update with the inputs
    that reproduce the workload's state, then the layer step; the oracle runs its own."""
    say("append + decode c4")
    wl = workloads.make_config("c4", device=dev())
    lay = wl.layers[0]
    si = workloads.make_embedding_step_inputs(wl, device=dev())
    want = oracle.append_project(lay, wl.seq_lens, si.q_pre, si.k_pre, si.k_new, si.v_new, si.Wq,
                                 si.Wk, wl.window, wl.sinks)
    olay = _oracle_layer(lay, want)
    sl = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev())
    rtp.rtp_append_project(lay, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks, si.q_pre,
                           si.k_pre, si.Wq, si.Wk, si.k_new, si.v_new)
    assert np.array_equal(_bits(oracle.np_of(lay.k_idx)), _bits(want[1]))
    assert np.array_equal(_bits(oracle.np_of(lay.q_idx)), _bits(want[0]))
    check_decode(rtp, wl, label="append-c4", oracle_layers=[olay])


@pytest.mark.parametrize("name", ["c1", "c2", "c4"])
def test_decode_step_retrieval_window_config(rtp, name):
    say("config", name, "retrieval + window")
    wl = workloads.make_config(name, device=dev())
    wl.ret_window = True
    check_decode(rtp, wl, label="%s-retwin" % name)


def test_decode_step_p1_is_dense_attention(rtp):
    say("decode_step p=1 dense")
    wl = workloads.make_workload("t", 2, [2500, 700], 8, 2, [[1, 0]], seed=62, p=1.0,
                                 dtype="f16", window=4096, sinks=4, device=dev())
    res = rtp.decode_workload(wl)[0]
    out = res[0].cpu().numpy()
    lay = wl.layers[0]
    for b, L in enumerate([2500, 700]):
        for h in range(8):
            if h < 4:
                K = oracle.np_of(lay.K_ret[b, 0, :L]).astype(np.float64)
                V = oracle.np_of(lay.V_ret[b, 0, :L]).astype(np.float64)
            else:
                slot = oracle.ring_slot(np.arange(L), 4096, 4)
                K = oracle.np_of(lay.K_loc[b, 0]).astype(np.float64)[slot]
                V = oracle.np_of(lay.V_loc[b, 0]).astype(np.float64)[slot]
            q = oracle.np_of(lay.q)[b, h].astype(np.float64)
            s = K @ q * wl.scale_attn
            w = np.exp(s - s.max())
            ref = (w[:, None] * V).sum(0) / w.sum()
            assert max_err(out[b, h], ref) <= 2e-3


def test_decode_step_empty_sequence(rtp):
    say("decode_step empty sequence")
    wl = workloads.make_workload("t", 2, [0, 1500], 8, 2, [[1, 0]], seed=63, p=0.9, dtype="f16",
                                 window=512, sinks=4, device=dev(), Lmax=1500)
    out, lse, thr, cnt = rtp.decode_workload(wl, want_debug=True)[0]
    out, lse, cnt = out.cpu().numpy(), lse.cpu().numpy(), cnt.cpu().numpy()
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf) and np.all(cnt[0] == 0)
    assert np.all(np.isfinite(out[1]))


HEAVY_WINDOW_LENS = [9000, 1, 700, 5000, 8196, 8197, 20000, 8200]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_step_heavy_window_ragged(rtp, dtype):
    """Eight sequences with three local heads each: their 8196-row rings need more window
    blocks than the launch holds beside the selection blocks at 256 rows, so every window
    block takes 512 rows and the step runs the heavy-window kernel (nontemporal rows through
    the rolling two-buffer loop).  The ragged lengths leave blocks with a full list, a
    partial list (700 rows: one block of 512, one of 188), a single row, and none."""
    say("decode_step heavy windows", dtype)
    wl = workloads.make_workload("t", 8, HEAVY_WINDOW_LENS, 32, 4, [[1, 0, 0, 0]], seed=65,
                                 p=0.9, dtype=dtype, window=8192, sinks=4, device=dev())
    check_decode(rtp, wl, label="heavy-window-%s" % dtype)


def test_decode_step_heavy_window_empty_sequence(rtp):
    """The heavy-window kernel with an empty sequence in the batch: its heads come out zero
    with lse = -inf, and the other sequences still match the oracle."""
    say("decode_step heavy windows, empty sequence")
    lens = [0] + HEAVY_WINDOW_LENS[1:]
    wl = workloads.make_workload("t", 8, lens, 32, 4, [[1, 0, 0, 0]], seed=66, p=0.9,
                                 dtype="f16", window=8192, sinks=4, device=dev())
    out, lse, thr, cnt = (t.cpu().numpy() for t in rtp.decode_workload(wl, want_debug=True)[0][:4])
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf) and np.all(cnt[0] == 0)
    orc = oracle.decode_layer(wl.layers[0], wl.seq_lens, wl.Hq, wl.Hkv, wl.p, wl.bin_width,
                              wl.scale_idx, wl.scale_attn, wl.window, wl.sinks,
                              heads=list(range(8, 32)), batches=range(1, 8))
    for (b, h), r in orc.items():
        e = max_err(out[b, h], r.out)
        assert e <= out_tol("f16"), "b %d head %d: max |dO| = %g" % (b, h, e)


def test_decode_step_deterministic(rtp):
    say("decode_step determinism")
    wl = workloads.make_workload("t", 2, [20000, 9000], 32, 4, [[1, 0, 0, 1]], seed=64, p=0.9,
                                 dtype="f16", device=dev())
    a = [t.clone() for t in rtp.decode_workload(wl, want_debug=True)[0]]
    b = rtp.decode_workload(wl, want_debug=True)[0]
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_decode_step_bf16_single_purpose(rtp):
    """bfloat16 caches with 20 query heads per KV head: the single-purpose kernels."""
    say("bf16 G=20")
    wl = workloads.make_workload("t", 3, [5000, 1, 2300], 60, 3, [[1, 0, 1]], seed=93, p=0.9,
                                 dtype="bf16", window=384, sinks=4, device=dev())
    check_decode(rtp, wl, label="bf16-G20")


def test_decode_step_bf16_64k(rtp):
    """bfloat16 caches at the 64K layout (the fused path on bf16 MFMAs)."""
    say("bf16 64K")
    wl = workloads.make_workload("c1-bf16", 1, [65536], 32, 4, [[1, 0, 0, 0]], seed=1,
                                 dtype="bf16", device=dev())
    check_decode(rtp, wl, label="c1-bf16")


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_decode_step_config_bf16(rtp, name):
    """The bench's `--dtype bf16` configurations at full size."""
    say("config", name, "bf16")
    wl = workloads.make_config(name, device=dev(), dtype="bf16")
    check_decode(rtp, wl, label="%s-bf16" % name)


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c4"])
def test_decode_step_config(rtp, name):
    say("config", name)
    wl = workloads.make_config(name, device=dev())
    check_decode(rtp, wl, label=name)


@pytest.mark.parametrize("p", [0.8, 0.95])
def test_decode_step_c4_p_sweep(rtp, p):
    say("config c4 p", p)
    wl = workloads.make_config("c4", device=dev(), p=p)
    check_decode(rtp, wl, label="c4-p%g" % p)


def test_decode_step_c3_48_layers(rtp):
    say("config c3 (48 layers; all retrieval heads, 8 local query heads per layer)")
    wl = workloads.make_config("c3", device=dev())
    check_decode(rtp, wl, local_sample=8, label="c3")


def test_decode_step_dense_window_1m(rtp):
    """The bench's dense reference (`--dense`): every KV head local, with a window that
    holds all 1M tokens, which is exact dense decode attention for the 32 query heads."""
    say("dense decode at 1M (window = L)")
    L = 1 << 20
    wl = workloads.make_workload("dense", 1, [L], 32, 4, [[0, 0, 0, 0]], seed=4, window=L,
                                 device=dev())
    check_decode(rtp, wl, label="dense-1M")


def test_decode_step_max_context(rtp):
    """The longest sequence the fused step takes, Lmax = 2^24 tokens (the 1M layer's heads
    and classes): 8192 histogram chunks, stage-T blocks of 32 chunks, 4096 selection blocks
    and 4096 partials per retrieval head in the merge (its limit), and suffix-table sums
    near the top of the fixed-point range."""
    say("config c4 at 2^24 tokens")
    wl = workloads.make_c4(device=dev(), L=1 << 24)
    check_decode(rtp, wl, label="c4-16M")


# ---------------------------------------------------------------------------
# rtp_prefill: causal attention of a prompt and the decode state it leaves
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("lens,window,sinks", [([300, 37, 1], 64, 4), ([17], 8, 0),
                                               ([200], 4096, 4)])
def test_prefill_matches_oracle(rtp, lens, window, sinks):
    say("prefill", lens, window, sinks)
    pr = workloads.make_prompt(lens, 8, 2, [1, 0], seed=91, device=dev())
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    scale = 1.0 / math.sqrt(128)
    pf = rtp.rtp_prefill(sl, pr.kv_is_retrieval, pr.q, pr.K, pr.V, window, sinks, scale,
                         pr.k_pre, pr.Wk, with_state=True)
    out = pf.out.cpu().numpy()
    ref = oracle.prefill_layer(pr.q, pr.K, pr.V, pr.kv_is_retrieval, lens, scale, window, sinks)
    worst = 0.0
    for (b, h, t), o in ref.items():
        e = max_err(out[b, h, t], o)
        worst = max(worst, e)
        assert e <= 2e-3, (b, h, t, e)
    say("worst |dO|", worst)
    want = oracle.prefill_state(pr.K, pr.V, pr.k_pre, pr.Wk, pr.kv_is_retrieval, lens, window,
                                sinks, max(lens))
    got = [pf.k_idx, pf.K_ret, pf.V_ret, pf.K_loc, pf.V_loc]
    for name, g, w in zip(["k_idx", "K_ret", "V_ret", "K_loc", "V_loc"], got, want):
        assert np.array_equal(_bits(oracle.np_of(g)), _bits(w)), name


def test_prefill_long_prompt_sampled(rtp):
    """A 9000-token prompt with the pages' window (8192 + 4 sinks): positions around the
    tile edges and the window's edges, every head, against the oracle."""
    say("prefill 9000 sampled")
    L = 9000
    pr = workloads.make_prompt([L], 8, 2, [1, 0], seed=92, device=dev(), with_kpre=False)
    sl = torch.tensor([L], dtype=torch.int32, device=dev())
    scale = 1.0 / math.sqrt(128)
    out = rtp.rtp_prefill(sl, pr.kv_is_retrieval, pr.q, pr.K, pr.V, 8192, 4, scale).out
    out = out.cpu().numpy()
    pos = [0, 1, 3, 4, 15, 16, 17, 31, 32, 4099, 8191, 8192, 8195, 8196, 8197, 8211, 8212,
           8999]
    ref = oracle.prefill_layer(pr.q, pr.K, pr.V, pr.kv_is_retrieval, [L], scale, 8192, 4,
                               positions=pos)
    for (b, h, t), o in ref.items():
        assert max_err(out[b, h, t], o) <= 2e-3, (h, t)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_64k_sampled(rtp, dtype):
    """The prefill the bench times (one 64K-token prompt, 32 query heads on 4 KV heads,
    KV head 0 dense, window 8192 + 4 sinks), every head at positions around the tile,
    stage and window edges, against the oracle."""
    L = 65536
    say("prefill 64K sampled", dtype)
    pr = workloads.make_prompt([L], 32, 4, [1, 0, 0, 0], seed=7, device=dev(), with_kpre=False,
                               dtype=dtype)
    sl = torch.tensor([L], dtype=torch.int32, device=dev())
    scale = 1.0 / math.sqrt(128)
    out = rtp.rtp_prefill(sl, pr.kv_is_retrieval, pr.q, pr.K, pr.V, 8192, 4, scale).out
    pos = [0, 3, 4, 31, 32, 127, 128, 8191, 8195, 8196, 8197, 8227, 32768, 40000, 65503,
           65504, 65535]
    got = out[0][:, pos].cpu().numpy()
    ref = oracle.prefill_layer(pr.q, pr.K, pr.V, pr.kv_is_retrieval, [L], scale, 8192, 4,
                               positions=pos)
    worst = 0.0
    for (b, h, t), o in ref.items():
        e = max_err(got[h, pos.index(t)], o)
        worst = max(worst, e)
        assert e <= 2e-3, (h, t, e)
    say("worst |dO|", worst)


def test_prefill_1m_sampled(rtp):
    """A 1M-token prompt (the context of the decode step), KV head 0 dense, window 8192 + 4
    sinks: every head at positions near the start, the window edge, the middle and the end,
    against the oracle's attention over the same key sets."""
    L = 1 << 20
    say("prefill 1M sampled")
    pr = workloads.make_prompt([L], 32, 4, [1, 0, 0, 0], seed=7, device=dev(), with_kpre=False)
    sl = torch.tensor([L], dtype=torch.int32, device=dev())
    scale = 1.0 / math.sqrt(128)
    out = rtp.rtp_prefill(sl, pr.kv_is_retrieval, pr.q, pr.K, pr.V, 8192, 4, scale).out
    pos = [0, 31, 32, 8195, 8196, 524287, 1048543, 1048575]
    got = out[0][:, pos].cpu().numpy()
    del out
    qs = pr.q[0][:, pos].cpu().numpy()
    Kn, Vn = oracle.np_of(pr.K[0]), oracle.np_of(pr.V[0])
    worst = 0.0
    for h in range(32):
        kv = h // 8
        for i, t in enumerate(pos):
            rows = oracle.prefill_rows(t, kv == 0, 8192, 4)
            o, _ = oracle.attention(qs[h, i], Kn[kv], Vn[kv], rows, scale)
            e = max_err(got[h, i], o)
            worst = max(worst, e)
            assert e <= 2e-3, (h, t, e)
    say("worst |dO|", worst)


def test_prefill_bf16_long_prompt_sampled(rtp):
    """A 9000-token bf16 prompt (its kernel stages 64 keys per barrier, fp16 128)."""
    L = 9000
    say("prefill bf16 9000 sampled")
    pr = workloads.make_prompt([L], 8, 2, [1, 0], seed=96, device=dev(), with_kpre=False,
                               dtype="bf16")
    sl = torch.tensor([L], dtype=torch.int32, device=dev())
    scale = 1.0 / math.sqrt(128)
    out = rtp.rtp_prefill(sl, pr.kv_is_retrieval, pr.q, pr.K, pr.V, 8192, 4, scale).out
    out = out.cpu().numpy()
    pos = [0, 1, 31, 32, 63, 64, 65, 4099, 8191, 8192, 8196, 8197, 8999]
    ref = oracle.prefill_layer(pr.q, pr.K, pr.V, pr.kv_is_retrieval, [L], scale, 8192, 4,
                               positions=pos)
    for (b, h, t), o in ref.items():
        assert max_err(out[b, h, t], o) <= 2e-3, (h, t)


@pytest.mark.parametrize("lens,window,sinks", [([300, 37, 1], 64, 4), ([200], 4096, 4)])
def test_prefill_bf16_matches_oracle(rtp, lens, window, sinks):
    """bf16 prompt: outputs within the 2e-3 bar, and the decode state (k_idx rounded to
    bf16, K/V rows, rings) bit-exact."""
    say("prefill bf16", lens, window, sinks)
    pr = workloads.make_prompt(lens, 8, 2, [1, 0], seed=95, device=dev(), dtype="bf16")
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    scale = 1.0 / math.sqrt(128)
    pf = rtp.rtp_prefill(sl, pr.kv_is_retrieval, pr.q, pr.K, pr.V, window, sinks, scale,
                         pr.k_pre, pr.Wk, with_state=True)
    out = pf.out.cpu().numpy()
    ref = oracle.prefill_layer(pr.q, pr.K, pr.V, pr.kv_is_retrieval, lens, scale, window, sinks)
    worst = 0.0
    for (b, h, t), o in ref.items():
        e = max_err(out[b, h, t], o)
        worst = max(worst, e)
        assert e <= 2e-3, (b, h, t, e)
    say("worst |dO|", worst)
    want = oracle.prefill_state(pr.K, pr.V, pr.k_pre, pr.Wk, pr.kv_is_retrieval, lens, window,
                                sinks, max(lens))
    got = [pf.k_idx, pf.K_ret, pf.V_ret, pf.K_loc, pf.V_loc]
    for name, g, w in zip(["k_idx", "K_ret", "V_ret", "K_loc", "V_loc"], got, want):
        assert g.dtype == torch.bfloat16, name
        assert np.array_equal(_bits(oracle.np_of(g)), _bits(w)), name


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (32, 2), (12, 4)])
def test_prefill_heads_per_kv(rtp, Hq, Hkv):
    """Query heads per KV head other than the eight wavefronts of a block: idle
    wavefronts (G < 8), a second pass (G = 16), and G = 3."""
    lens = [130, 47]
    say("prefill heads", Hq, Hkv, lens)
    mask = [1] + [0] * (Hkv - 1)
    pr = workloads.make_prompt(lens, Hq, Hkv, mask, seed=94, device=dev())
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    scale = 1.0 / math.sqrt(128)
    out = rtp.rtp_prefill(sl, pr.kv_is_retrieval, pr.q, pr.K, pr.V, 32, 2, scale).out
    out = out.cpu().numpy()
    ref = oracle.prefill_layer(pr.q, pr.K, pr.V, pr.kv_is_retrieval, lens, scale, 32, 2)
    for (b, h, t), o in ref.items():
        assert max_err(out[b, h, t], o) <= 2e-3, (b, h, t)
