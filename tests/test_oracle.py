"""Pins of the CPU oracle against what the method and the mathematics fix.

None of these compares the oracle with a copy of itself: they check hand-worked
examples (tests/golden/worked_examples.json), exact small-integer cases, error
bounds, the exact sort-based top-p the histogram rule must contain, textbook
dense attention (torch's scaled_dot_product_attention in fp64), and invariants
of the rule (monotone in p, permutation equivariant, shift invariant).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def gold():
    with open(GOLD) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# fp16 decoding
# ---------------------------------------------------------------------------
def test_half_decode_matches_numpy_for_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    f = oracle.lib().rtpo_half_to_double
    got = np.array([f(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.isinf(got[np.isinf(ref)]))
    assert np.all(np.isnan(got[np.isnan(ref)]))


# ---------------------------------------------------------------------------
# indexer score
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_index_score_exact_on_small_integers(dt):
    # every product and partial sum is a small integer: the fma chain is exact and
    # z must equal scale * (q . k) exactly, for every token and every dimension.
    rng = np.random.default_rng(11)
    L, r = 257, 16
    q = rng.integers(-20, 21, r).astype(np.float32)
    k = rng.integers(-30, 31, (L, r)).astype(dt)
    z = oracle.index_score(q, k, 0.25)
    exact = 0.25 * (k.astype(np.int64) @ q.astype(np.int64))
    assert np.array_equal(z.astype(np.float64), exact.astype(np.float64))


def test_index_score_each_dimension_counts():
    # a one-hot key picks exactly one q component: catches dropped or shifted terms
    r = 16
    q = (np.arange(r, dtype=np.float32) + 1.0) * np.float32(1.5)
    k = np.eye(r, dtype=np.float16)
    z = oracle.index_score(q, k, 0.5)
    assert np.array_equal(z, (0.5 * q).astype(np.float32))


def test_index_score_within_fma_chain_error_bound():
    rng = np.random.default_rng(12)
    L, r = 4096, 16
    q = (rng.standard_normal(r) * 4).astype(np.float32)
    k = rng.standard_normal((L, r)).astype(np.float16)
    z = oracle.index_score(q, k, 0.25).astype(np.float64)
    prod = k.astype(np.float64) * q.astype(np.float64)[None, :]
    exact = 0.25 * prod.sum(1)
    bound = 0.25 * (r + 1) * 2.0 ** -24 * np.abs(prod).sum(1) + 2.0 ** -24 * np.abs(exact)
    assert np.all(np.abs(z - exact) <= bound)
    # and a transposed / wrong-head query would be far outside the bound
    z_bad = oracle.index_score(q[::-1].copy(), k, 0.25).astype(np.float64)
    assert np.mean(np.abs(z_bad - exact) > bound) > 0.9


# ---------------------------------------------------------------------------
# histogram top-p: hand-worked examples
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ex", gold()["select"], ids=lambda e: e["name"])
def test_worked_example_select(ex):
    z = np.array(ex["z"], dtype=np.float32)
    s = oracle.topp_select(z, ex["p"], ex["w"])
    assert s.A == ex["A"]
    assert s.bstar == ex["bstar"]
    assert s.idx.tolist() == ex["S"]
    assert oracle.cells(z, ex["w"]).tolist() == ex["cells"]
    Z = s.hist.sum()
    assert abs(Z - ex["Z"]) < 1e-6
    for j, m in ex["masses"].items():
        assert abs(s.hist[int(j)] - m) < 1e-6
    nz = {int(j) for j in ex["masses"]}
    for j in range(256):
        if j not in nz and j != 255:
            assert s.hist[j] == 0.0
    assert abs(s.hist[:s.bstar + 1].sum() / Z - ex["mass_frac"]) < 1e-6
    assert set(ex["exact_topp"]) <= set(s.idx.tolist())


@pytest.mark.parametrize("ex", gold()["attention"], ids=lambda e: e["name"])
def test_worked_example_attention(ex):
    K = np.array(ex["K"], dtype=np.float32)
    V = np.array(ex["V"], dtype=np.float32)
    o, lse = oracle.attention(np.array(ex["q"]), K, V, ex["S"], ex["scale"])
    assert np.allclose(o, ex["out"], atol=1e-6)
    s = np.array([ex["scale"] * 1.0, 0.0])
    assert abs(lse - math.log(np.exp(s).sum())) < 1e-12


# ---------------------------------------------------------------------------
# histogram top-p: exact top-p containment and invariants
# ---------------------------------------------------------------------------
def exact_topp(z, p):
    """Exact top-p by sorting: the shortest prefix of tokens in descending logit order
    whose softmax mass reaches p (fp64)."""
    z64 = np.asarray(z, dtype=np.float64)
    e = np.exp(z64 - z64.max())
    order = np.argsort(-z64, kind="stable")
    cum = np.cumsum(e[order])
    k = int(np.searchsorted(cum, p * cum[-1] * (1 - 1e-12))) + 1
    return order[:min(k, len(z64))], e


def _logit_sets():
    rng = np.random.default_rng(2024)
    out = []
    for L in [1, 2, 3, 7, 64, 255, 256, 1000, 4099]:
        for sig in [0.05, 1.0, 3.0, 12.0]:
            out.append(("g%d_%g" % (L, sig), (sig * rng.standard_normal(L)).astype(np.float32)))
    # planted spikes on a flat background
    z = rng.standard_normal(5000).astype(np.float32)
    z[rng.choice(5000, 3, replace=False)] = 14.0
    out.append(("spike3", z))
    # broad: many moderately high tokens
    z = (rng.standard_normal(8000) - 5).astype(np.float32)
    z[rng.choice(8000, 800, replace=False)] = (2 + 0.7 * rng.standard_normal(800)).astype(np.float32)
    out.append(("broad", z))
    # ties and values exactly on cell edges
    out.append(("allequal", np.full(300, 1.7, dtype=np.float32)))
    out.append(("edges", (rng.integers(-80, 40, 2000) * 0.125).astype(np.float32)))
    out.append(("coarse", (rng.integers(-8, 8, 500) * 0.5).astype(np.float32)))
    # huge range: tail bin populated
    z = (rng.standard_normal(3000) * 20).astype(np.float32)
    out.append(("wide", z))
    out.append(("neg", (-1000 + rng.standard_normal(700)).astype(np.float32)))
    return out


LOGITS = _logit_sets()
PS = [0.1, 0.5, 0.8, 0.9, 0.95, 0.999]


@pytest.mark.parametrize("name,z", LOGITS, ids=[n for n, _ in LOGITS])
def test_rule_contains_exact_topp_and_reaches_p(name, z):
    L = len(z)
    prev = None
    for p in PS:
        s = oracle.topp_select(z, p)
        idx = s.idx
        assert 1 <= len(idx) <= L
        assert np.all(np.diff(idx) > 0) and idx[0] >= 0 and idx[-1] < L
        ex, e = exact_topp(z, p)
        assert set(ex.tolist()) <= set(idx.tolist()), (name, p)
        assert e[idx].sum() >= p * e.sum() * (1 - 1e-12)
        # the threshold bin is the first whose cumulative mass reaches p*Z
        C = np.cumsum(s.hist)
        assert C[s.bstar] >= p * C[-1]
        if s.bstar > 0:
            assert C[s.bstar - 1] < p * C[-1]
        # the maximum sits in bin 0, so bin 0 is never empty
        assert s.hist[0] > 0
        # bin totals equal the softmax normaliser relative to exp((A+1)w)
        Zref = np.exp(z.astype(np.float64) - (s.A + 1) * 0.125).sum()
        assert abs(C[-1] - Zref) <= 1e-12 * Zref
        assert s.A == int(np.floor(z.astype(np.float64).max() / 0.125))
        if prev is not None:
            assert set(prev.tolist()) <= set(idx.tolist())   # monotone in p
        prev = idx
    assert oracle.topp_select(z, 1.0).count == L


@pytest.mark.parametrize("name,z", LOGITS[::3], ids=[n for n, _ in LOGITS[::3]])
def test_rule_permutation_equivariant(name, z):
    rng = np.random.default_rng(5)
    perm = rng.permutation(len(z))
    for p in [0.5, 0.9]:
        s = oracle.topp_select(z, p)
        sp = oracle.topp_select(z[perm], p)
        back = set(perm[sp.idx].tolist())
        assert back == set(s.idx.tolist())


def test_rule_shift_by_whole_cells_keeps_set():
    rng = np.random.default_rng(6)
    z = (rng.integers(-400, 400, 3000) / 1024.0).astype(np.float32)
    for k in [-24, -1, 1, 7, 80]:
        for p in [0.3, 0.9]:
            a = oracle.topp_select(z, p)
            b = oracle.topp_select((z + np.float32(k * 0.125)).astype(np.float32), p)
            assert np.array_equal(a.idx, b.idx)
            assert b.A == a.A + k and b.bstar == a.bstar
            assert np.allclose(a.hist, b.hist, rtol=1e-12, atol=0)


def test_tail_bin_catches_far_tokens():
    z = np.array([10.0] + [10.0 - 40.0] * 50 + [10.0 - 31.0], dtype=np.float32)
    s = oracle.topp_select(z, 0.9)
    assert s.idx.tolist() == [0]
    # cells 248 below the top land in bin 248; 320 below land in the tail bin 255
    assert s.hist[248] > 0 and s.hist[255] > 0
    assert oracle.topp_select(z, 1.0).count == len(z)


def test_bin_width_is_a_parameter():
    z = np.array([0.0, 0.3, 0.55, 1.0], dtype=np.float32)
    s = oracle.topp_select(z, 0.2, bin_width=0.5)
    # w = 1/2: cells 0,0,1,2 -> A = 2, bins 2,2,1,0; masses e^{z-1.5}: bin 0 = 0.6065,
    # bin 1 = 0.3867, bin 2 = 0.5243 (Z = 1.5175).  p = 0.2 stops in bin 0, p = 0.5 in bin 1.
    assert s.A == 2
    assert s.idx.tolist() == [3]
    s = oracle.topp_select(z, 0.5, bin_width=0.5)
    assert s.idx.tolist() == [2, 3]


# ---------------------------------------------------------------------------
# attention: textbook special cases
# ---------------------------------------------------------------------------
def sdpa64(q, K, V, scale, mask=None):
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64)).view(1, 1, 1, -1)
    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64)).view(1, 1, K.shape[0], -1)
    Vt = torch.from_numpy(np.asarray(V, dtype=np.float64)).view(1, 1, V.shape[0], -1)
    m = None if mask is None else torch.from_numpy(mask).view(1, 1, 1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m,
                                                            scale=scale).view(-1).numpy()


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_attention_all_rows_is_dense_softmax_attention(dt):
    rng = np.random.default_rng(7)
    N, d = 777, 128
    K = rng.standard_normal((N, d)).astype(dt)
    V = rng.standard_normal((N, d)).astype(dt)
    q = rng.standard_normal(d).astype(dt)
    o, lse = oracle.attention(q, K, V, np.arange(N), 1 / math.sqrt(d))
    ref = sdpa64(q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), 1 / math.sqrt(d))
    assert np.allclose(o, ref, atol=1e-12, rtol=0)
    from scipy.special import logsumexp
    s = (K.astype(np.float64) @ q.astype(np.float64)) / math.sqrt(d)
    assert abs(lse - logsumexp(s)) < 1e-12


def test_attention_subset_is_masked_dense_attention():
    rng = np.random.default_rng(8)
    N, d = 500, 64
    K = rng.standard_normal((N, d)).astype(np.float16)
    V = rng.standard_normal((N, d)).astype(np.float16)
    q = rng.standard_normal(d)
    rows = np.sort(rng.choice(N, 37, replace=False))
    o, _ = oracle.attention(q, K, V, rows, 0.2)
    mask = np.zeros(N, dtype=bool)
    mask[rows] = True
    ref = sdpa64(q, K.astype(np.float64), V.astype(np.float64), 0.2, mask)
    assert np.allclose(o, ref, atol=1e-12, rtol=0)
    # row order does not matter
    o2, _ = oracle.attention(q, K, V, rows[::-1].copy(), 0.2)
    assert np.allclose(o, o2, atol=1e-13, rtol=0)


def test_attention_special_cases():
    rng = np.random.default_rng(9)
    N, d = 64, 128
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    rows = np.array([3, 9, 10, 40])
    # q = 0: uniform weights, output is the mean of the selected rows
    o, lse = oracle.attention(np.zeros(d), K, V, rows, 0.1)
    assert np.allclose(o, V[rows].astype(np.float64).mean(0), atol=1e-14)
    assert abs(lse - math.log(4)) < 1e-14
    # identical value rows: output is that row
    Vc = np.tile(V[5:6], (N, 1))
    o, _ = oracle.attention(rng.standard_normal(d), K, Vc, rows, 0.3)
    assert np.allclose(o, Vc[0], atol=1e-12)
    # a single row: output is that row, lse is its logit
    qv = rng.standard_normal(d)
    o, lse = oracle.attention(qv, K, V, [17], 0.3)
    assert np.array_equal(o, V[17].astype(np.float64))
    assert abs(lse - 0.3 * float(qv @ K[17].astype(np.float64))) < 1e-12


# ---------------------------------------------------------------------------
# window set and ring layout
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("window,sinks", [(8192, 4), (16, 4), (5, 2), (8, 0), (1, 4)])
def test_window_positions_and_ring_slots(window, sinks):
    for L in list(range(1, 40)) + [window + sinks - 1, window + sinks, window + sinks + 1,
                                   3 * window + 7, 100000]:
        pos = oracle.window_positions(L, window, sinks)
        brute = [n for n in range(max(0, L - window - sinks - 1), L)
                 if n >= L - window] + [n for n in range(min(sinks, L))]
        assert sorted(set(brute)) == sorted(pos.tolist()) and len(set(pos.tolist())) == len(pos)
        if L <= window + sinks:
            assert sorted(pos.tolist()) == list(range(L))
        slots = oracle.ring_slot(pos, window, sinks)
        assert len(set(slots.tolist())) == len(slots)          # no two positions share a slot
        assert slots.min() >= 0 and slots.max() < window + sinks


# ---------------------------------------------------------------------------
# a whole layer against dense attention
# ---------------------------------------------------------------------------
def _layer_dense_reference(wl, layer, b, h):
    G = wl.G
    kh = h // G
    mask = layer.kv_is_retrieval
    L = int(wl.seq_lens[b])
    q = oracle.np_of(layer.q)[b, h].astype(np.float64)
    if mask[kh]:
        kr = layer.ret_heads.index(kh)
        K = oracle.np_of(layer.K_ret[b, kr, :L]).astype(np.float64)
        V = oracle.np_of(layer.V_ret[b, kr, :L]).astype(np.float64)
    else:
        kl = layer.loc_heads.index(kh)
        Kr = oracle.np_of(layer.K_loc[b, kl]).astype(np.float64)
        Vr = oracle.np_of(layer.V_loc[b, kl]).astype(np.float64)
        slot = oracle.ring_slot(np.arange(L), wl.window, wl.sinks)
        K, V = Kr[slot], Vr[slot]
    return K, V, q


def test_layer_with_p1_and_full_window_is_dense_attention():
    import workloads
    wl = workloads.make_workload("t", 2, [300, 171], 8, 4, [[1, 0, 1, 0]], seed=5, p=1.0,
                                 window=512, sinks=4, dtype="f16")
    res = oracle.decode_step(wl)[0]
    layer = wl.layers[0]
    for b in range(2):
        for h in range(8):
            K, V, q = _layer_dense_reference(wl, layer, b, h)
            ref = sdpa64(q, K, V, wl.scale_attn)
            assert np.allclose(res[(b, h)].out, ref, atol=1e-12, rtol=0), (b, h)
            if layer.kv_is_retrieval[h // 2]:
                assert res[(b, h)].sel.count == int(wl.seq_lens[b])


def test_layer_local_heads_use_window_and_sinks():
    import workloads
    wl = workloads.make_workload("t", 1, [203], 4, 2, [[0, 1]], seed=6, p=0.9, window=32,
                                 sinks=4, dtype="f32")
    res = oracle.decode_step(wl)[0]
    layer = wl.layers[0]
    L = 203
    for h in range(2):   # KV head 0 is local
        K, V, q = _layer_dense_reference(wl, layer, 0, h)
        m = np.zeros(L, dtype=bool)
        m[:4] = True
        m[L - 32:] = True
        ref = sdpa64(q, K, V, wl.scale_attn, m)
        assert np.allclose(res[(0, h)].out, ref, atol=1e-12, rtol=0)
    for h in range(2, 4):  # KV head 1 is a retrieval head: masked attention over S
        K, V, q = _layer_dense_reference(wl, layer, 0, h)
        m = np.zeros(L, dtype=bool)
        m[res[(0, h)].sel.idx] = True
        ref = sdpa64(q, K, V, wl.scale_attn, m)
        assert np.allclose(res[(0, h)].out, ref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# fixed top-k through the same histogram
# ---------------------------------------------------------------------------
GOLD_TOPK = os.path.join(os.path.dirname(__file__), "golden", "topk_examples.json")


def _topk_gold():
    with open(GOLD_TOPK) as f:
        return json.load(f)["select"]


@pytest.mark.parametrize("ex", _topk_gold(), ids=lambda e: e["name"])
def test_topk_worked_example(ex):
    z = np.asarray(ex["z"], dtype=np.float32)
    s = oracle.topk_select(z, ex["k"], ex["w"])
    assert s.A == ex["A"]
    assert s.bstar == ex["bstar"]
    assert s.idx.tolist() == ex["S"]
    want = np.zeros(256)
    for j, c in ex["counts"].items():
        want[int(j)] = c
    assert np.array_equal(s.hist, want)


def _topk_by_sorting_cells(z, k, w=0.125):
    """Brute force from another angle: visit the occupied cells from the top down (every
    cell 255 or more below the top counts as one tail cell) and keep whole cells until
    at least k tokens are kept."""
    g = np.floor(np.asarray(z, dtype=np.float32).astype(np.float64) / w).astype(np.int64)
    A = g.max()
    key = np.maximum(g, A - 255)
    kept = np.zeros(len(z), dtype=bool)
    for c in sorted(set(key.tolist()), reverse=True):
        kept |= key == c
        if kept.sum() >= k:
            break
    return np.nonzero(kept)[0]


KS = [1, 2, 3, 10, 100, 2048, 4096, 10 ** 6]


@pytest.mark.parametrize("name,z", LOGITS, ids=[n for n, _ in LOGITS])
def test_topk_rule_contains_top_k_and_is_minimal(name, z):
    L = len(z)
    zs = np.sort(z.astype(np.float64))[::-1]
    prev = None
    for k in KS:
        s = oracle.topk_select(z, k)
        idx = s.idx
        assert np.all(np.diff(idx) > 0)
        assert len(idx) >= min(k, L)
        # every token at or above the k-th largest logit is kept (ties included) ...
        kth = zs[min(k, L) - 1]
        assert set(np.nonzero(z.astype(np.float64) >= kth)[0].tolist()) <= set(idx.tolist())
        # ... the kept set is an upper set in z ...
        out = np.setdiff1d(np.arange(L), idx)
        if len(out):
            assert z[out].max() < z[idx].min()
        # ... counts are exact and the threshold bin is the first to reach k
        assert s.hist.sum() == L and np.all(s.hist == np.round(s.hist))
        C = np.cumsum(s.hist)
        if k <= L:
            assert C[s.bstar] >= k
        else:
            assert s.bstar == 255 and len(idx) == L
        if s.bstar > 0 and k <= L:
            assert C[s.bstar - 1] < k
        assert np.array_equal(idx, _topk_by_sorting_cells(z, k))
        if prev is not None:
            assert set(prev.tolist()) <= set(idx.tolist())   # monotone in k
        prev = idx


@pytest.mark.parametrize("name,z", LOGITS[::3], ids=[n for n, _ in LOGITS[::3]])
def test_topk_permutation_and_cell_shift(name, z):
    rng = np.random.default_rng(7)
    perm = rng.permutation(len(z))
    for k in [1, 5, 300]:
        s = oracle.topk_select(z, k)
        sp = oracle.topk_select(z[perm], k)
        assert set(perm[sp.idx].tolist()) == set(s.idx.tolist())
        sh = oracle.topk_select((z.astype(np.float64) + 3 * 0.125).astype(np.float32), k)
        if np.array_equal(np.floor(z.astype(np.float64) / 0.125) + 3,
                          np.floor((z.astype(np.float64) + 0.375).astype(np.float32) / 0.125)):
            assert np.array_equal(sh.idx, s.idx) and sh.A == s.A + 3


# ---------------------------------------------------------------------------
# indexer projection and the cache append of a decode step
# ---------------------------------------------------------------------------
def test_project_exact_on_small_integers():
    rng = np.random.default_rng(11)
    x = rng.integers(-8, 8, 128).astype(np.float32)
    W = rng.integers(-8, 8, (128, 16)).astype(np.float32)
    want = x.astype(np.int64) @ W.astype(np.int64)
    assert np.array_equal(oracle.project(x, W), want.astype(np.float32))


def test_project_each_input_counts_once():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(128).astype(np.float32)
    W = rng.standard_normal((128, 16)).astype(np.float32)
    for c in [0, 1, 63, 127]:
        e = np.zeros(128, dtype=np.float32)
        e[c] = 1.0
        assert np.array_equal(oracle.project(e, W), W[c])
        U = np.zeros((128, 16), dtype=np.float32)
        U[c, 5] = 1.0
        out = oracle.project(x, U)
        assert out[5] == x[c] and np.all(np.delete(out, 5) == 0)


def test_project_follows_the_left_to_right_chain():
    # in the prescribed order 1e8 + 1 rounds back to 1e8 before -1e8 cancels it: 0; any
    # order that cancels the large terms first would give 1
    x = np.array([1e8, 1.0, -1e8], dtype=np.float32)
    W = np.ones((3, 1), dtype=np.float32)
    assert oracle.project(x, W)[0] == 0.0
    assert oracle.project(x[[0, 2, 1]], W)[0] == 1.0


def test_project_within_fma_chain_error_bound():
    rng = np.random.default_rng(13)
    u = 2.0 ** -24
    for _ in range(20):
        x = rng.standard_normal(128).astype(np.float32)
        W = (rng.standard_normal((128, 16)) / math.sqrt(128)).astype(np.float32)
        exact = x.astype(np.float64) @ W.astype(np.float64)
        bound = 128 * u / (1 - 128 * u) * (np.abs(x).astype(np.float64) @ np.abs(W).astype(np.float64))
        assert np.all(np.abs(oracle.project(x, W) - exact) <= bound)


class _Lay:
    def __init__(self, mask, q_idx, k_idx, K_ret, V_ret, K_loc, V_loc):
        self.kv_is_retrieval = np.asarray(mask, dtype=np.uint8)
        self.q_idx, self.k_idx, self.K_ret, self.V_ret = q_idx, k_idx, K_ret, V_ret
        self.K_loc, self.V_loc = K_loc, V_loc


def test_append_places_rows_and_rounds_to_half():
    B, Hkv, G, d, r, Lmax, window, sinks = 2, 2, 2, 1, 1, 12, 6, 2
    lay = _Lay([1, 0], np.full((B, Hkv * G, r), 7.0, np.float32),
               np.zeros((B, 1, Lmax, r), np.float16), np.zeros((B, 1, Lmax, d), np.float16),
               np.zeros((B, 1, Lmax, d), np.float16), np.zeros((B, 1, window + sinks, d), np.float16),
               np.zeros((B, 1, window + sinks, d), np.float16))
    q_pre = np.ones((B, Hkv * G, d), np.float32)
    k_pre = np.ones((B, Hkv, d), np.float32)
    k_new = np.array([[[1.5], [2.5]], [[3.5], [4.5]]], np.float16)
    v_new = -k_new
    # 1 + 2^-11 lies halfway between fp16 1 and 1 + 2^-10: ties to even give 1;
    # 1 + 3 * 2^-11 lies halfway between 1 + 2^-10 and 1 + 2^-9: ties to even give 1 + 2^-9
    Wq = np.array([[[0.5]], [[0.25]], [[9.0]], [[9.0]]], np.float32)
    for wk, want in [(1 + 2 ** -11, 1.0), (1 + 3 * 2 ** -11, 1 + 2 ** -9)]:
        Wk = np.array([[[wk]]], np.float32)
        q_idx, k_idx, K_ret, V_ret, K_loc, V_loc = oracle.append_project(
            lay, [10, 0], q_pre, k_pre, k_new, v_new, Wq, Wk, window, sinks)
        assert float(k_idx[0, 0, 9, 0]) == want
        assert np.count_nonzero(k_idx) == 1          # only row 9 of sequence 0
        assert K_ret[0, 0, 9, 0] == 1.5 and V_ret[0, 0, 9, 0] == -1.5
        assert np.count_nonzero(K_ret) == 1
        # position 9 of a local head: slot 2 + 9 % 6 = 5
        assert K_loc[0, 0, 5, 0] == 2.5 and V_loc[0, 0, 5, 0] == -2.5
        assert np.count_nonzero(K_loc) == 1
        # query heads 0, 1 (retrieval KV head 0) are projected, the local heads' keep theirs
        assert q_idx[0, 0, 0] == 0.5 and q_idx[0, 1, 0] == 0.25
        assert np.all(q_idx[0, 2:] == 7.0) and np.all(q_idx[1] == 7.0)


def test_append_sink_position_and_empty_sequence():
    B, Hkv, G, d, r, Lmax, window, sinks = 2, 2, 1, 1, 1, 12, 6, 2
    z16 = lambda *s: np.zeros(s, np.float16)
    lay = _Lay([0, 1], np.zeros((B, 2, r), np.float32), z16(B, 1, Lmax, r), z16(B, 1, Lmax, d),
               z16(B, 1, Lmax, d), z16(B, 1, window + sinks, d), z16(B, 1, window + sinks, d))
    k_new = np.full((B, Hkv, d), 2.0, np.float16)
    out = oracle.append_project(lay, [0, 2], np.ones((B, 2, d), np.float32),
                                np.ones((B, Hkv, d), np.float32), k_new, k_new,
                                np.ones((2, d, r), np.float32), np.full((1, d, r), 3.0, np.float32),
                                window, sinks)
    q_idx, k_idx, K_ret, V_ret, K_loc, V_loc = out
    assert np.count_nonzero(K_loc[0]) == 0 and np.count_nonzero(K_ret[0]) == 0   # L = 0
    assert K_loc[1, 0, 1, 0] == 2.0 and np.count_nonzero(K_loc) == 1             # sink slot 1
    assert K_ret[1, 0, 1, 0] == 2.0 and k_idx[1, 0, 1, 0] == 3.0
    assert q_idx[1, 1, 0] == 1.0 and q_idx[1, 0, 0] == 0.0   # only the retrieval head's query


def test_embedding_step_inputs_leave_the_layer_unchanged():
    import workloads
    wl = workloads.make_workload("t", 2, [300, 9], 8, 2, [[1, 0]], seed=3, window=16, sinks=4)
    lay = wl.layers[0]
    si = workloads.make_embedding_step_inputs(wl)
    out = oracle.append_project(lay, wl.seq_lens, si.q_pre, si.k_pre, si.k_new, si.v_new, si.Wq,
                                si.Wk, wl.window, wl.sinks)
    before = [oracle.np_of(t) for t in (lay.q_idx, lay.k_idx, lay.K_ret, lay.V_ret, lay.K_loc,
                                        lay.V_loc)]
    for name, a, b in zip(["q_idx", "k_idx", "K_ret", "V_ret", "K_loc", "V_loc"], out, before):
        a16 = a.view(np.uint16) if a.dtype == np.float16 else a.view(np.uint32)
        b16 = b.view(np.uint16) if b.dtype == np.float16 else b.view(np.uint32)
        assert np.array_equal(a16, b16), name


def test_layer_retrieval_heads_with_the_window_attend_to_the_union():
    """With the window variant a retrieval head attends to S united with the sinks and the
    last `window` positions; with p chosen so that S is the single top token, that is
    the window set plus that token, checked against dense attention on those rows."""
    import workloads
    wl = workloads.make_workload("t", 1, [600], 4, 1, [[1]], seed=9, dtype="f32", window=64,
                                 sinks=4, p=1e-6, classes=lambda b, k, r: ["concentrated"] * 4,
                                 fixed_k={"concentrated": 2})
    wl.ret_window = True
    res = oracle.decode_step(wl)[0]
    lay = wl.layers[0]
    for h in range(4):
        r = res[(0, h)]
        win = oracle.window_positions(600, 64, 4)
        assert np.array_equal(r.rows, np.union1d(r.sel.idx, win))
        assert len(r.rows) >= 68
        K = oracle.np_of(lay.K_ret[0, 0]).astype(np.float64)[r.rows]
        V = oracle.np_of(lay.V_ret[0, 0]).astype(np.float64)[r.rows]
        s = K @ oracle.np_of(lay.q)[0, h].astype(np.float64) * wl.scale_attn
        e = np.exp(s - s.max())
        assert np.allclose(r.out, (e[:, None] * V).sum(0) / e.sum(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# prefill: causal attention of a prompt and the decode state it leaves
# ---------------------------------------------------------------------------
def _masked_attention_matrix(q, K, V, scale, allowed):
    """Textbook masked attention in fp64: scores q K^T * scale, -inf where not allowed,
    row softmax, times V (numpy matrix form, one call for every query)."""
    S = q.astype(np.float64) @ K.astype(np.float64).T * scale
    S = np.where(allowed, S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    return P @ V.astype(np.float64)


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_prefill_is_masked_dense_attention(dt):
    rng = np.random.default_rng(21)
    B, Hq, Hkv, L, d, window, sinks = 1, 4, 2, 150, 32, 40, 3
    q = rng.standard_normal((B, Hq, L, d)).astype(dt)
    K = rng.standard_normal((B, Hkv, L, d)).astype(dt)
    V = rng.standard_normal((B, Hkv, L, d)).astype(dt)
    res = oracle.prefill_layer(q, K, V, [1, 0], [L], 0.2, window, sinks)
    t = np.arange(L)[:, None]
    n = np.arange(L)[None, :]
    causal = n <= t
    local = causal & ((n < sinks) | (n > t - window))
    for h in range(Hq):
        allowed = causal if h // 2 == 0 else local
        ref = _masked_attention_matrix(q[0, h], K[0, h // 2], V[0, h // 2], 0.2, allowed)
        got = np.stack([res[(0, h, tt)] for tt in range(L)])
        assert np.max(np.abs(got - ref)) <= 1e-12, h


def test_prefill_last_row_is_the_decode_step():
    """Query position L-1 of a prompt attends exactly like a decode step at length L:
    p = 1 for a retrieval head (every token), the sink + window set for a local head."""
    import workloads
    wl = workloads.make_workload("t", 1, [300], 4, 2, [[1, 0]], seed=5, dtype="f32", p=1.0,
                                 window=64, sinks=4)
    lay = wl.layers[0]
    dec = oracle.decode_step(wl)[0]
    q = np.zeros((1, 4, 300, wl.d), np.float32)
    q[0, :, 299] = oracle.np_of(lay.q)[0]
    Kp = np.zeros((1, 2, 300, wl.d), np.float32)
    Vp = np.zeros((1, 2, 300, wl.d), np.float32)
    Kp[0, 0], Vp[0, 0] = oracle.np_of(lay.K_ret)[0, 0], oracle.np_of(lay.V_ret)[0, 0]
    pos = oracle.window_positions(300, 64, 4)
    slots = oracle.ring_slot(pos, 64, 4)
    Kp[0, 1, pos] = oracle.np_of(lay.K_loc)[0, 0, slots]
    Vp[0, 1, pos] = oracle.np_of(lay.V_loc)[0, 0, slots]
    pre = oracle.prefill_layer(q, Kp, Vp, [1, 0], [300], wl.scale_attn, 64, 4, positions=[299])
    for h in range(4):
        assert np.max(np.abs(pre[(0, h, 299)] - dec[(0, h)].out)) <= 1e-12, h


def test_prefill_state_places_the_prompt():
    rng = np.random.default_rng(22)
    B, Hkv, Lmax, d, r, window, sinks = 2, 2, 20, 4, 2, 6, 2
    K = rng.standard_normal((B, Hkv, Lmax, d)).astype(np.float16)
    V = rng.standard_normal((B, Hkv, Lmax, d)).astype(np.float16)
    k_pre = rng.standard_normal((B, Hkv, Lmax, d)).astype(np.float32)
    Wk = rng.standard_normal((1, d, r)).astype(np.float32)
    k_idx, K_ret, V_ret, K_loc, V_loc = oracle.prefill_state(K, V, k_pre, Wk, [0, 1], [17, 3],
                                                             window, sinks, Lmax)
    # retrieval KV head 1: rows < L copied, k_idx projected; nothing past L
    assert np.array_equal(K_ret[0, 0, :17], K[0, 1, :17]) and not K_ret[0, 0, 17:].any()
    assert np.array_equal(k_idx[1, 0, 2], oracle.project(k_pre[1, 1, 2], Wk[0]).astype(np.float16))
    assert not k_idx[1, 0, 3:].any()
    # local KV head 0 at L = 17: sinks 0, 1 in slots 0, 1; positions 11..16 in 2 + n % 6
    for n in [0, 1]:
        assert np.array_equal(K_loc[0, 0, n], K[0, 0, n])
    for n in range(11, 17):
        assert np.array_equal(V_loc[0, 0, 2 + n % 6], V[0, 0, n])
    # L = 3: only slots 0, 1 (sinks) and 2 + 2 % 6 = 4 are written
    assert [s for s in range(8) if K_loc[1, 0, s].any()] == [0, 1, 4]


def test_prefill_state_bf16_rounds_the_projection():
    # bf16 caches: each k_idx value is a bfloat16 number (low 16 bits of its fp32 zero)
    # within half a bfloat16 ulp (2^-8 relative) of the fp32 projection; K/V rows copy as is
    import workloads
    pr = workloads.make_prompt([9], 2, 2, [1, 0], seed=5, dtype="bf16")
    k_idx, K_ret, _, K_loc, _ = oracle.prefill_state(pr.K, pr.V, pr.k_pre, pr.Wk,
                                                     pr.kv_is_retrieval, [9], 4, 1, 9)
    assert k_idx.dtype == np.float32
    assert not (k_idx.view(np.uint32) & 0xFFFF).any()
    exact = np.stack([oracle.project(oracle.np_of(pr.k_pre)[0, 0, n], oracle.np_of(pr.Wk)[0])
                      for n in range(9)]).astype(np.float64)
    err = np.abs(k_idx[0, 0].astype(np.float64) - exact)
    assert (err <= np.abs(exact) * 2.0 ** -8).all() and err.max() > 0
    assert np.array_equal(K_ret[0, 0], oracle.np_of(pr.K)[0, 0])
    assert np.array_equal(K_loc[0, 0, 0], oracle.np_of(pr.K)[0, 1, 0])


def test_round_bf16_ties_and_library_conversion():
    # 1 + 2^-8 lies halfway between bf16 1 and 1 + 2^-7: ties to even give 1; 1 + 3 * 2^-8
    # lies halfway between 1 + 2^-7 and 1 + 2^-6: ties to even give 1 + 2^-6
    assert oracle.round_bf16([1 + 2 ** -8])[0] == 1.0
    assert oracle.round_bf16([1 + 3 * 2 ** -8])[0] == 1 + 2 ** -6
    assert oracle.round_bf16([-(1 + 3 * 2 ** -8)])[0] == -(1 + 2 ** -6)
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
                        np.array([0.0, 3e-39, -1e-40, 2.0 ** -126, 1e38])]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.round_bf16(x), want)


# ---------------------------------------------------------------------------
# the set rule at a given (A, b*): the form the GPU parity checker falls back to when
# the GPU's top cell or threshold bin differs from the oracle's by a tie
# ---------------------------------------------------------------------------
GOLD_SWB = os.path.join(os.path.dirname(__file__), "golden", "select_with_bstar.json")


def _swb_cases():
    with open(GOLD_SWB) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("ex", _swb_cases(), ids=lambda e: e["name"])
def test_select_with_bstar_worked_examples(ex):
    z = np.array(ex["z"], dtype=np.float32)
    if "cells" in ex:
        assert oracle.cells(z).tolist() == ex["cells"]
    got = oracle.select_with_bstar(z, ex["A"], ex["bstar"])
    assert got.tolist() == ex["S"]
    assert got.dtype == np.int32


@pytest.mark.parametrize("name,z", LOGITS, ids=[n for n, _ in LOGITS])
def test_select_with_bstar_reproduces_the_rule(name, z):
    """At the oracle's own (A, b*), the set must be the C rule's set, for top-p at every p
    of the sweep and for top-k at several budgets; one bin more or less must give the
    nested sets that the bins' definition implies."""
    for p in PS + [1.0]:
        s = oracle.topp_select(z, p)
        got = oracle.select_with_bstar(z, s.A, s.bstar)
        assert np.array_equal(got, s.idx), (name, p)
        # b* + 1 adds exactly the tokens of bin b* + 1 (the tail bin holds everything further)
        if s.bstar < 255:
            up = oracle.select_with_bstar(z, s.A, s.bstar + 1)
            j = np.minimum(s.A - oracle.cells(z), 255)
            assert set(up.tolist()) == set(s.idx.tolist()) | set(np.nonzero(j == s.bstar + 1)[0].tolist())
    for k in (1, 7, 100, 3000):
        s = oracle.topk_select(z, k)
        assert np.array_equal(oracle.select_with_bstar(z, s.A, s.bstar), s.idx), (name, k)
