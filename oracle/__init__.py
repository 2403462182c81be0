"""Plain CPU oracle of one RTPurbo decode step (fp64 masses and attention).

TEST INFRASTRUCTURE.  Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it; both take their inputs from the
``workloads`` generator.

The arithmetic lives in ``rtp_oracle.c`` (plain loops, single thread); this
module converts arrays and walks the heads of a layer:

* retrieval query heads: indexer score -> 256-bin histogram top-p -> exact
  softmax attention over the selected rows (Full Attention Strikes Back,
  xllm-io paper review, section 三 核心公式, the two adaptive-sparse-attention
  equations; section 三 硬件感知解码内核 for the histogram);
* local query heads: exact softmax attention over the 4 sink tokens and the
  last 8192 positions (same page, section 五, test-configuration table;
  gist.science summary, section 1: local heads use a sliding window with
  attention sinks).

Readings taken where the pages are silent (bin grid, threshold bin kept whole,
p >= 1 keeps every token, window includes the current token, a ring slot
layout for local heads) are stated next to the functions that use them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rtp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a build of the same source to load instead (the sanitizer test's instrumented copy)
_LIB_OVERRIDE = os.environ.get("RTP_ORACLE_LIBRARY")
NBINS = 256

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (host only, no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                               "-shared", "-std=c99", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out: str) -> str:
    """The same source under AddressSanitizer and UndefinedBehaviorSanitizer (for a child
    process that preloads libasan and names `out` in RTP_ORACLE_LIBRARY)."""
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
                           "-fno-fast-math", "-fPIC", "-shared", "-std=c99",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-o", out, _SRC, "-lm"])
    return out


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.rtpo_half_to_double.restype = ctypes.c_double
        L.rtpo_half_to_double.argtypes = [ctypes.c_uint16]
        L.rtpo_index_score.restype = None
        L.rtpo_index_score.argtypes = [P, P, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_float, P]
        L.rtpo_topp_select.restype = ctypes.c_int64
        L.rtpo_topp_select.argtypes = [P, ctypes.c_int64, ctypes.c_double, ctypes.c_double, P, P,
                                       P, P]
        L.rtpo_topk_select.restype = ctypes.c_int64
        L.rtpo_topk_select.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, P, P,
                                       P, P]
        L.rtpo_project.restype = None
        L.rtpo_project.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P]
        L.rtpo_round_bf16.restype = ctypes.c_double
        L.rtpo_round_bf16.argtypes = [ctypes.c_double]
        L.rtpo_attention.restype = None
        L.rtpo_attention.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int64,
                                     ctypes.c_double, P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError("oracle takes fp16 or fp32 arrays, got %s" % a.dtype)


def np_of(x) -> np.ndarray:
    """numpy view of a CPU array or torch tensor (no arithmetic; bfloat16 tensors become
    fp32 arrays, which hold every bfloat16 value exactly)."""
    if hasattr(x, "detach"):
        x = x.detach()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.cpu().numpy()
    return np.ascontiguousarray(x)


def round_bf16(x) -> np.ndarray:
    """Each value rounded to bfloat16 (see rtp_oracle.c), as fp32."""
    a = np.asarray(x, dtype=np.float64)
    f = lib().rtpo_round_bf16
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.float32).reshape(a.shape)


def _to_cache(values, like) -> np.ndarray:
    """Values stored into a cache of `like`'s dtype (round to nearest even)."""
    if hasattr(like, "dtype") and str(like.dtype) == "torch.bfloat16":
        return round_bf16(values)
    return np.asarray(values).astype(np_of(like[:0]).dtype if hasattr(like, "detach") else like.dtype)


# ----------------------------------------------------------------------------
# single-purpose functions
# ----------------------------------------------------------------------------
def index_score(q_idx, k_idx, scale: float) -> np.ndarray:
    """z[n] = fl32(scale * fp32-fma-chain(q_idx, k_idx[n])) for k_idx [L, r]."""
    q = np.ascontiguousarray(q_idx, dtype=np.float32)
    k = np.ascontiguousarray(k_idx)
    L, r = k.shape
    assert q.shape == (r,)
    z = np.empty(L, dtype=np.float32)
    kk = k.view(np.uint16) if k.dtype == np.float16 else k
    lib().rtpo_index_score(_ptr(q), _ptr(kk), _dtype_code(k), L, r, ctypes.c_float(scale), _ptr(z))
    return z


@dataclass
class Selection:
    idx: np.ndarray       # ascending int32 token indices
    hist: np.ndarray      # [256] fp64 bin masses relative to exp((A+1) w)
    A: int                # top occupied cell
    bstar: int            # threshold bin

    @property
    def count(self) -> int:
        return int(self.idx.shape[0])


def topp_select(z, p: float, bin_width: float = 0.125) -> Selection:
    """256-bin histogram top-p over one head's logits z[0:L] (see rtp_oracle.c)."""
    zz = np.ascontiguousarray(z, dtype=np.float32)
    L = zz.shape[0]
    assert L >= 1 and np.all(np.isfinite(zz)), "oracle requires L >= 1 and finite logits"
    sel = np.empty(L, dtype=np.int32)
    hist = np.empty(NBINS, dtype=np.float64)
    A = ctypes.c_int64()
    b = ctypes.c_int32()
    n = lib().rtpo_topp_select(_ptr(zz), L, float(p), float(bin_width), _ptr(sel), _ptr(hist),
                               ctypes.byref(A), ctypes.byref(b))
    return Selection(sel[:n].copy(), hist, int(A.value), int(b.value))


def topk_select(z, k: int, bin_width: float = 0.125) -> Selection:
    """Fixed top-k through the same 256-bin histogram: every token weighs one, b* is
    the least bin whose cumulative count reaches k (see rtp_oracle.c).  `hist` holds
    the counts."""
    zz = np.ascontiguousarray(z, dtype=np.float32)
    L = zz.shape[0]
    assert L >= 1 and np.all(np.isfinite(zz)), "oracle requires L >= 1 and finite logits"
    assert int(k) >= 1, "top-k needs k >= 1"
    sel = np.empty(L, dtype=np.int32)
    hist = np.empty(NBINS, dtype=np.float64)
    A = ctypes.c_int64()
    b = ctypes.c_int32()
    n = lib().rtpo_topk_select(_ptr(zz), L, int(k), float(bin_width), _ptr(sel), _ptr(hist),
                               ctypes.byref(A), ctypes.byref(b))
    return Selection(sel[:n].copy(), hist, int(A.value), int(b.value))


def project(x, W) -> np.ndarray:
    """Indexer projection of one pre-RoPE vector x [d] by W [d, r]: an fp32 fma chain
    over the d inputs in order, per output feature (see rtp_oracle.c)."""
    xx = np.ascontiguousarray(x, dtype=np.float32)
    WW = np.ascontiguousarray(W, dtype=np.float32)
    d, r = WW.shape
    assert xx.shape == (d,)
    out = np.empty(r, dtype=np.float32)
    lib().rtpo_project(_ptr(xx), _ptr(WW), d, r, _ptr(out))
    return out


def append_project(layer, new_lens, q_pre, k_pre, k_new, v_new, Wq, Wk, window: int,
                   sinks: int):
    """One decode step's cache update, on numpy copies of a layer's arrays.

    Per sequence b whose length after the step is L = new_lens[b] >= 1 (the new token
    sits at position n = L - 1):
      * q_idx[b, h] = project(q_pre[b, h], Wq[h]) for every query head of a retrieval KV
        head (other rows keep their values);
      * retrieval KV head kr: k_idx[b, kr, n] = fl16(project(k_pre[b, kv], Wk[kr])) in
        the cache's dtype, K_ret/V_ret[b, kr, n] = k_new/v_new[b, kv];
      * local KV head: K_loc/V_loc[b, kl, ring_slot(n)] = k_new/v_new[b, kv].
    Returns the updated (q_idx, k_idx, K_ret, V_ret, K_loc, V_loc)."""
    mask = np.asarray(layer.kv_is_retrieval)
    ret = [int(h) for h in np.nonzero(mask)[0]]
    loc = [int(h) for h in np.nonzero(mask == 0)[0]]
    q_idx, k_idx = np_of(layer.q_idx).copy(), np_of(layer.k_idx).copy()
    K_ret, V_ret = np_of(layer.K_ret).copy(), np_of(layer.V_ret).copy()
    K_loc, V_loc = np_of(layer.K_loc).copy(), np_of(layer.V_loc).copy()
    q_pre, k_pre = np_of(q_pre), np_of(k_pre)
    k_new, v_new = np_of(k_new), np_of(v_new)
    Wq, Wk = np_of(Wq), np_of(Wk)
    Hkv = mask.shape[0]
    G = q_idx.shape[1] // Hkv
    for b, L in enumerate(np.asarray(new_lens).tolist()):
        if L < 1:
            continue
        n = L - 1
        for kr, kv in enumerate(ret):
            for g in range(G):
                h = kv * G + g
                q_idx[b, h] = project(q_pre[b, h], Wq[h])
            k_idx[b, kr, n] = _to_cache(project(k_pre[b, kv], Wk[kr]), layer.k_idx)
            K_ret[b, kr, n] = k_new[b, kv]
            V_ret[b, kr, n] = v_new[b, kv]
        for kl, kv in enumerate(loc):
            slot = int(ring_slot(np.array([n]), window, sinks)[0])
            K_loc[b, kl, slot] = k_new[b, kv]
            V_loc[b, kl, slot] = v_new[b, kv]
    return q_idx, k_idx, K_ret, V_ret, K_loc, V_loc


def cells(z, bin_width: float = 0.125) -> np.ndarray:
    """g_n = floor(z_n / w) (exact for a power-of-two w)."""
    return np.floor(np.asarray(z, dtype=np.float32).astype(np.float64) / bin_width).astype(np.int64)


def select_with_bstar(z, A: int, bstar: int, bin_width: float = 0.125) -> np.ndarray:
    """The rule's set for a given (A, b*): { n : min(A - g_n, 255) <= b* }."""
    j = np.minimum(A - cells(z, bin_width), NBINS - 1)
    return np.nonzero(j <= bstar)[0].astype(np.int32)


def attention(q, K, V, rows, scale: float):
    """fp64 softmax attention of q [d] over rows of K, V ([N, d], fp16 or fp32)."""
    qq = np.ascontiguousarray(np.asarray(q).astype(np.float64))
    KK = np.ascontiguousarray(K)
    VV = np.ascontiguousarray(V)
    assert KK.dtype == VV.dtype
    d = KK.shape[-1]
    rr = np.ascontiguousarray(rows, dtype=np.int64)
    assert rr.size >= 1
    out = np.empty(d, dtype=np.float64)
    lse = ctypes.c_double()
    kv = (lambda a: a.view(np.uint16)) if KK.dtype == np.float16 else (lambda a: a)
    lib().rtpo_attention(_ptr(qq), _ptr(kv(KK)), _ptr(kv(VV)), _dtype_code(KK), d, _ptr(rr),
                         rr.size, float(scale), _ptr(out), ctypes.byref(lse))
    return out, float(lse.value)


def window_positions(L: int, window: int, sinks: int) -> np.ndarray:
    """Positions a local head attends to: the first `sinks` positions and the last
    `window` positions (the current token included), each counted once."""
    first = np.arange(min(sinks, L), dtype=np.int64)
    rest = np.arange(max(sinks, L - window), L, dtype=np.int64)
    return np.concatenate([first, rest])


def ring_slot(pos: np.ndarray, window: int, sinks: int) -> np.ndarray:
    """Ring layout of a local head's cache: sink position n < sinks in slot n, any later
    position n in slot sinks + (n mod window)."""
    pos = np.asarray(pos, dtype=np.int64)
    return np.where(pos < sinks, pos, sinks + pos % window)


# ----------------------------------------------------------------------------
# one decode step over a layer
# ----------------------------------------------------------------------------
@dataclass
class HeadResult:
    out: np.ndarray
    lse: float
    sel: Optional[Selection] = None
    z: Optional[np.ndarray] = None     # indexer logits of a retrieval head
    rows: Optional[np.ndarray] = None  # the rows attended to (retrieval heads)


def decode_layer(layer, seq_lens, Hq: int, Hkv: int, p: float, bin_width: float,
                 scale_idx: float, scale_attn: float, window: int, sinks: int,
                 heads: Optional[List[int]] = None, batches: Optional[List[int]] = None,
                 topk: int = 0, ret_window: bool = False) -> Dict[tuple, HeadResult]:
    """Oracle outputs of one layer keyed by (b, query head).  `heads` / `batches`
    restrict the work to a sample of query heads / sequences.  topk > 0 selects with
    the fixed top-k rule instead of top-p.  ret_window: retrieval heads attend to their
    selected set united with the sink and window positions (rows of the full cache)."""
    G = Hq // Hkv
    mask = np.asarray(layer.kv_is_retrieval)
    ret = [int(h) for h in np.nonzero(mask)[0]]
    loc = [int(h) for h in np.nonzero(mask == 0)[0]]
    q = np_of(layer.q)
    q_idx = np_of(layer.q_idx)
    res = {}
    B = len(seq_lens)
    for b in (batches if batches is not None else range(B)):
        L = int(seq_lens[b])
        for kh in range(Hkv):
            hs = [kh * G + g for g in range(G) if heads is None or kh * G + g in heads]
            if not hs:
                continue
            if mask[kh]:
                kr = ret.index(kh)
                kidx = np_of(layer.k_idx[b, kr, :L])
                Kh = np_of(layer.K_ret[b, kr, :L])
                Vh = np_of(layer.V_ret[b, kr, :L])
                for h in hs:
                    z = index_score(q_idx[b, h], kidx, scale_idx)
                    s = topk_select(z, topk, bin_width) if topk > 0 else topp_select(z, p, bin_width)
                    rows = s.idx
                    if ret_window:
                        rows = np.union1d(rows, window_positions(L, window, sinks))
                    o, lse = attention(q[b, h], Kh, Vh, rows, scale_attn)
                    res[(b, h)] = HeadResult(o, lse, s, z, np.asarray(rows, dtype=np.int64))
            else:
                kl = loc.index(kh)
                rows = ring_slot(window_positions(L, window, sinks), window, sinks)
                Kh = np_of(layer.K_loc[b, kl])
                Vh = np_of(layer.V_loc[b, kl])
                for h in hs:
                    o, lse = attention(q[b, h], Kh, Vh, rows, scale_attn)
                    res[(b, h)] = HeadResult(o, lse, None)
    return res


# ----------------------------------------------------------------------------
# prefill of a prompt (dense causal attention for retrieval heads, causal window +
# sinks for local heads) and the decode state it leaves
# ----------------------------------------------------------------------------
def prefill_rows(t: int, retrieval: bool, window: int, sinks: int) -> np.ndarray:
    """Keys query position t attends to: every n <= t (retrieval heads), or the first
    `sinks` positions and the last `window` positions up to t (local heads: the decode
    window of a sequence of length t + 1)."""
    if retrieval:
        return np.arange(t + 1, dtype=np.int64)
    return window_positions(t + 1, window, sinks)


def prefill_layer(q, K, V, kv_is_retrieval, seq_lens, scale: float, window: int, sinks: int,
                  heads: Optional[List[int]] = None, positions: Optional[List[int]] = None):
    """Prefill attention outputs {(b, h, t): out [d] fp64} for q [B, Hq, Lmax, d] and
    K, V [B, Hkv, Lmax, d] (fp16 or fp32), query head h on KV head h // G.  `heads` /
    `positions` restrict the work to a sample."""
    qn, Kn, Vn = np_of(q), np_of(K), np_of(V)
    B, Hq = qn.shape[0], qn.shape[1]
    Hkv = Kn.shape[1]
    G = Hq // Hkv
    mask = np.asarray(kv_is_retrieval)
    res = {}
    for b in range(B):
        L = int(seq_lens[b])
        for h in (heads if heads is not None else range(Hq)):
            kv = h // G
            for t in (positions if positions is not None else range(L)):
                if t >= L:
                    continue
                rows = prefill_rows(t, bool(mask[kv]), window, sinks)
                o, _ = attention(qn[b, h, t], Kn[b, kv], Vn[b, kv], rows, scale)
                res[(b, h, t)] = o
    return res


def prefill_state(K, V, k_pre, Wk, kv_is_retrieval, seq_lens, window: int, sinks: int,
                  Lmax: int):
    """The decode state a prompt leaves: for retrieval KV head kv (the kr-th flagged),
    k_idx[b, kr, n] = project(k_pre[b, kv, n], Wk[kr]) rounded to K's dtype (nearest even;
    bfloat16 tensors give fp32 arrays of bfloat16 values) and the K/V rows
    copied for every n < L; for local KV heads the ring [sinks + window] holding the
    positions of window_positions(L) at their ring slots (other slots zero)."""
    Kn, Vn, kp, W = np_of(K), np_of(V), np_of(k_pre), np_of(Wk)
    mask = np.asarray(kv_is_retrieval)
    ret = [int(h) for h in np.nonzero(mask)[0]]
    loc = [int(h) for h in np.nonzero(mask == 0)[0]]
    B, d = Kn.shape[0], Kn.shape[-1]
    r = W.shape[-1]
    k_idx = np.zeros((B, len(ret), Lmax, r), Kn.dtype)
    K_ret = np.zeros((B, len(ret), Lmax, d), Kn.dtype)
    V_ret = np.zeros((B, len(ret), Lmax, d), Kn.dtype)
    K_loc = np.zeros((B, len(loc), sinks + window, d), Kn.dtype)
    V_loc = np.zeros((B, len(loc), sinks + window, d), Kn.dtype)
    for b in range(B):
        L = int(seq_lens[b])
        for kr, kv in enumerate(ret):
            for n in range(L):
                k_idx[b, kr, n] = _to_cache(project(kp[b, kv, n], W[kr]), K)
            K_ret[b, kr, :L] = Kn[b, kv, :L]
            V_ret[b, kr, :L] = Vn[b, kv, :L]
        pos = window_positions(L, window, sinks)
        slots = ring_slot(pos, window, sinks)
        for kl, kv in enumerate(loc):
            K_loc[b, kl, slots] = Kn[b, kv, pos]
            V_loc[b, kl, slots] = Vn[b, kv, pos]
    return k_idx, K_ret, V_ret, K_loc, V_loc


def decode_step(wl, layers: Optional[List[int]] = None, heads=None, batches=None):
    """Oracle outputs for a whole workload: list (per layer) of {(b, h): HeadResult}."""
    out = []
    for li, layer in enumerate(wl.layers):
        if layers is not None and li not in layers:
            out.append({})
            continue
        out.append(decode_layer(layer, wl.seq_lens, wl.Hq, wl.Hkv, wl.p, wl.bin_width,
                                wl.scale_idx, wl.scale_attn, wl.window, wl.sinks, heads, batches,
                                getattr(wl, "topk", 0), getattr(wl, "ret_window", False)))
    return out
