"""Seeded synthetic inputs for one RTPurbo decode step.

This module builds inputs only: the query/key/value tensors, the 16-dim indexer
features and the sequence lengths.  It computes no score, histogram, selection
or attention, so both the CPU oracle and the HIP path can take their inputs from
here without sharing any of the method's arithmetic.

What the inputs imitate (Full Attention Strikes Back, xllm-io paper review):
  * head-wise split: a few retrieval KV heads keep the whole cache, the rest are
    local heads with an 8192-token window and 4 sink tokens (section 五, the
    test-configuration table);
  * query classes whose indexer-softmax mass is concentrated on 2 tokens
    (section 三, insight 3, figure 3(b)), spread over ~500 tokens (section 五,
    the layer-25 dynamic-sparsity table) or broad, ~8.5k tokens for 90% of the
    mass (section 三, the top-k vs top-p table).

Planted-logit construction (retrieval heads).  A seeded 16x16 orthogonal matrix
U gives one direction u_g per query head g of a KV head; the remaining columns
span the complement.  With q_idx[g] = a*u_g (a = 8) and
k_idx[n] = sum_g z[n,g]/(tau*a) * u_g + sum_{j>=G} eps[n,j] * u_j
(tau = 1/4, eps ~ N(0,1)), the indexer logit tau * q_idx[g].k_idx[n] equals the
chosen target z[n,g] up to the fp16 rounding of k_idx.  Targets: background
z ~ N(mu_bg, 1); k planted positions (uniform, without replacement) carry the
class's logits, sized so that the planted tokens hold a share f = 0.93 of the
expected softmax mass.

Large K/V/q tensors use a counter-based generator: element i of stream s under
seed S is T[h(S, s, i) >> 16], where h is a 32-bit integer hash (Chris
Wellons' "lowbias32" finalizer, applied twice) and T holds the 65536 standard
normal quantiles Phi^-1((k + 0.5)/65536) rounded to fp16.  Only integer
arithmetic and a table lookup are involved, so CPU and GPU produce identical
values for any slice.

Notation N(mu, v) in the configuration text gives the *variance* v.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

M32 = 0xFFFFFFFF
PLANTED_SHARE = 0.93      # f: planted share of the expected softmax mass
INDEX_AMPLITUDE = 8.0     # a: |q_idx| per query head in the planted construction
INDEX_TAU = 0.25          # 1/sqrt(16): the indexer softmax temperature the targets assume
WINDOW = 8192
SINKS = 4

# ----------------------------------------------------------------------------
# counter-based fp16 normals
# ----------------------------------------------------------------------------
_TABLE_CACHE = {}


def normal_table_f16() -> np.ndarray:
    """The 65536 standard-normal quantiles at (k+0.5)/65536, as fp16."""
    if "t" not in _TABLE_CACHE:
        from scipy.special import ndtri
        u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _TABLE_CACHE["t"] = ndtri(u).astype(np.float16)
    return _TABLE_CACHE["t"]


def _mul32_t(x: torch.Tensor, c: int) -> torch.Tensor:
    # (x * c) mod 2^32 for int64 x in [0, 2^32), without leaving int64 range.
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + ((hi * c) & 0xFFFF) * 65536) & M32


def _mix32_t(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32_t(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32_t(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix32_i(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def counter_normal_f16(shape: Sequence[int], seed: int, stream: int,
                       device="cpu", slice_elems: int = 1 << 26) -> torch.Tensor:
    """fp16 N(0,1) tensor; element i depends only on (seed, stream, i)."""
    n = int(np.prod(shape)) if len(shape) else 1
    table = torch.from_numpy(normal_table_f16().view(np.int16)).to(device)
    out = torch.empty(n, dtype=torch.int16, device=device)
    k1 = _mix32_i(seed * 0x9E3779B1 + stream * 0x85EBCA77 + 0x165667B1)
    k2 = _mix32_i(k1 ^ 0xC2B2AE3D)
    for s in range(0, n, slice_elems):
        e = min(n, s + slice_elems)
        i = torch.arange(s, e, dtype=torch.int64, device=device)
        h = _mix32_t((i & M32) ^ k1)
        h = _mix32_t(h ^ (((i >> 32) + k2) & M32))
        out[s:e] = table[h >> 16]
    return out.view(torch.float16).view(*shape)


# ----------------------------------------------------------------------------
# workload description
# ----------------------------------------------------------------------------
@dataclass
class HeadPlan:
    """What was planted for one retrieval query head (for reporting only)."""
    cls: str
    k: int
    positions: np.ndarray


@dataclass
class Layer:
    kv_is_retrieval: np.ndarray            # [Hkv] uint8
    q: torch.Tensor                        # [B, Hq, d]   kv dtype
    q_idx: torch.Tensor                    # [B, Hq, r]   fp32 (rows of local heads unused)
    k_idx: torch.Tensor                    # [B, Hret, Lmax, r]
    K_ret: torch.Tensor                    # [B, Hret, Lmax, d]
    V_ret: torch.Tensor
    K_loc: torch.Tensor                    # [B, Hloc, sinks + window, d] ring
    V_loc: torch.Tensor
    plans: dict = field(default_factory=dict)   # (b, query head) -> HeadPlan

    @property
    def ret_heads(self) -> List[int]:
        return [int(h) for h in np.nonzero(self.kv_is_retrieval)[0]]

    @property
    def loc_heads(self) -> List[int]:
        return [int(h) for h in np.nonzero(self.kv_is_retrieval == 0)[0]]


@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    r: int
    Lmax: int
    seq_lens: np.ndarray                   # [B] int32
    window: int
    sinks: int
    dtype: str                             # "f16" | "bf16" | "f32"  (K, V, q, k_idx)
    p: float
    bin_width: float
    scale_idx: float
    scale_attn: float
    layers: List[Layer]
    seed: int = 0
    topk: int = 0                          # > 0: fixed top-k selection instead of top-p
    ret_window: bool = False               # retrieval heads also attend to sinks + window

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def to(self, device) -> "Workload":
        ls = []
        for l in self.layers:
            ls.append(Layer(l.kv_is_retrieval, l.q.to(device), l.q_idx.to(device),
                            l.k_idx.to(device), l.K_ret.to(device), l.V_ret.to(device),
                            l.K_loc.to(device), l.V_loc.to(device), l.plans))
        w = Workload(**{k: getattr(self, k) for k in self.__dataclass_fields__ if k != "layers"},
                     layers=ls)
        return w


# ----------------------------------------------------------------------------
# planted logit targets
# ----------------------------------------------------------------------------
def _orthogonal16(rng: np.random.Generator, r: int) -> np.ndarray:
    m = rng.standard_normal((r, r))
    qm, rm = np.linalg.qr(m)
    return qm * np.sign(np.diag(rm))[None, :]


def _targets(rng: np.random.Generator, L: int, cls: str, k: int):
    """Target logits z[0:L] for one query head; returns (z, positions)."""
    f = PLANTED_SHARE
    odds = f / (1.0 - f)
    if L == 0:
        return np.zeros(0), np.zeros(0, dtype=np.int64)
    k = max(1, min(k, L))
    if cls in ("concentrated", "needle"):
        z = rng.standard_normal(L)
        pos = np.sort(rng.choice(L, k, replace=False))
        z[pos] = math.log(odds * L * math.exp(0.5) / k)
    elif cls == "mid":
        z = rng.standard_normal(L)
        pos = np.sort(rng.choice(L, k, replace=False))
        delta = math.log(odds * L * math.exp(0.5) / (k * math.exp(0.25)))
        z[pos] = delta + math.sqrt(0.5) * rng.standard_normal(k)
    elif cls == "broad":
        mu_bg = 1.75 + math.log(k / (odds * L))
        z = mu_bg + rng.standard_normal(L)
        pos = np.sort(rng.choice(L, k, replace=False))
        z[pos] = 2.0 + math.sqrt(0.5) * rng.standard_normal(k)
    elif cls == "gaussian":
        z = 3.0 * rng.standard_normal(L)
        pos = np.zeros(0, dtype=np.int64)
    else:
        raise ValueError(cls)
    return z, pos


def _class_k(rng: np.random.Generator, cls: str, L: int, fixed: Optional[int]) -> int:
    if fixed is not None:
        return fixed
    if cls == "concentrated":
        return int(rng.integers(2, 9))
    if cls == "broad":
        return int(min(L // 2, rng.integers(4000, 8001))) if L > 16000 else max(1, L // 10)
    if cls == "mid":
        return min(500, max(1, L // 20))
    if cls == "needle":
        return 2
    return 0


def _build_index(rng, Ls, Lmax, G, r, classes_per_b, fixed_k, dtype_np, poison):
    """k_idx [B, Lmax, r] and q_idx [B, G, r] for one retrieval KV head."""
    B = len(Ls)
    U = _orthogonal16(rng, r)
    # at most r heads get planted targets (one direction each); with G > r the remaining
    # heads reuse the directions cyclically and see whatever logits those give
    Gp = min(G, r)
    kidx = np.zeros((B, Lmax, r), dtype=dtype_np)
    qidx = np.zeros((B, G, r), dtype=np.float32)
    plans = {}
    for b in range(B):
        L = int(Ls[b])
        Z = np.zeros((L, Gp))
        for g in range(Gp):
            cls = classes_per_b[b][g]
            k = _class_k(rng, cls, L, fixed_k.get(cls) if fixed_k else None)
            z, pos = _targets(rng, L, cls, k)
            Z[:, g] = z
            plans[(b, g)] = HeadPlan(cls, len(pos), pos)
        eps = rng.standard_normal((L, r - Gp))
        kv = (Z / (INDEX_TAU * INDEX_AMPLITUDE)) @ U[:, :Gp].T + eps @ U[:, Gp:].T
        kidx[b, :L] = kv.astype(dtype_np)
        if poison and L < Lmax:
            kidx[b, L:] = dtype_np(30000.0) if dtype_np == np.float16 else dtype_np(1e30)
        qidx[b] = (INDEX_AMPLITUDE * U[:, np.arange(G) % r].T).astype(np.float32)
    return kidx, qidx, plans


# ----------------------------------------------------------------------------
# generic builder
# ----------------------------------------------------------------------------
def make_layer(seed: int, layer_id: int, B: int, seq_lens, Lmax: int, Hq: int, Hkv: int,
               kv_is_retrieval, d: int = 128, r: int = 16, dtype: str = "f16",
               window: int = WINDOW, sinks: int = SINKS, classes=None, fixed_k=None,
               device="cpu", poison: bool = True, rng: Optional[np.random.Generator] = None) -> Layer:
    """One attention layer of seeded synthetic decode inputs.

    classes: callable (b, kv_head_rank, rng) -> list of G class names, or None for the
    half-concentrated / half-broad mix.
    """
    G = Hq // Hkv
    mask = np.asarray(kv_is_retrieval, dtype=np.uint8)
    ret = [int(h) for h in np.nonzero(mask)[0]]
    loc = [int(h) for h in np.nonzero(mask == 0)[0]]
    rng = rng if rng is not None else np.random.default_rng(seed * 7919 + layer_id)
    tdt = {"f16": torch.float16, "f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    ndt = np.float16 if dtype == "f16" else np.float32   # bf16 keys are rounded on assignment
    base = 1000 * layer_id

    # attention tensors from the counter-based generator (bf16: its fp16 values rounded)
    def cn(shape, stream):
        t = counter_normal_f16(shape, seed, base + stream, device)
        return t if tdt == torch.float16 else t.to(tdt)

    q = cn((B, Hq, d), 1)
    K_ret = cn((B, len(ret), Lmax, d), 2)
    V_ret = cn((B, len(ret), Lmax, d), 3)
    ring = sinks + window
    K_loc = cn((B, len(loc), ring, d), 4)
    V_loc = cn((B, len(loc), ring, d), 5)
    if poison:
        nanv = float("nan")
        for b in range(B):
            L = int(seq_lens[b])
            if L < Lmax:
                K_ret[b, :, L:] = nanv
                V_ret[b, :, L:] = nanv
            # ring slots that hold no position of the window set
            used = np.zeros(ring, dtype=bool)
            used[:min(sinks, L)] = True
            for n in range(max(sinks, L - window), L):
                used[sinks + (n % window)] = True
            if not used.all():
                idx = torch.from_numpy(np.nonzero(~used)[0]).to(device)
                K_loc[b, :, idx] = nanv
                V_loc[b, :, idx] = nanv

    k_idx = torch.zeros((B, len(ret), Lmax, r), dtype=tdt)
    q_idx = torch.zeros((B, Hq, r), dtype=torch.float32)
    plans = {}
    for ki, h in enumerate(ret):
        cl = [classes(b, ki, rng) if classes else
              ["concentrated"] * (G // 2) + ["broad"] * (G - G // 2) for b in range(B)]
        kx, qx, pl = _build_index(rng, seq_lens, Lmax, G, r, cl, fixed_k, ndt, poison)
        k_idx[:, ki] = torch.from_numpy(kx)
        q_idx[:, h * G:(h + 1) * G] = torch.from_numpy(qx)
        for (b, g), v in pl.items():
            plans[(b, h * G + g)] = v
    return Layer(mask, q, q_idx.to(device), k_idx.to(device), K_ret, V_ret, K_loc, V_loc, plans)


def make_workload(name: str, B: int, seq_lens, Hq: int, Hkv: int, kv_masks, seed: int = 0,
                  d: int = 128, r: int = 16, dtype: str = "f16", p: float = 0.9,
                  window: int = WINDOW, sinks: int = SINKS, classes=None, fixed_k=None,
                  device="cpu", poison: bool = True, Lmax: Optional[int] = None,
                  bin_width: float = 0.125) -> Workload:
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    Lmax = int(Lmax if Lmax is not None else seq_lens.max())
    rng = np.random.default_rng(seed)
    layers = [make_layer(seed, li, B, seq_lens, Lmax, Hq, Hkv, m, d, r, dtype, window, sinks,
                         classes, fixed_k, device, poison, rng) for li, m in enumerate(kv_masks)]
    return Workload(name, B, Hq, Hkv, d, r, Lmax, seq_lens, window, sinks, dtype, p, bin_width,
                    1.0 / math.sqrt(r), 1.0 / math.sqrt(d), layers, seed)


# ----------------------------------------------------------------------------
# the five named configurations
# ----------------------------------------------------------------------------
def make_c0(device="cpu", p: float = 0.9) -> Workload:
    """Single head, L=4096, d=128, r=16, fp32; q_idx = 4 * (sum of 8 planted k_idx rows)
    + N(0, 0.1) noise; K, V, k_idx, q ~ N(0, 1).  Seed 0; draws in this order:
    K, V, k_idx, planted rows, noise, q, W^Q_idx, W^K_idx (the last two are drawn for
    completeness and are not used by the decode step)."""
    rng = np.random.default_rng(0)
    L, d, r = 4096, 128, 16
    K = rng.standard_normal((L, d)).astype(np.float32)
    V = rng.standard_normal((L, d)).astype(np.float32)
    kidx = rng.standard_normal((L, r)).astype(np.float32)
    planted = rng.choice(L, 8, replace=False)
    noise = rng.standard_normal(r) * math.sqrt(0.1)
    qidx = (4.0 * kidx[planted].astype(np.float64).sum(0) + noise).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    _wq = rng.standard_normal((d, r)) * math.sqrt(1.0 / 128)
    _wk = rng.standard_normal((d, r)) * math.sqrt(1.0 / 128)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    lay = Layer(np.array([1], dtype=np.uint8), t(q.reshape(1, 1, d)), t(qidx.reshape(1, 1, r)),
                t(kidx.reshape(1, 1, L, r)), t(K.reshape(1, 1, L, d)), t(V.reshape(1, 1, L, d)),
                torch.zeros((1, 0, SINKS + WINDOW, d), dtype=torch.float32, device=device),
                torch.zeros((1, 0, SINKS + WINDOW, d), dtype=torch.float32, device=device),
                {(0, 0): HeadPlan("planted8", 8, np.sort(planted))})
    return Workload("c0", 1, 1, 1, d, r, L, np.array([L], dtype=np.int32), WINDOW, SINKS, "f32",
                    p, 0.125, 0.25, 1.0 / math.sqrt(d), [lay], 0)


def make_c1(device="cpu", p: float = 0.9, L: int = 65536, dtype: str = "f16") -> Workload:
    """One layer, B=1, L=64K, 32 q heads / 4 KV heads; KV head 0 retrieval (q heads 0-3
    concentrated, 4-7 broad), KV heads 1-3 local.  Seed 1."""
    return make_workload("c1", 1, [L], 32, 4, [[1, 0, 0, 0]], seed=1, p=p, device=device,
                         dtype=dtype)


def make_c2(device="cpu", p: float = 0.9, L: int = 131072, B: int = 8,
            dtype: str = "f16") -> Workload:
    """One layer, B=8, L=128K each, KV head 0 retrieval; per sequence b a generator seeded
    2000+b picks which 4 of the 8 query heads are concentrated (the rest broad)."""
    def classes(b, ki, _rng):
        rb = np.random.default_rng(2000 + b)
        conc = set(rb.permutation(8)[:4].tolist())
        return ["concentrated" if g in conc else "broad" for g in range(8)]
    return make_workload("c2", B, [L] * B, 32, 4, [[1, 0, 0, 0]], seed=2, p=p, device=device,
                         classes=classes, dtype=dtype)


def c3_masks(layers: int = 48, hkv: int = 4, n_ret: int = 29, seed: int = 3):
    rng = np.random.default_rng(seed)
    chosen = set(rng.choice(layers * hkv, n_ret, replace=False).tolist())
    return [[1 if l * hkv + h in chosen else 0 for h in range(hkv)] for l in range(layers)]


def make_c3(device="cpu", p: float = 0.9, L: int = 524288, layers: int = 48) -> Workload:
    """48 layers, B=1, L=512K, 32/4 heads per layer; 29 of the 192 KV heads are retrieval
    heads chosen by a generator seeded 3; class mix as in the 64K config."""
    return make_workload("c3", 1, [L], 32, 4, c3_masks(layers), seed=3, p=p, device=device)


def make_c4(device="cpu", p: float = 0.9, L: int = 1048576, dtype: str = "f16") -> Workload:
    """One layer, B=1, L=1M, KV head 0 retrieval: q heads 0-1 needle (2 tokens), 2-5 mid
    (~500 tokens), 6-7 broad (~8.5k tokens, logits N(2, 0.5)).  Seed 4."""
    def classes(b, ki, _rng):
        return ["needle"] * 2 + ["mid"] * 4 + ["broad"] * 2
    return make_workload("c4", 1, [L], 32, 4, [[1, 0, 0, 0]], seed=4, p=p, device=device,
                         classes=classes, fixed_k={"needle": 2, "mid": 500, "broad": 8500},
                         dtype=dtype)


@dataclass
class StepInputs:
    """The new token of one decode step: pre-RoPE vectors for the indexer projections,
    the projection weights and the new K/V rows."""
    q_pre: torch.Tensor   # [B, Hq, d] fp32
    k_pre: torch.Tensor   # [B, Hkv, d] fp32
    Wq: torch.Tensor      # [Hq, d, r] fp32, N(0, 1/d)
    Wk: torch.Tensor      # [Hret, d, r] fp32, N(0, 1/d)
    k_new: torch.Tensor   # [B, Hkv, d] cache dtype
    v_new: torch.Tensor


def make_step_inputs(wl: Workload, layer_id: int = 0, seed: int = 0, device="cpu") -> StepInputs:
    """Seeded N(0, 1) pre-RoPE vectors and new K/V rows; projection weights N(0, 1/d) as in
    the single-head config's W^Q_idx / W^K_idx.  Draw order: q_pre, k_pre, Wq, Wk, k_new,
    v_new."""
    rng = np.random.default_rng(10_000 + 97 * seed + layer_id)
    nret = int(np.asarray(wl.layers[layer_id].kv_is_retrieval).sum())
    B, Hq, Hkv, d, r = wl.B, wl.Hq, wl.Hkv, wl.d, wl.r
    kv = np.float16 if wl.dtype == "f16" else np.float32
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    tkv = (lambda a: t(a).to(torch.bfloat16)) if wl.dtype == "bf16" else t
    q_pre = rng.standard_normal((B, Hq, d)).astype(np.float32)
    k_pre = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    Wq = (rng.standard_normal((Hq, d, r)) * math.sqrt(1.0 / d)).astype(np.float32)
    Wk = (rng.standard_normal((max(nret, 1), d, r)) * math.sqrt(1.0 / d)).astype(np.float32)
    k_new = rng.standard_normal((B, Hkv, d)).astype(kv)
    v_new = rng.standard_normal((B, Hkv, d)).astype(kv)
    return StepInputs(t(q_pre), t(k_pre), t(Wq), t(Wk), tkv(k_new), tkv(v_new))


def make_embedding_step_inputs(wl: Workload, layer_id: int = 0, device="cpu") -> StepInputs:
    """Step inputs that reproduce the workload's own state: q_pre and k_pre carry the
    existing q_idx and the k_idx row at position L-1 in their first r entries (zeros
    after), the weights embed those entries by the identity, and k_new / v_new are the
    K/V rows already at position L-1.  A cache update with these inputs rewrites the
    values the caches already hold, so a timed step sees the planted selection."""
    lay = wl.layers[layer_id]
    mask = np.asarray(lay.kv_is_retrieval)
    ret = [int(h) for h in np.nonzero(mask)[0]]
    loc = [int(h) for h in np.nonzero(mask == 0)[0]]
    B, Hq, Hkv, d, r, G = wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.G
    q_idx = lay.q_idx.detach().cpu().numpy()
    q_pre = np.zeros((B, Hq, d), np.float32)
    q_pre[:, :, :r] = q_idx
    k_pre = np.zeros((B, Hkv, d), np.float32)
    kdt = lay.K_ret.dtype if ret else lay.K_loc.dtype
    k_new = torch.zeros((B, Hkv, d), dtype=kdt)
    v_new = torch.zeros((B, Hkv, d), dtype=kdt)
    eye = np.zeros((d, r), np.float32)
    eye[np.arange(r), np.arange(r)] = 1.0
    Wq = np.broadcast_to(eye, (Hq, d, r)).copy()
    Wk = np.broadcast_to(eye, (max(len(ret), 1), d, r)).copy()
    for b in range(B):
        L = int(wl.seq_lens[b])
        if L < 1:
            continue
        n = L - 1
        for kr, kv in enumerate(ret):
            k_pre[b, kv, :r] = lay.k_idx[b, kr, n].detach().float().cpu().numpy()
            k_new[b, kv] = lay.K_ret[b, kr, n].detach().cpu()
            v_new[b, kv] = lay.V_ret[b, kr, n].detach().cpu()
        for kl, kv in enumerate(loc):
            slot = n if n < wl.sinks else wl.sinks + n % wl.window
            k_new[b, kv] = lay.K_loc[b, kl, slot].detach().cpu()
            v_new[b, kv] = lay.V_loc[b, kl, slot].detach().cpu()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return StepInputs(t(q_pre), t(k_pre), t(Wq), t(Wk), k_new.to(device), v_new.to(device))


@dataclass
class Prompt:
    """A prompt for prefill: post-RoPE q/K/V (fp16, counter-based N(0, 1)), pre-RoPE keys
    for the indexer projection (fp32 N(0, 1)) and the projection weights N(0, 1/d)."""
    kv_is_retrieval: np.ndarray   # [Hkv] uint8
    seq_lens: np.ndarray          # [B] int32
    q: torch.Tensor               # [B, Hq, Lmax, d] fp16
    K: torch.Tensor               # [B, Hkv, Lmax, d] fp16
    V: torch.Tensor
    k_pre: torch.Tensor           # [B, Hkv, Lmax, d] fp32
    Wk: torch.Tensor              # [Hret, d, r] fp32


def make_prompt(seq_lens, Hq: int, Hkv: int, mask, seed: int = 0, d: int = 128, r: int = 16,
                device="cpu", Lmax: Optional[int] = None, with_kpre: bool = True,
                dtype: str = "f16") -> Prompt:
    """q, K, V are N(0, 1) draws of the counter generator in fp16; dtype "bf16" converts
    those fp16 values to bfloat16."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    Lmax = int(Lmax if Lmax is not None else seq_lens.max())
    q = counter_normal_f16((B, Hq, Lmax, d), seed, 11, device)
    K = counter_normal_f16((B, Hkv, Lmax, d), seed, 12, device)
    V = counter_normal_f16((B, Hkv, Lmax, d), seed, 13, device)
    if dtype == "bf16":
        q, K, V = q.to(torch.bfloat16), K.to(torch.bfloat16), V.to(torch.bfloat16)
    elif dtype != "f16":
        raise ValueError("prompt dtype must be f16 or bf16")
    nret = int(np.asarray(mask).sum())
    rng = np.random.default_rng(20_000 + seed)
    if with_kpre:
        k_pre = counter_normal_f16((B, Hkv, Lmax, d), seed, 14, device).float()
    else:
        k_pre = torch.zeros((0,), dtype=torch.float32, device=device)
    Wk = torch.from_numpy((rng.standard_normal((max(nret, 1), d, r)) *
                           math.sqrt(1.0 / d)).astype(np.float32)).to(device)
    return Prompt(np.asarray(mask, dtype=np.uint8), seq_lens, q, K, V, k_pre, Wk)


CONFIGS = {"c0": make_c0, "c1": make_c1, "c2": make_c2, "c3": make_c3, "c4": make_c4}


def make_config(name: str, device="cpu", **kw) -> Workload:
    return CONFIGS[name](device=device, **kw)
