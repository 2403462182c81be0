"""MI355X-native RTPurbo decode attention: Python binding of librtp.so.

Argument marshalling only.  Every step of the decode path runs in the HIP kernels
of librtp.so (``csrc/``); PyTorch provides device memory and the current stream.
The names follow the C ABI in ``include/rtp.h``:

* ``rtp_index_score``   indexer logits z = q_idx . k_idx (fp32 fma chain)
* ``rtp_topp_select``   256-bin histogram top-p over the indexer softmax
* ``rtp_topk_select``   fixed top-k through the same histogram (token counts per bin)
* ``rtp_sparse_decode`` exact softmax attention over the selected tokens
* ``rtp_window_decode`` window + sink attention of local heads
* ``rtp_decode_step``   a whole layer: retrieval heads sparse, local heads windowed
* ``rtp_append_project`` the step's cache update: indexer projections of the new token
  and the append of its K/V rows
* ``rtp_prefill``       causal attention of a prompt (retrieval heads dense, local heads
  windowed) and the decode state it leaves

If the library is missing or fails to load, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# RTP_LIBRARY names another build of the same sources to load (the host-sanitizer build)
LIB_PATH = os.environ.get("RTP_LIBRARY") or os.path.join(_HERE, "librtp.so")

RTP_OK, RTP_EINVAL, RTP_EUNSUPPORTED, RTP_EWORKSPACE, RTP_EHIP, RTP_ESCRATCH = 0, -1, -2, -3, -4, -5
RTP_F32, RTP_F16, RTP_BF16 = 0, 1, 2
NBINS = 256
EXPORTED = [
    "rtp_status_string", "rtp_abi_version", "rtp_index_score",
    "rtp_topp_select_workspace_size", "rtp_topp_select",
    "rtp_topk_select_workspace_size", "rtp_topk_select",
    "rtp_sparse_decode_workspace_size", "rtp_sparse_decode",
    "rtp_window_decode_workspace_size", "rtp_window_decode",
    "rtp_decode_step_workspace_size", "rtp_decode_step", "rtp_decode_step_profiled",
    "rtp_decode_step_noalloc", "rtp_append_project", "rtp_prefill",
]

_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int32
F32 = ctypes.c_float
F64 = ctypes.c_double
SZ = ctypes.c_size_t


class LayerDesc(ctypes.Structure):
    """Mirror of rtp_layer_desc."""
    _fields_ = [
        ("B", I32), ("Hq", I32), ("Hkv", I32), ("d", I32), ("r", I32), ("Lmax", I32),
        ("window", I32), ("sinks", I32), ("kv_dtype", I32),
        ("kv_is_retrieval", P), ("q", P), ("q_idx", P), ("K_ret", P), ("V_ret", P),
        ("k_idx", P), ("K_loc", P), ("V_loc", P), ("seq_lens", P),
        ("p", F64), ("bin_width", F32), ("scale_idx", F32), ("scale_attn", F32),
        ("out", P), ("lse", P), ("thresh_out", P), ("count_out", P),
        ("topk", I32), ("ret_window", I32),
        ("sel_idx", P), ("sel_count", P), ("sel_cap", I32),
        ("append", P),
    ]


class StepAppend(ctypes.Structure):
    """Mirror of rtp_step_append (the cache update fused into the decode step)."""
    _fields_ = [("q_pre", P), ("k_pre", P), ("Wq_idx", P), ("Wk_idx", P), ("k_new", P),
                ("v_new", P)]


class AppendDesc(ctypes.Structure):
    """Mirror of rtp_append_desc."""
    _fields_ = [
        ("B", I32), ("Hq", I32), ("Hkv", I32), ("d", I32), ("r", I32), ("Lmax", I32),
        ("window", I32), ("sinks", I32), ("kv_dtype", I32),
        ("kv_is_retrieval", P), ("q_pre", P), ("k_pre", P), ("Wq_idx", P), ("Wk_idx", P),
        ("k_new", P), ("v_new", P), ("seq_lens", P), ("q_idx", P), ("k_idx", P),
        ("K_ret", P), ("V_ret", P), ("K_loc", P), ("V_loc", P),
    ]


class PrefillDesc(ctypes.Structure):
    """Mirror of rtp_prefill_desc."""
    _fields_ = [
        ("B", I32), ("Hq", I32), ("Hkv", I32), ("d", I32), ("r", I32), ("Lmax", I32),
        ("window", I32), ("sinks", I32), ("kv_dtype", I32),
        ("kv_is_retrieval", P), ("q", P), ("K", P), ("V", P), ("seq_lens", P),
        ("scale_attn", F32), ("out", P), ("k_pre", P), ("Wk_idx", P), ("k_idx", P),
        ("K_ret", P), ("V_ret", P), ("K_loc", P), ("V_loc", P),
    ]


class RtpError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(lib().rtp_status_string(code).decode())
        self.code = code


def lib():
    """The loaded librtp.so (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("librtp.so not built: run `python -m head_wise_sparse_rtp_amd.build` "
                               "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.rtp_status_string.restype = ctypes.c_char_p
        L.rtp_status_string.argtypes = [I32]
        L.rtp_abi_version.restype = I32
        L.rtp_abi_version.argtypes = []
        L.rtp_index_score.restype = I32
        L.rtp_index_score.argtypes = [P, P, I32, P, I32, I32, I32, I32, I32, F32, P, P]
        L.rtp_topp_select_workspace_size.restype = SZ
        L.rtp_topp_select_workspace_size.argtypes = [I32, I32, I32]
        L.rtp_topp_select.restype = I32
        L.rtp_topp_select.argtypes = [P, P, I32, I32, I32, F64, F32, P, P, I32, P, P, P, SZ, P]
        L.rtp_topk_select_workspace_size.restype = SZ
        L.rtp_topk_select_workspace_size.argtypes = [I32, I32, I32]
        L.rtp_topk_select.restype = I32
        L.rtp_topk_select.argtypes = [P, P, I32, I32, I32, I32, F32, P, P, I32, P, P, P, SZ, P]
        L.rtp_sparse_decode_workspace_size.restype = SZ
        L.rtp_sparse_decode_workspace_size.argtypes = [I32, I32, I32, I32]
        L.rtp_sparse_decode.restype = I32
        L.rtp_sparse_decode.argtypes = [P, P, P, I32, P, P, I32, I32, I32, I32, I32, I32, F32, P,
                                        P, P, SZ, P]
        L.rtp_window_decode_workspace_size.restype = SZ
        L.rtp_window_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32]
        L.rtp_window_decode.restype = I32
        L.rtp_window_decode.argtypes = [P, P, P, I32, P, I32, I32, I32, I32, I32, I32, F32, P, P,
                                        P, SZ, P]
        L.rtp_decode_step_workspace_size.restype = SZ
        L.rtp_decode_step_workspace_size.argtypes = [ctypes.POINTER(LayerDesc)]
        L.rtp_decode_step.restype = I32
        L.rtp_decode_step.argtypes = [ctypes.POINTER(LayerDesc), P, SZ, P]
        L.rtp_decode_step_profiled.restype = I32
        L.rtp_decode_step_profiled.argtypes = [ctypes.POINTER(LayerDesc), P, SZ, P, P * 4]
        L.rtp_decode_step_noalloc.restype = I32
        L.rtp_decode_step_noalloc.argtypes = [ctypes.POINTER(LayerDesc), P]
        L.rtp_append_project.restype = I32
        L.rtp_append_project.argtypes = [ctypes.POINTER(AppendDesc), P]
        L.rtp_prefill.restype = I32
        L.rtp_prefill.argtypes = [ctypes.POINTER(PrefillDesc), P]
        _lib = L
    return _lib


def _check(code: int):
    if code != RTP_OK:
        raise RtpError(code)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("rtp: tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("rtp: tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return RTP_F16
    if t.dtype == torch.float32:
        return RTP_F32
    if t.dtype == torch.bfloat16:
        return RTP_BF16
    raise ValueError("rtp: K/V/q/k_idx must be fp16, bf16 or fp32, got %s" % t.dtype)


def workspace(nbytes: int, device) -> torch.Tensor:
    """Workspace of `nbytes` bytes on `device` (zero-filled; the kernels need no
    particular contents)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# single-purpose entry points
# ---------------------------------------------------------------------------
def rtp_index_score(q_idx: torch.Tensor, k_idx: torch.Tensor, seq_lens: torch.Tensor,
                    scale_idx: float, z: Optional[torch.Tensor] = None, stream=None):
    """z [B, Hr*G, Lmax] fp32 from q_idx [B, Hr*G, r] fp32 and k_idx [B, Hr, Lmax, r]."""
    B, Hr, Lmax, r = k_idx.shape
    H = q_idx.shape[1]
    G = H // Hr
    if q_idx.dtype != torch.float32 or seq_lens.dtype != torch.int32:
        raise ValueError("rtp_index_score: q_idx fp32, seq_lens int32")
    if z is None:
        z = torch.empty((B, H, Lmax), dtype=torch.float32, device=k_idx.device)
    _check(lib().rtp_index_score(_ptr(q_idx), _ptr(k_idx), _kv_dtype(k_idx), _ptr(seq_lens), B, Hr,
                                 G, Lmax, r, scale_idx, _ptr(z), _stream(stream)))
    return z


def rtp_topp_select(z: torch.Tensor, seq_lens: torch.Tensor, p: float, bin_width: float = 0.125,
                    cap: Optional[int] = None, want_hist: bool = True, ws=None, stream=None):
    """Returns (sel_idx [B,H,cap] int32, sel_count [B,H] int32, hist [B,H,256] fp32 or None,
    thresh [B,H,2] int32 = {A, b*})."""
    B, H, Lmax = z.shape
    cap = Lmax if cap is None else int(cap)
    dev = z.device
    sel_idx = torch.full((B, H, max(cap, 1)), -1, dtype=torch.int32, device=dev)
    sel_count = torch.empty((B, H), dtype=torch.int32, device=dev)
    hist = torch.empty((B, H, NBINS), dtype=torch.float32, device=dev) if want_hist else None
    thresh = torch.empty((B, H, 2), dtype=torch.int32, device=dev)
    nb = lib().rtp_topp_select_workspace_size(B, H, Lmax)
    if ws is None:
        ws = workspace(nb, dev)
    _check(lib().rtp_topp_select(_ptr(z), _ptr(seq_lens), B, H, Lmax, float(p), float(bin_width),
                                 _ptr(sel_idx), _ptr(sel_count), cap, _ptr(hist), _ptr(thresh),
                                 _ptr(ws), ws.numel(), _stream(stream)))
    return sel_idx, sel_count, hist, thresh


def rtp_topk_select(z: torch.Tensor, seq_lens: torch.Tensor, k: int, bin_width: float = 0.125,
                    cap: Optional[int] = None, want_hist: bool = True, ws=None, stream=None):
    """Fixed top-k through the 256-bin histogram.  Returns (sel_idx [B,H,cap] int32,
    sel_count [B,H] int32, hist [B,H,256] fp32 token counts or None, thresh [B,H,2])."""
    B, H, Lmax = z.shape
    cap = Lmax if cap is None else int(cap)
    dev = z.device
    sel_idx = torch.full((B, H, max(cap, 1)), -1, dtype=torch.int32, device=dev)
    sel_count = torch.empty((B, H), dtype=torch.int32, device=dev)
    hist = torch.empty((B, H, NBINS), dtype=torch.float32, device=dev) if want_hist else None
    thresh = torch.empty((B, H, 2), dtype=torch.int32, device=dev)
    nb = lib().rtp_topk_select_workspace_size(B, H, Lmax)
    if ws is None:
        ws = workspace(nb, dev)
    _check(lib().rtp_topk_select(_ptr(z), _ptr(seq_lens), B, H, Lmax, int(k), float(bin_width),
                                 _ptr(sel_idx), _ptr(sel_count), cap, _ptr(hist), _ptr(thresh),
                                 _ptr(ws), ws.numel(), _stream(stream)))
    return sel_idx, sel_count, hist, thresh


def rtp_sparse_decode(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, sel_idx: torch.Tensor,
                      sel_count: torch.Tensor, scale_attn: float, want_lse: bool = True, ws=None,
                      stream=None):
    """out [B, Hr*G, d] fp32 (and lse [B, Hr*G]) over sel_idx [B, Hr*G, cap]."""
    B, Hr, Lmax, d = K.shape
    H = q.shape[1]
    G = H // Hr
    cap = sel_idx.shape[2]
    dev = q.device
    out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev) if want_lse else None
    nb = lib().rtp_sparse_decode_workspace_size(B, Hr, G, cap)
    if ws is None:
        ws = workspace(nb, dev)
    _check(lib().rtp_sparse_decode(_ptr(q), _ptr(K), _ptr(V), _kv_dtype(K), _ptr(sel_idx),
                                   _ptr(sel_count), cap, B, Hr, G, Lmax, d, scale_attn, _ptr(out),
                                   _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse


def rtp_window_decode(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, seq_lens: torch.Tensor,
                      window: int, sinks: int, scale_attn: float, want_lse: bool = True, ws=None,
                      stream=None):
    """out [B, Hl*G, d] fp32 over the ring K, V [B, Hl, sinks+window, d]."""
    B, Hl, ring, d = K.shape
    if ring != window + sinks:
        raise ValueError("rtp_window_decode: ring size must be sinks + window")
    H = q.shape[1]
    G = H // Hl
    dev = q.device
    out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev) if want_lse else None
    nb = lib().rtp_window_decode_workspace_size(B, Hl, G, window, sinks)
    if ws is None:
        ws = workspace(nb, dev)
    _check(lib().rtp_window_decode(_ptr(q), _ptr(K), _ptr(V), _kv_dtype(K), _ptr(seq_lens), B, Hl, G,
                                   d, window, sinks, scale_attn, _ptr(out), _ptr(lse), _ptr(ws),
                                   ws.numel(), _stream(stream)))
    return out, lse


# ---------------------------------------------------------------------------
# one decode step of a layer
# ---------------------------------------------------------------------------
class DecodeStep:
    """Holds the descriptor, host mask and workspace of one layer so that repeated
    calls (a decode loop, a captured graph) only enqueue kernels.  want_sets > 0 also
    exports the token set each retrieval query head attended to (sel_idx [B, Hq,
    want_sets]: the first sel_count entries ascending, the rest left as they were, -1
    after construction; sel_count [B, Hq])."""

    def __init__(self, layer, seq_lens: torch.Tensor, B: int, Hq: int, Hkv: int, Lmax: int,
                 window: int, sinks: int, p: float, bin_width: float, scale_idx: float,
                 scale_attn: float, out: Optional[torch.Tensor] = None, want_lse: bool = True,
                 want_debug: bool = False, ws: Optional[torch.Tensor] = None, topk: int = 0,
                 ret_window: bool = False, want_sets: int = 0, append=None):
        dev = layer.q.device
        self.keep = [layer.q, layer.q_idx, layer.K_ret, layer.V_ret, layer.k_idx, layer.K_loc,
                     layer.V_loc, seq_lens]
        self.mask = (ctypes.c_uint8 * Hkv)(*[int(x) for x in layer.kv_is_retrieval])
        d = layer.q.shape[-1]
        self.out = out if out is not None else torch.empty((B, Hq, d), dtype=torch.float32,
                                                           device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if want_lse else None
        self.thresh = (torch.zeros((B, Hq, 2), dtype=torch.int32, device=dev)
                       if want_debug else None)
        self.count = torch.zeros((B, Hq), dtype=torch.int32, device=dev) if want_debug else None
        self.sel_idx = self.sel_count = None
        if want_sets:
            self.sel_idx = torch.full((B, Hq, int(want_sets)), -1, dtype=torch.int32, device=dev)
            self.sel_count = torch.full((B, Hq), -1, dtype=torch.int32, device=dev)
        nret = int(sum(int(x) for x in layer.kv_is_retrieval))
        nloc = Hkv - nret

        def ptr_or_none(t, needed):
            return _ptr(t) if needed and t is not None and t.numel() > 0 else None

        self.desc = LayerDesc(
            B, Hq, Hkv, d, layer.q_idx.shape[-1], Lmax, window, sinks, _kv_dtype(layer.q),
            ctypes.cast(self.mask, ctypes.c_void_p), _ptr(layer.q), ptr_or_none(layer.q_idx, nret),
            ptr_or_none(layer.K_ret, nret), ptr_or_none(layer.V_ret, nret),
            ptr_or_none(layer.k_idx, nret), ptr_or_none(layer.K_loc, nloc),
            ptr_or_none(layer.V_loc, nloc), _ptr(seq_lens), float(p), float(bin_width),
            float(scale_idx), float(scale_attn), _ptr(self.out), _ptr(self.lse),
            _ptr(self.thresh), _ptr(self.count))
        self.desc.topk = int(topk)
        self.desc.ret_window = 1 if ret_window else 0
        self.desc.sel_idx = _ptr(self.sel_idx)
        self.desc.sel_count = _ptr(self.sel_count)
        self.desc.sel_cap = int(want_sets)
        self.app = None
        if append is not None:
            # the new token's cache update, fused into the step: `append` holds q_pre,
            # k_pre, Wq, Wk, k_new, v_new (see rtp_step_append); the layer's caches are
            # updated in place by every call
            self.keep += [append.q_pre, append.k_pre, append.Wq, append.Wk, append.k_new,
                          append.v_new]
            self.app = StepAppend(_ptr(append.q_pre), _ptr(append.k_pre), _ptr(append.Wq),
                                  _ptr(append.Wk), _ptr(append.k_new), _ptr(append.v_new))
            self.desc.append = ctypes.cast(ctypes.pointer(self.app), ctypes.c_void_p)
        nb = lib().rtp_decode_step_workspace_size(ctypes.byref(self.desc))
        if nb == 0:
            raise RtpError(RTP_EINVAL)
        self.ws = ws if ws is not None and ws.numel() >= nb else workspace(nb, dev)
        self.ws_bytes = nb

    def __call__(self, stream=None):
        _check(lib().rtp_decode_step(ctypes.byref(self.desc), _ptr(self.ws), self.ws.numel(),
                                     _stream(stream)))
        return self.out

    def noalloc(self, stream=None):
        """The same step on the library's fixed scratch (rtp_decode_step_noalloc): no
        workspace is used and nothing is allocated."""
        _check(lib().rtp_decode_step_noalloc(ctypes.byref(self.desc), _stream(stream)))
        return self.out

    def profiled(self, events, stream=None):
        """One call with kernel timing events (hipEvent_t handles as ints or None, four of
        them; see rtp_decode_step_profiled)."""
        ev = (P * 4)(*[e for e in events])
        _check(lib().rtp_decode_step_profiled(ctypes.byref(self.desc), _ptr(self.ws),
                                              self.ws.numel(), _stream(stream), ev))
        return self.out


def rtp_decode_step(layer, seq_lens, B, Hq, Hkv, Lmax, window, sinks, p, bin_width, scale_idx,
                    scale_attn, want_debug=False, stream=None, topk=0, ret_window=False,
                    want_sets=0, append=None):
    """One layer's decode step; returns (out, lse, thresh, count), followed by (sel_idx,
    sel_count) when want_sets > 0.  topk > 0 selects the retrieval heads' tokens with the
    fixed top-k rule instead of top-p."""
    st = DecodeStep(layer, seq_lens, B, Hq, Hkv, Lmax, window, sinks, p, bin_width, scale_idx,
                    scale_attn, want_debug=want_debug, topk=topk, ret_window=ret_window,
                    want_sets=want_sets, append=append)
    st(stream)
    if want_sets:
        return st.out, st.lse, st.thresh, st.count, st.sel_idx, st.sel_count
    return st.out, st.lse, st.thresh, st.count


class AppendProject:
    """Holds the descriptor of one layer's cache update so that repeated calls (a decode
    loop, a captured graph) only enqueue the kernel.  The caches of `layer` are updated in
    place; seq_lens holds the lengths after the append."""

    def __init__(self, layer, seq_lens: torch.Tensor, B: int, Hq: int, Hkv: int, Lmax: int,
                 window: int, sinks: int, q_pre: torch.Tensor, k_pre: torch.Tensor,
                 Wq: torch.Tensor, Wk: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor):
        self.keep = [layer.q_idx, layer.k_idx, layer.K_ret, layer.V_ret, layer.K_loc, layer.V_loc,
                     seq_lens, q_pre, k_pre, Wq, Wk, k_new, v_new]
        self.mask = (ctypes.c_uint8 * Hkv)(*[int(x) for x in layer.kv_is_retrieval])
        nret = int(sum(int(x) for x in layer.kv_is_retrieval))
        nloc = Hkv - nret

        def opt(t, needed):
            return _ptr(t) if needed and t is not None and t.numel() > 0 else None

        self.desc = AppendDesc(
            B, Hq, Hkv, k_new.shape[-1], layer.q_idx.shape[-1], Lmax, window, sinks,
            _kv_dtype(k_new), ctypes.cast(self.mask, ctypes.c_void_p), opt(q_pre, nret),
            opt(k_pre, nret), opt(Wq, nret), opt(Wk, nret), _ptr(k_new), _ptr(v_new),
            _ptr(seq_lens), opt(layer.q_idx, nret), opt(layer.k_idx, nret),
            opt(layer.K_ret, nret), opt(layer.V_ret, nret), opt(layer.K_loc, nloc),
            opt(layer.V_loc, nloc))

    def __call__(self, stream=None):
        _check(lib().rtp_append_project(ctypes.byref(self.desc), _stream(stream)))


def rtp_append_project(layer, seq_lens, B, Hq, Hkv, Lmax, window, sinks, q_pre, k_pre, Wq, Wk,
                       k_new, v_new, stream=None):
    """One layer's cache update in place (see AppendProject)."""
    AppendProject(layer, seq_lens, B, Hq, Hkv, Lmax, window, sinks, q_pre, k_pre, Wq, Wk,
                  k_new, v_new)(stream)


class Prefill:
    """Holds the descriptor of one prompt's prefill (so that repeated calls only enqueue
    the kernels).  out [B, Hq, Lmax, d] fp32; with_state also allocates the decode state
    (k_idx, K_ret, V_ret of the retrieval heads, the local heads' rings)."""

    def __init__(self, seq_lens: torch.Tensor, mask, q: torch.Tensor, K: torch.Tensor,
                 V: torch.Tensor, window: int, sinks: int, scale_attn: float,
                 k_pre: Optional[torch.Tensor] = None, Wk: Optional[torch.Tensor] = None,
                 with_state: bool = False, out: Optional[torch.Tensor] = None):
        B, Hq, Lmax, d = q.shape
        Hkv = K.shape[1]
        dev = q.device
        self.mask = (ctypes.c_uint8 * Hkv)(*[int(x) for x in mask])
        nret = int(sum(int(x) for x in mask))
        nloc = Hkv - nret
        self.out = out if out is not None else torch.empty((B, Hq, Lmax, d), dtype=torch.float32,
                                                           device=dev)
        self.k_idx = self.K_ret = self.V_ret = self.K_loc = self.V_loc = None
        if with_state:
            r = Wk.shape[-1]
            if nret:
                self.k_idx = torch.zeros((B, nret, Lmax, r), dtype=K.dtype, device=dev)
                self.K_ret = torch.zeros((B, nret, Lmax, d), dtype=K.dtype, device=dev)
                self.V_ret = torch.zeros_like(self.K_ret)
            if nloc:
                self.K_loc = torch.zeros((B, nloc, sinks + window, d), dtype=K.dtype, device=dev)
                self.V_loc = torch.zeros_like(self.K_loc)
        self.keep = [seq_lens, q, K, V, k_pre, Wk]
        self.desc = PrefillDesc(
            B, Hq, Hkv, d, Wk.shape[-1] if Wk is not None else 16, Lmax, window, sinks,
            _kv_dtype(q), ctypes.cast(self.mask, ctypes.c_void_p), _ptr(q), _ptr(K), _ptr(V),
            _ptr(seq_lens), float(scale_attn), _ptr(self.out),
            _ptr(k_pre) if self.k_idx is not None else None,
            _ptr(Wk) if self.k_idx is not None else None, _ptr(self.k_idx), _ptr(self.K_ret),
            _ptr(self.V_ret), _ptr(self.K_loc), _ptr(self.V_loc))

    def __call__(self, stream=None):
        _check(lib().rtp_prefill(ctypes.byref(self.desc), _stream(stream)))
        return self.out


def rtp_prefill(seq_lens, mask, q, K, V, window, sinks, scale_attn, k_pre=None, Wk=None,
                with_state=False, stream=None):
    """One prompt's prefill; returns the Prefill object (out and, with_state, the state)."""
    pf = Prefill(seq_lens, mask, q, K, V, window, sinks, scale_attn, k_pre, Wk, with_state)
    pf(stream)
    return pf


def decode_workload(wl, want_debug: bool = False, stream=None, want_sets: int = 0,
                    appends=None):
    """Run every layer of a `workloads.Workload` already on the GPU; returns per-layer
    (out, lse, thresh, count), plus (sel_idx, sel_count) when want_sets > 0.  appends, when
    given, holds per layer the inputs of the cache update fused into its step (or None)."""
    sl = torch.as_tensor(wl.seq_lens, dtype=torch.int32).to(wl.layers[0].q.device)
    res = []
    for li, layer in enumerate(wl.layers):
        res.append(rtp_decode_step(layer, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks,
                                   wl.p, wl.bin_width, wl.scale_idx, wl.scale_attn, want_debug,
                                   stream, getattr(wl, "topk", 0), getattr(wl, "ret_window", False),
                                   want_sets, appends[li] if appends is not None else None))
    return res
