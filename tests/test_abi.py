"""The C ABI without a GPU: the library loads, exports every declared entry point, and
rejects invalid arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtp.h")


@pytest.fixture(scope="module")
def lib():
    import head_wise_sparse_rtp_amd as m
    if not os.path.exists(m.LIB_PATH):
        from head_wise_sparse_rtp_amd import build
        build.build()
    return m.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(rtp_[a-z_]+)\s*\(", src)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    import head_wise_sparse_rtp_amd as m
    names = declared_functions()
    assert set(names) == set(m.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.rtp_abi_version() == 3
    for code in [0, -1, -2, -3, -4, -5]:
        assert lib.rtp_status_string(code).startswith(b"RTP_")
    assert lib.rtp_status_string(7) == b"unknown rtp_status"


FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced on the host
MIS = ctypes.c_void_p(0x10004)        # misaligned


def test_index_score_validation(lib):
    f = lib.rtp_index_score
    ok = (FAKE, FAKE, 1, FAKE, 1, 1, 8, 1024, 16, 0.25, FAKE, None)
    bad = [
        ((None,) + ok[1:], -1),
        ((MIS,) + ok[1:], -1),
        (ok[:8] + (15,) + ok[9:], -2),          # r != 16
        (ok[:2] + (7,) + ok[3:], -2),           # dtype
        (ok[:6] + (0,) + ok[7:], -2),           # G = 0
        (ok[:7] + (0,) + ok[8:], -1),           # Lmax = 0
        (ok[:7] + ((1 << 24) + 1,) + ok[8:], -2),
        (ok[:9] + (float("inf"),) + ok[10:], -1),
    ]
    for args, code in bad:
        assert f(*args) == code, args


def test_topp_select_validation_and_workspace(lib):
    f = lib.rtp_topp_select
    nb = lib.rtp_topp_select_workspace_size(2, 8, 100000)
    assert nb > 2 * 8 * 1024  # at least the per-head histograms
    assert lib.rtp_topp_select_workspace_size(0, 8, 10) == 0
    ok = [FAKE, FAKE, 2, 8, 100000, 0.9, 0.125, FAKE, FAKE, 100000, None, None, FAKE, nb, None]

    def call(**kw):
        a = list(ok)
        names = ["z", "sl", "B", "H", "Lmax", "p", "w", "si", "sc", "cap", "hist", "thr", "ws",
                 "wsb", "st"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(p=0.0) == -1
    assert call(p=float("nan")) == -1
    assert call(w=0.1) == -1            # not a power of two
    assert call(w=2.0) == -1            # outside 2^-10 .. 1
    assert call(ws=MIS) == -1
    assert call(hist=MIS) == -1
    assert call(wsb=nb - 1) == -3
    assert call(cap=-1) == -1
    assert call(z=None) == -1


def test_topk_select_validation_and_workspace(lib):
    f = lib.rtp_topk_select
    nb = lib.rtp_topk_select_workspace_size(2, 8, 100000)
    assert nb == lib.rtp_topp_select_workspace_size(2, 8, 100000)
    ok = [FAKE, FAKE, 2, 8, 100000, 2048, 0.125, FAKE, FAKE, 100000, None, None, FAKE, nb, None]
    names = ["z", "sl", "B", "H", "Lmax", "k", "w", "si", "sc", "cap", "hist", "thr", "ws", "wsb",
             "st"]

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(k=0) == -1
    assert call(k=-5) == -1
    assert call(w=0.3) == -1
    assert call(wsb=nb - 1) == -3
    assert call(thr=MIS) == -1
    assert call(sc=None) == -1
    assert call(Lmax=(1 << 24) + 1) == -2


def test_layer_desc_matches_the_header():
    import head_wise_sparse_rtp_amd as m
    # the ctypes mirror lists the header's fields in the header's order
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} rtp_layer_desc;", src, re.S).group(1)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        for part in decl.split(","):
            names.append(re.findall(r"(\w+)\s*(?:\[\d+\])?\s*$", part.strip())[0])
    assert names == [f[0] for f in m.LayerDesc._fields_]


def test_append_desc_matches_the_header():
    import head_wise_sparse_rtp_amd as m
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^{}]*)\} rtp_append_desc;", src).group(1)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if decl:
            names += [re.findall(r"(\w+)\s*$", part.strip())[0] for part in decl.split(",")]
    assert names == [f[0] for f in m.AppendDesc._fields_]


def test_prefill_desc_matches_the_header():
    import head_wise_sparse_rtp_amd as m
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^{}]*)\} rtp_prefill_desc;", src).group(1)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if decl:
            names += [re.findall(r"(\w+)\s*$", part.strip())[0] for part in decl.split(",")]
    assert names == [f[0] for f in m.PrefillDesc._fields_]


def test_prefill_validation(lib):
    import head_wise_sparse_rtp_amd as m
    mask = (ctypes.c_uint8 * 4)(1, 0, 0, 0)
    d = m.PrefillDesc(1, 32, 4, 128, 16, 4096, 8192, 4, 1, ctypes.cast(mask, ctypes.c_void_p),
                      FAKE, FAKE, FAKE, FAKE, 0.088, FAKE, None, None, None, None, None, None,
                      None)
    f = lambda: lib.rtp_prefill(ctypes.byref(d), None)
    d.kv_dtype = 0
    assert f() == -2                     # fp16 or bf16 only
    d.kv_dtype = 5
    assert f() == -2
    d.kv_dtype = 2
    d.K_ret = FAKE                       # K_ret without V_ret (bf16)
    assert f() == -1
    d.K_ret = None
    d.kv_dtype = 1
    d.K_ret = FAKE                       # K_ret without V_ret
    assert f() == -1
    d.K_ret = None
    d.k_idx = FAKE                       # k_idx without k_pre / Wk_idx
    assert f() == -1
    d.k_idx = None
    d.window = 0
    assert f() == -1
    d.window = 8192
    d.out = MIS
    assert f() == -1
    d.out = FAKE
    for bad in (0.0, -0.088, float("nan")):
        d.scale_attn = bad
        assert f() == -1, bad
    assert lib.rtp_prefill(None, None) == -1


def test_append_project_validation(lib):
    import head_wise_sparse_rtp_amd as m
    mask = (ctypes.c_uint8 * 4)(1, 0, 0, 0)
    d = m.AppendDesc(1, 32, 4, 128, 16, 65536, 8192, 4, 1, ctypes.cast(mask, ctypes.c_void_p),
                     *([FAKE] * 13))
    f = lambda: lib.rtp_append_project(ctypes.byref(d), None)
    d.r = 8
    assert f() == -2
    d.r = 16
    d.Hq = 30
    assert f() == -1
    d.Hq = 32
    d.Wk_idx = None                      # needed: KV head 0 is a retrieval head
    assert f() == -1
    d.Wk_idx = FAKE
    d.K_loc = MIS
    assert f() == -1
    d.K_loc = FAKE
    d.window = 0
    assert f() == -1
    d.window = 8192
    d.kv_dtype = 5
    assert f() == -2
    assert lib.rtp_append_project(None, None) == -1


def test_sparse_and_window_validation(lib):
    nb = lib.rtp_sparse_decode_workspace_size(1, 1, 8, 4096)
    assert nb > 0
    f = lib.rtp_sparse_decode
    ok = [FAKE, FAKE, FAKE, 1, FAKE, FAKE, 4096, 1, 1, 8, 65536, 128, 0.088, FAKE, None, FAKE, nb,
          None]
    a = list(ok); a[11] = 64
    assert f(*a) == -2                  # d != 128
    a = list(ok); a[16] = nb - 1
    assert f(*a) == -3
    a = list(ok); a[3] = 5
    assert f(*a) == -2                  # bad dtype
    nbw = lib.rtp_window_decode_workspace_size(1, 3, 8, 8192, 4)
    g = lib.rtp_window_decode
    okw = [FAKE, FAKE, FAKE, 1, FAKE, 1, 3, 8, 128, 8192, 4, 0.088, FAKE, None, FAKE, nbw, None]
    a = list(okw); a[9] = 0
    assert g(*a) == -1                  # window = 0
    a = list(okw); a[15] = 0
    assert g(*a) == -3
    a = list(okw); a[1] = MIS
    assert g(*a) == -1
    # the attention scale is a softmax temperature: positive and finite
    for bad in (0.0, -0.088, float("nan"), float("inf")):
        a = list(ok); a[12] = bad
        assert f(*a) == -1, bad
        a = list(okw); a[11] = bad
        assert g(*a) == -1, bad


def test_decode_step_validation(lib):
    import head_wise_sparse_rtp_amd as m
    mask = (ctypes.c_uint8 * 4)(1, 0, 0, 0)
    d = m.LayerDesc(1, 32, 4, 128, 16, 65536, 8192, 4, 1, ctypes.cast(mask, ctypes.c_void_p),
                    FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.9, 0.125, 0.25, 0.088,
                    FAKE, None, None, None)
    nb = lib.rtp_decode_step_workspace_size(ctypes.byref(d))
    assert nb > 0
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nb - 1, None) == -3
    d.Hq = 30                           # not a multiple of Hkv
    assert lib.rtp_decode_step_workspace_size(ctypes.byref(d)) == 0
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nb, None) == -1
    d.Hq = 32
    d.r = 8
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nb, None) == -2
    d.r = 16
    d.p = -1.0
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nb, None) == -1
    d.topk = 64                         # top-k: same workspace, p not consulted
    assert lib.rtp_decode_step_workspace_size(ctypes.byref(d)) == nb
    d.topk = -1
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nb, None) == -1
    d.topk = 0
    d.ret_window = 2
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nb, None) == -1
    d.ret_window = 0
    d.p = 0.9
    d.k_idx = None
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nb, None) == -1
    d.k_idx = FAKE
    # a negative or zero attention scale would turn the MFMA tile's row maxima into minima
    for bad in (0.0, -0.088, float("nan")):
        d.scale_attn = bad
        assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nb, None) == -1, bad
    d.scale_attn = 0.088


def test_decode_step_set_export_and_profiled_validation(lib):
    import head_wise_sparse_rtp_amd as m
    mask = (ctypes.c_uint8 * 4)(1, 0, 0, 0)
    d = m.LayerDesc(1, 32, 4, 128, 16, 65536, 8192, 4, 1, ctypes.cast(mask, ctypes.c_void_p),
                    FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.9, 0.125, 0.25, 0.088,
                    FAKE, None, None, None)
    nb = lib.rtp_decode_step_workspace_size(ctypes.byref(d))
    d.sel_idx, d.sel_count, d.sel_cap = FAKE, FAKE, 4096
    nbx = lib.rtp_decode_step_workspace_size(ctypes.byref(d))
    assert nbx > nb                      # the exported lists need room of their own
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nbx - 1, None) == -3
    d.sel_count = None                   # one without the other
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nbx, None) == -1
    d.sel_count = MIS
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nbx, None) == -1
    d.sel_count = FAKE
    d.sel_cap = 0
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, nbx, None) == -1
    # the profiled call validates exactly like the plain one (nothing is enqueued)
    ev = (ctypes.c_void_p * 4)()
    assert lib.rtp_decode_step_profiled(ctypes.byref(d), FAKE, nbx, None, ev) == -1
    d.sel_cap = 4096
    assert lib.rtp_decode_step_profiled(ctypes.byref(d), FAKE, nbx - 1, None, ev) == -3
    assert lib.rtp_decode_step_profiled(None, FAKE, nbx, None, ev) == -1


def test_decode_step_noalloc_checks_before_any_device_call(lib):
    import head_wise_sparse_rtp_amd as m
    mask = (ctypes.c_uint8 * 4)(1, 0, 0, 0)
    d = m.LayerDesc(1, 32, 4, 128, 16, 1 << 24, 8192, 4, 1, ctypes.cast(mask, ctypes.c_void_p),
                    FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.9, 0.125, 0.25, 0.088,
                    FAKE, None, None, None)
    # 2^24 tokens need about 209 MiB of workspace: beyond the fixed 64 MiB scratch
    assert lib.rtp_decode_step_workspace_size(ctypes.byref(d)) > 64 << 20
    assert lib.rtp_decode_step_noalloc(ctypes.byref(d), None) == -5
    assert lib.rtp_status_string(-5).startswith(b"RTP_ESCRATCH")
    # an invalid descriptor is reported as rtp_decode_step reports it
    d.Lmax = 65536
    d.Hq = 30
    assert lib.rtp_decode_step_noalloc(ctypes.byref(d), None) == -1
    assert lib.rtp_decode_step_noalloc(None, None) == -1


def test_batch_rows_beyond_the_grid_limit_are_unsupported(lib):
    """B x query heads above 65535 would exceed a launch's y/z grid dimension (or push a
    one-dimensional block count towards the int range): every entry point says so on the
    host, and the size queries return 0."""
    import head_wise_sparse_rtp_amd as m
    # index score: B x Hr x G rows
    assert lib.rtp_index_score(FAKE, FAKE, 1, FAKE, 8193, 1, 8, 1024, 16, 0.25, FAKE, None) == -2
    # selection: B x H rows
    assert lib.rtp_topp_select_workspace_size(8191, 8, 4096) > 0   # 65528 rows
    assert lib.rtp_topp_select_workspace_size(8193, 8, 4096) == 0
    assert lib.rtp_topk_select_workspace_size(8193, 8, 4096) == 0
    args = [FAKE, FAKE, 8193, 8, 4096, 0.9, 0.125, FAKE, FAKE, 4096, None, None, FAKE, 1 << 40, None]
    assert lib.rtp_topp_select(*args) == -2
    args[5] = 64
    assert lib.rtp_topk_select(*args) == -2
    # sparse and window decode: B x heads x G rows
    assert lib.rtp_sparse_decode_workspace_size(8193, 1, 8, 4096) == 0
    assert lib.rtp_sparse_decode(FAKE, FAKE, FAKE, 1, FAKE, FAKE, 4096, 8193, 1, 8, 4096, 128,
                                 0.088, FAKE, None, FAKE, 1 << 40, None) == -2
    assert lib.rtp_window_decode_workspace_size(2731, 3, 8, 8192, 4) == 0
    assert lib.rtp_window_decode(FAKE, FAKE, FAKE, 1, FAKE, 2731, 3, 8, 128, 8192, 4, 0.088, FAKE,
                                 None, FAKE, 1 << 40, None) == -2
    # the decode step, the cache update and the prefill: B x Hq rows
    mask = (ctypes.c_uint8 * 4)(1, 0, 0, 0)
    d = m.LayerDesc(2047, 32, 4, 128, 16, 4096, 8192, 4, 1, ctypes.cast(mask, ctypes.c_void_p),
                    FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.9, 0.125, 0.25, 0.088,
                    FAKE, None, None, None)
    assert lib.rtp_decode_step_workspace_size(ctypes.byref(d)) > 0   # 65504 rows
    d.B = 2048                                                         # 65536 rows
    assert lib.rtp_decode_step_workspace_size(ctypes.byref(d)) == 0
    assert lib.rtp_decode_step(ctypes.byref(d), FAKE, 1 << 40, None) == -2
    a = m.AppendDesc(2049, 32, 4, 128, 16, 4096, 8192, 4, 1, ctypes.cast(mask, ctypes.c_void_p),
                     *([FAKE] * 13))
    assert lib.rtp_append_project(ctypes.byref(a), None) == -2
    pd = m.PrefillDesc(2049, 32, 4, 128, 16, 4096, 8192, 4, 1, ctypes.cast(mask, ctypes.c_void_p),
                       FAKE, FAKE, FAKE, FAKE, 0.088, FAKE, None, None, None, None, None, None,
                       None)
    assert lib.rtp_prefill(ctypes.byref(pd), None) == -2
    # a long prompt over many heads: the prefill's one-dimensional grid would pass 2^31 blocks
    pd.B, pd.Hq, pd.Hkv, pd.Lmax = 64, 64, 64, 1 << 24
    mask64 = (ctypes.c_uint8 * 64)(*([0] * 64))
    pd.kv_is_retrieval = ctypes.cast(mask64, ctypes.c_void_p)
    assert lib.rtp_prefill(ctypes.byref(pd), None) == -2

