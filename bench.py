"""Benchmark: one RTPurbo decode step (all heads of a layer) on one MI355X.

Default workload: 1M-token context, batch 1, 32 query / 4 KV heads, head size 128,
fp16 K/V; KV head 0 is a retrieval head (indexer r = 16, p = 0.9; 2 needle, 4 mid and
2 broad query heads), KV heads 1-3 are local heads (window 8192 + 4 sinks).

A step is one call of rtp_decode_step: indexer score + 256-bin histogram top-p +
sparse attention for the retrieval head, window attention for the local heads, and
the split-K merges.  Inputs are resident in HBM; R rotated copies of every input
defeat the 256 MB Infinity Cache between consecutive steps.

value = algorithmic HBM bytes per step / time per step (GB/s), where the algorithmic
bytes are: the indexer keys (L * 16 * 2 B per retrieval KV head), the K and V rows of
the union of the selected sets over the KV head's query heads (512 B per token), and
each local head's window+sink rows (512 B per row).
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
REPEATS = 5  # timed repeats of K steps; the median is the reported time


def context_label(L):
    """A context length as the metric names it: 64K, 1M, 1.5M, 12345."""
    for unit, name in ((1 << 20, "M"), (1 << 10, "K")):
        if L >= unit and L % (unit // 2) == 0:
            v = L / unit
            return ("%d%s" % (v, name)) if v == int(v) else ("%.1f%s" % (v, name))
    return str(L)


def decode_metric(L):
    return "decode attention us/step and achieved HBM GB/s (% of peak) at " + context_label(L) + " context"


def hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


HIP_EVENT_TIMING_NO_FENCE = 0x20000000  # no system-scope cache flush around the timestamp


def make_events(h, n, flags=0):
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        assert h.hipEventCreateWithFlags(ctypes.byref(e), flags) == 0
        evs.append(e)
    return evs


def elapsed_ms(h, a, b):
    ms = ctypes.c_float()
    assert h.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    return ms.value


def algorithmic_bytes(rtp, wl, layer, torch, topk=0, ret_window=False):
    """Realised bytes of one step.  The union of the selected sets per retrieval KV head
    comes from the sets the step itself attended to (exported by rtp_decode_step, the rule
    the timed step runs: top-p, or the fixed top-k when topk > 0; with ret_window the sink
    and window rows are part of them).  Also returns, per retrieval query head, the share of
    the indexer softmax mass that its selected set holds (outside any timed region)."""
    dev = layer.q.device
    sl = torch.as_tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    e_idx = 4 if wl.dtype == "f32" else 2
    e_kv = e_idx
    detail = {"kidx": 0, "sparse_kv": 0, "window_kv": 0, "union_tokens": 0, "sel_tokens": [],
              "sel_mass": []}
    G = wl.G
    ret = layer.ret_heads
    if ret:
        _, _, _, _, sidx, scnt = rtp.rtp_decode_step(
            layer, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks, wl.p, wl.bin_width,
            wl.scale_idx, wl.scale_attn, topk=topk, ret_window=ret_window, want_sets=wl.Lmax)
        qi = torch.stack([layer.q_idx[:, h * G:(h + 1) * G] for h in ret], 1).reshape(
            wl.B, len(ret) * G, wl.r).contiguous()
        z = rtp.rtp_index_score(qi, layer.k_idx, sl, wl.scale_idx).double().cpu()
        sidx, scnt = sidx.cpu(), scnt.cpu()
        for b in range(wl.B):
            L = int(wl.seq_lens[b])
            for k, kv in enumerate(ret):
                u = set()
                for g in range(G):
                    h = kv * G + g
                    n = int(scnt[b, h])
                    detail["sel_tokens"].append(n)
                    idx = sidx[b, h, :n].long()
                    zz = z[b, k * G + g, :L]
                    e = torch.exp(zz - zz.max())
                    detail["sel_mass"].append(round(float(e[idx].sum() / e.sum()), 4))
                    u.update(idx.tolist())
                detail["kidx"] += L * wl.r * e_idx
                detail["sparse_kv"] += len(u) * 2 * wl.d * e_kv
                detail["union_tokens"] += len(u)
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        detail["window_kv"] += len(layer.loc_heads) * min(L, wl.window + wl.sinks) * 2 * wl.d * e_kv
    total = detail["kidx"] + detail["sparse_kv"] + detail["window_kv"]
    return total, detail


HBM_READ_LIB = os.path.join(ROOT, "head_wise_sparse_rtp_amd", "libhbmread.so")


def hbm_read_ceiling(torch, gib=4, reps=8):
    """Streaming-read ceiling of this GPU's HBM: the hand-written read kernels of
    libhbmread.so (16-byte loads in grid-stride or per-block span order, 4 to 16 in flight
    per thread, plain or nontemporal) over a `gib` GiB buffer, the best of a few grid sizes;
    GB/s."""
    lib = ctypes.CDLL(HBM_READ_LIB)
    lib.hbm_read.restype = ctypes.c_int
    lib.hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                             ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    grids = (256, 512, 1024, 2048, 4096, 8192, 16384)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    best = (0.0, None)
    for blocks in grids:
        for var in range(8):
            def run():
                rc = lib.hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                  ctypes.c_void_p(sink.data_ptr()), blocks, var, sp)
                assert rc == 0, rc
            run()
            run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                run()
            e1.record(st)
            e1.synchronize()
            gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if gbs > best[0]:
                best = (gbs, {"blocks": blocks, "order": "span" if var >= 4 else "grid-stride",
                              "loads_in_flight": (4, 8, 8, 16)[var // 4 * 2 + var % 2],
                              "nontemporal": var % 4 >= 2})
    del buf, sink
    torch.cuda.synchronize()
    return {"value": round(best[0], 1), "unit": "GB/s", "bytes": nbytes,
            "kernel": "hbm_read (libhbmread.so)", "best_shape": best[1]}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fused_step_c4.json")
KERNEL_SOURCE = os.path.join(ROOT, "head_wise_sparse_rtp_amd", "csrc", "rtp_step.hip")
TRAFFIC_KERNELS = ("k_stage_a", "k_stage_b")


def source_sha256() -> str:
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when
    there is none for this workload or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("source_sha256") != source_sha256():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def summarize_pmc(fetch_csv, write_csv, workload, copy_bytes, out):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the step's kernels and of the
    calibration copy kernel (a unary elementwise kernel over copy_bytes bytes) from two
    rocprofv3 --pmc runs; each counter is scaled by copy_bytes / (its reading for the
    copy)."""
    import csv
    import re

    def per_kernel(path, counter):
        agg = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                n = re.sub(r"\(.*", "", r["Kernel_Name"].replace("(anonymous namespace)::", ""))
                agg.setdefault(n, []).append(float(r["Counter_Value"]))
        return agg

    res = {"workload": workload, "source_sha256": source_sha256(), "copy_bytes": copy_bytes,
           "kernels": {}}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        agg = per_kernel(path, counter)
        copy = [v for n, vs in agg.items() if "neg_kernel" in n for v in vs]
        if not copy:
            raise SystemExit("no %s readings for the copy kernel in %s" % (counter, path))
        copy_kib = max(copy)  # the large calibration copies (the bench also negates tiny tensors)
        factor = copy_bytes / (copy_kib * 1024.0)
        res.setdefault("scale", {})[counter] = {"copy_kib": round(copy_kib, 1),
                                                "factor": round(factor, 4)}
        for kern in TRAFFIC_KERNELS:
            vals = [v for n, vs in agg.items() if kern in n for v in vs]
            if not vals:
                raise SystemExit("no %s readings for %s in %s" % (counter, kern, path))
            kib = sum(vals) / len(vals)
            res["kernels"].setdefault(kern, {})[counter] = {
                "kib_per_launch": round(kib, 1), "bytes_per_launch": round(kib * 1024.0 * factor)}
    for kern, d in res["kernels"].items():
        d["bytes_per_launch"] = d["FETCH_SIZE"]["bytes_per_launch"] + d["WRITE_SIZE"]["bytes_per_launch"]
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))


def calibrate_copy(mib: int, reps: int):
    """A plain device copy of known size (negation: read N bytes, write N bytes) for
    scaling the HBM byte counters."""
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "reps": reps}), flush=True)


def cpu_baseline(wl, bytes_per_step, budget_s):
    """The oracle as it is, timed on this host: its per-head C loops run for every
    (sequence, query head) of the step, the heads spread over a thread pool (the C calls
    release the interpreter lock), as many threads as the host gives this process, at most
    16 (one GPU's share of the box)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    cpu_wl = wl.to("cpu")
    host = len(os.sched_getaffinity(0))
    tasks = [(li, b, h) for li in range(len(cpu_wl.layers)) for b in range(cpu_wl.B)
             for h in range(cpu_wl.Hq)]
    nthr = max(1, min(16, host, len(tasks)))

    def one(t):
        li, b, h = t
        lay = cpu_wl.layers[li]
        return oracle.decode_layer(lay, cpu_wl.seq_lens, cpu_wl.Hq, cpu_wl.Hkv, cpu_wl.p,
                                   cpu_wl.bin_width, cpu_wl.scale_idx, cpu_wl.scale_attn,
                                   cpu_wl.window, cpu_wl.sinks, heads=[h], batches=[b],
                                   topk=getattr(cpu_wl, "topk", 0),
                                   ret_window=getattr(cpu_wl, "ret_window", False))

    with ThreadPoolExecutor(nthr) as pool:
        t0 = time.perf_counter()
        n = 0
        while True:
            list(pool.map(one, tasks))
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / n
    return {"value": round(bytes_per_step / dt / 1e9, 4), "unit": "GB/s", "cores": nthr,
            "host_cores": host, "kind": "oracle", "s_per_step": round(dt, 4),
            "sample": "%d full decode step(s) of the same workload (all %d query heads), the C "
                      "oracle per (sequence, query head) on %d threads, inputs copied to host "
                      "memory" % (n, cpu_wl.Hq, nthr)}


PEAK_MFMA_F16_TFLOPS = 2500.0


def prefill_pairs(L: int, retrieval: bool, window: int, sinks: int) -> int:
    """Query-key pairs a prompt of length L attends: every n <= t for a retrieval head, the
    sinks plus the last `window` positions up to t for a local head."""
    if retrieval:
        return L * (L + 1) // 2
    tot = 0
    W = window + sinks
    full = min(L, W)
    tot += full * (full + 1) // 2          # t + 1 <= window + sinks: every n <= t
    tot += max(0, L - W) * W               # later: the sinks and the last `window`
    return tot


def bench_prefill(args):
    """Prefill of one prompt at the decode configurations' head layout: 32 query heads on
    4 KV heads, KV head 0 dense (retrieval), the others windowed (8192 + 4 sinks)."""
    import torch
    import head_wise_sparse_rtp_amd as rtp
    import workloads
    dev = torch.device("cuda:0")
    L, Hq, Hkv, d, window, sinks = args.prefill, 32, 4, 128, 8192, 4
    # --dense: every KV head dense causal, the dense prefill of the same prompt
    mask = [1, 1, 1, 1] if args.dense else [1, 0, 0, 0]
    pr = workloads.make_prompt([L], Hq, Hkv, mask, seed=7, device=dev, dtype=args.dtype)
    sl = torch.tensor([L], dtype=torch.int32, device=dev)
    pf = rtp.Prefill(sl, mask, pr.q, pr.K, pr.V, window, sinks, 1.0 / math.sqrt(d), pr.k_pre,
                     pr.Wk, with_state=True)
    for _ in range(args.warmup):
        pf()
    torch.cuda.synchronize()
    h = hip()
    stream = torch.cuda.current_stream()
    e0, e1 = make_events(h, 2)
    h.hipEventRecord(e0, ctypes.c_void_p(stream.cuda_stream))
    for _ in range(args.steps):
        pf()
    h.hipEventRecord(e1, ctypes.c_void_p(stream.cuda_stream))
    h.hipEventSynchronize(e1)
    ms = elapsed_ms(h, e0, e1) / args.steps
    G = Hq // Hkv
    pairs = sum(G * prefill_pairs(L, bool(m), window, sinks) for m in mask)
    dense = Hq * prefill_pairs(L, True, window, sinks)
    flops = 4 * d * pairs
    tfs = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "prefill attention TFLOP/s (algorithmic: 4*d flops per attended query-key pair)",
        "value": round(tfs, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_prefill": round(ms, 4), "higher_is_better": True,
        "dtype": "%s q/K/V, fp32 accumulation" % args.dtype,
        "data": "synthetic (counter-based N(0,1))",
        "config": {"workload": "prefill: B=1, L=%d, Hq=%d, Hkv=%d (retrieval %s), d=%d, "
                               "window=%d+%d sinks; with the decode state (k_idx, caches, rings)"
                               % (L, Hq, Hkv, [i for i, m in enumerate(mask) if m], d, window,
                                  sinks)},
        "attended_pairs": pairs, "dense_causal_pairs": dense,
        "dense_over_sparse_work": round(dense / pairs, 3),
        "roofline": {"kernel": "k_prefill_attn (MFMA 16x16x32 %s)" % args.dtype, "bound": "mfma",
                     "achieved": round(tfs, 2), "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tfs / PEAK_MFMA_F16_TFLOPS, 4), "traffic": None},
    }
    print(json.dumps(res), flush=True)


def bench_layers(args, wl):
    """A whole multi-layer decode step: every layer of the workload in sequence on one
    stream (one captured graph per step); the caches of all layers stay resident."""
    import torch
    import head_wise_sparse_rtp_amd as rtp
    dev = torch.device("cuda:0")
    sl = torch.as_tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    bytes_step, kidx_bytes, union = 0, 0, 0
    for layer in wl.layers:
        b, det = algorithmic_bytes(rtp, wl, layer, torch)
        bytes_step += b
        kidx_bytes += det["kidx"]
        union += det["union_tokens"]
    steps, ws, out = [], None, None
    for layer in wl.layers:
        st = rtp.DecodeStep(layer, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks, wl.p,
                            wl.bin_width, wl.scale_idx, wl.scale_attn, out=out, want_lse=False,
                            ws=ws)
        ws, out = st.ws, st.out
        steps.append(st)
    for _ in range(max(1, args.warmup // 10)):
        for st in steps:
            st()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for st in steps:
            st()
    g.replay()
    torch.cuda.synchronize()
    h = hip()
    stream = torch.cuda.current_stream()
    e0, e1 = make_events(h, 2)
    K = args.steps
    h.hipEventRecord(e0, ctypes.c_void_p(stream.cuda_stream))
    for _ in range(K):
        g.replay()
    h.hipEventRecord(e1, ctypes.c_void_p(stream.cuda_stream))
    h.hipEventSynchronize(e1)
    ms_step = elapsed_ms(h, e0, e1) / K
    # stage A of the layers with retrieval heads, timed with fence-free events
    evs = make_events(h, 4, HIP_EVENT_TIMING_NO_FENCE)
    a_tot, a_n = 0.0, 0
    for st, layer in zip(steps, wl.layers):
        if not layer.ret_heads:
            continue
        torch.cuda._sleep(200000)
        st.profiled([e.value for e in evs])
        torch.cuda.synchronize()
        a_tot += elapsed_ms(h, evs[0], evs[1])
        a_n += 1
    a_us = a_tot / max(a_n, 1) * 1000.0
    nret = sum(len(l.ret_heads) for l in wl.layers)
    a_bytes = kidx_bytes / max(a_n, 1)
    achieved = a_bytes / (a_us * 1e-6) / 1e9 if a_us > 0 else 0.0
    value = bytes_step / (ms_step * 1e-3) / 1e9
    res = {
        "metric": "decode attention us/step and achieved HBM GB/s (%% of peak), %d layers" % len(wl.layers),
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "us_per_step": round(ms_step * 1000.0, 2),
        "us_per_layer": round(ms_step * 1000.0 / len(wl.layers), 2),
        "pct_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 K/V, fp32 accumulation",
        "data": "synthetic (seeded planted-logit indexer keys, counter-based N(0,1) K/V)",
        "config": {"workload": "%s: %d layers, B=%d, L=%d, Hq=%d, Hkv=%d, %d retrieval KV heads, "
                               "d=%d, r=%d, window=%d+%d sinks, p=%g" % (
                                   args.workload, len(wl.layers), wl.B, int(wl.seq_lens.max()),
                                   wl.Hq, wl.Hkv, nret, wl.d, wl.r, wl.window, wl.sinks, wl.p),
                   "global_batch": wl.B, "seq_len": int(wl.seq_lens.max()),
                   "parallelism": "single GPU", "graph": True, "rotations": 1},
        "bytes_per_step": bytes_step, "union_tokens": union,
        "roofline": {"kernel": "k_stage_a (mean over the %d layers with retrieval heads)" % a_n,
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "avg_us": round(a_us, 3), "algorithmic_bytes_per_launch": round(a_bytes)},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--context", type=int, default=0, metavar="L",
                    help="sequence length of the c3/c4 workload (default: its own)")
    ap.add_argument("--dense", action="store_true",
                    help="the dense counterpart on the same GPU: decode, C4's shape with every KV "
                         "head local and a window covering the whole context; with --prefill, "
                         "every KV head dense causal")
    ap.add_argument("--p", type=float, default=None)
    ap.add_argument("--topk", type=int, default=0,
                    help="fixed top-k through the histogram instead of top-p")
    ap.add_argument("--dtype", default="f16", choices=["f16", "bf16"],
                    help="cache dtype of the single-layer configs (fp16 or bf16; both run the fused "
                         "kernels)")
    ap.add_argument("--ret-window", action="store_true",
                    help="retrieval heads also attend to the sinks and the window")
    ap.add_argument("--with-append", action="store_true",
                    help="each step also runs the cache update of the new token "
                         "(indexer projections + K/V append), fused into the step")
    ap.add_argument("--separate-append", action="store_true",
                    help="with --with-append: the update as its own kernel (rtp_append_project) "
                         "before the step, instead of fused into it")
    ap.add_argument("--rotations", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measurement")
    ap.add_argument("--phases", action="store_true", help="print a per-phase breakdown")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the k_stage_a traffic summary from two rocprofv3 --pmc runs")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--prefill", type=int, default=0, metavar="L",
                    help="time the prefill of an L-token prompt instead of the decode step")
    args = ap.parse_args()
    if args.prefill:
        if args.gpus != 1:
            print("bench.py measures one GPU", file=sys.stderr, flush=True)
            sys.exit(2)
        bench_prefill(args)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                      args.copy_mib * 2 ** 20, TRAFFIC_FILE)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 3)
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import head_wise_sparse_rtp_amd as rtp
    import workloads

    dev = torch.device("cuda:0")
    kw = {} if args.p is None else {"p": args.p}
    if args.dtype != "f16":
        kw["dtype"] = args.dtype
    if args.context:
        if args.workload not in ("c3", "c4"):
            sys.exit("--context applies to the c3 and c4 workloads")
        kw["L"] = args.context
    if args.dense and not args.prefill:
        # a window of L positions (plus the sinks) holds every token: exact dense attention
        # for all 32 query heads, through the same fused step
        if args.workload != "c4" or args.topk or args.ret_window or args.with_append:
            sys.exit("--dense is the c4 shape alone")
        L = args.context or 1048576
        args.workload = "dense"
        wl = workloads.make_workload("dense", 1, [L], 32, 4, [[0, 0, 0, 0]], seed=4, window=L,
                                     device=dev, dtype=args.dtype)
    else:
        wl = workloads.make_config(args.workload, device=dev, **kw)
    if len(wl.layers) > 1:
        bench_layers(args, wl)
        return
    layer = wl.layers[0]
    sl = torch.as_tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    # the cache update's inputs reproduce the workload's own last row and q_idx, so the
    # timed step keeps the planted selection (the update's work does not depend on values)
    si = workloads.make_embedding_step_inputs(wl, device=dev) if args.with_append else None
    if si is not None:
        # the update is idempotent: apply it once, so that the byte count and every
        # rotated copy see the appended caches and the projected q_idx
        rtp.rtp_append_project(layer, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks,
                               si.q_pre, si.k_pre, si.Wq, si.Wk, si.k_new, si.v_new)
    bytes_step, detail = algorithmic_bytes(rtp, wl, layer, torch, args.topk, args.ret_window)
    touched = max(bytes_step, 1)
    R = args.rotations or max(1, math.ceil(512 * 2 ** 20 / touched))

    # R rotated copies of every input, one workspace and one output shared by all
    layers = [layer]
    for _ in range(R - 1):
        layers.append(workloads.Layer(layer.kv_is_retrieval, layer.q.clone(), layer.q_idx.clone(),
                                      layer.k_idx.clone(), layer.K_ret.clone(), layer.V_ret.clone(),
                                      layer.K_loc.clone(), layer.V_loc.clone(), layer.plans))
    steps = []
    apps = []
    ws = None
    out = None
    fused_app = si is not None and not args.separate_append
    for lay in layers:
        st = rtp.DecodeStep(lay, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window, wl.sinks, wl.p,
                            wl.bin_width, wl.scale_idx, wl.scale_attn, out=out, want_lse=False,
                            ws=ws, topk=args.topk, ret_window=args.ret_window,
                            append=si if fused_app else None)
        ws, out = st.ws, st.out
        steps.append(st)
        if si is not None and not fused_app:
            apps.append(rtp.AppendProject(lay, sl, wl.B, wl.Hq, wl.Hkv, wl.Lmax, wl.window,
                                          wl.sinks, si.q_pre, si.k_pre, si.Wq, si.Wk, si.k_new,
                                          si.v_new))

    def step(i):
        if apps:
            apps[i]()
        steps[i]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    h = hip()

    # ---- warmup + graph capture: one graph runs the R rotations in order (a decode loop
    # captures its layers the same way); a second graph holds the K % R remaining steps
    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()
    K = args.steps
    g_full = g_rest = None
    if not args.no_graph:
        g_full = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_full):
            for i in range(R):
                step(i)
        if K % R:
            g_rest = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_rest):
                for i in range(K % R):
                    step(i)
        for _ in range(max(1, args.warmup // R)):
            g_full.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly K steps, repeated REPEATS times; the median is reported ----
    e0, e1 = make_events(h, 2)
    rep_ms = []
    for _ in range(REPEATS):
        torch.cuda.synchronize()
        h.hipEventRecord(e0, ctypes.c_void_p(stream.cuda_stream))
        if g_full is not None:
            for _ in range(K // R):
                g_full.replay()
            if g_rest is not None:
                g_rest.replay()
        else:
            for i in range(K):
                step(i % R)
        h.hipEventRecord(e1, ctypes.c_void_p(stream.cuda_stream))
        h.hipEventSynchronize(e1)
        torch.cuda.synchronize()
        rep_ms.append(elapsed_ms(h, e0, e1) / K)
    ms_step = sorted(rep_ms)[len(rep_ms) // 2]

    # ---- per-kernel durations, timed live with HIP events on the launch stream ----
    # events [0]/[1] are bound to stage A's execution (indexer score + chunk histograms)
    # and [2]/[3] to stage B's (selection + sparse and window attention); two more,
    # recorded on the stream around the call, time the whole eager step.  Each profiled
    # step is queued behind a short busy kernel, so that all of its commands wait in the
    # queue when the GPU reaches them and the events time the kernels, not the host-side
    # enqueue.
    ph = {"stageA_score_hist": 0.0, "stageB_select_attend": 0.0, "eager_step": 0.0}
    has_ret = bool(layer.ret_heads)
    evs = make_events(h, 4, HIP_EVENT_TIMING_NO_FENCE)
    ew = make_events(h, 2, HIP_EVENT_TIMING_NO_FENCE)
    torch.cuda.synchronize()
    for k in range(K):
        st = steps[k % R]
        torch.cuda._sleep(200000)  # a spinning kernel (tens of us, touches no memory)
        h.hipEventRecord(ew[0], ctypes.c_void_p(stream.cuda_stream))
        st.profiled([e.value for e in evs])
        h.hipEventRecord(ew[1], ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        if has_ret:
            ph["stageA_score_hist"] += elapsed_ms(h, evs[0], evs[1])
        ph["stageB_select_attend"] += elapsed_ms(h, evs[2], evs[3])
        ph["eager_step"] += elapsed_ms(h, ew[0], ew[1])
    ph = {k: v / K * 1000.0 for k, v in ph.items()}  # microseconds
    if apps:
        # the cache update alone, timed the same way
        tot = 0.0
        for k in range(K):
            torch.cuda._sleep(200000)
            h.hipEventRecord(evs[0], ctypes.c_void_p(stream.cuda_stream))
            apps[k % R]()
            h.hipEventRecord(evs[1], ctypes.c_void_p(stream.cuda_stream))
            torch.cuda.synchronize()
            tot += elapsed_ms(h, evs[0], evs[1])
        ph["append_project"] = tot / K * 1000.0

    def roofline(kernel, desc, us, nbytes):
        gbs = nbytes / (us * 1e-6) / 1e9 if us > 0 else 0.0
        wl_key = args.workload if not (args.topk or args.context or args.dtype != "f16"
                                       or args.ret_window or si is not None) else None
        return {"kernel": "%s (%s)" % (kernel, desc), "bound": "hbm", "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                # the counters were taken on the fp16 top-p step of the workload at its own
                # length
                "traffic": measured_traffic(wl_key, kernel) if wl_key else None,
                "avg_us": round(us, 3), "algorithmic_bytes_per_launch": nbytes}

    kern = {}
    if has_ret:
        kern["k_stage_a"] = roofline("k_stage_a", "indexer score on MFMA + 256-bin chunk "
                                     "histograms; algorithmic bytes: the indexer keys",
                                     ph["stageA_score_hist"], detail["kidx"])
    kern["k_stage_b"] = roofline("k_stage_b", "selection + sparse attention + window attention; "
                                 "algorithmic bytes: the selected and the window K/V rows",
                                 ph["stageB_select_attend"],
                                 detail["sparse_kv"] + detail["window_kv"])
    dominant = max(kern, key=lambda k: kern[k]["avg_us"])

    ceiling = hbm_read_ceiling(torch) if not args.skip_ceiling else None
    value = bytes_step / (ms_step * 1e-3) / 1e9
    res = {
        "metric": decode_metric(wl.Lmax),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1000.0, 2),
        "repeats": REPEATS,
        "repeat_us_per_step": [round(x * 1000.0, 3) for x in rep_ms],
        "pct_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "%s K/V, fp32 accumulation" % args.dtype,
        "data": "synthetic (seeded planted-logit indexer keys, counter-based N(0,1) K/V)",
        "config": {"workload": "%s: B=%d, L=%d, Hq=%d, Hkv=%d (retrieval %s), d=%d, r=%d, "
                               "window=%d+%d sinks, %s" % (
                                   args.workload, wl.B, int(wl.seq_lens.max()), wl.Hq, wl.Hkv,
                                   layer.ret_heads, wl.d, wl.r, wl.window, wl.sinks,
                                   "top-k k=%d" % args.topk if args.topk else "p=%g" % wl.p),
                   "global_batch": wl.B, "seq_len": int(wl.seq_lens.max()),
                   "parallelism": "single GPU", "graph": g_full is not None, "rotations": R,
                   "with_append": ("fused" if si is not None and not args.separate_append
                                   else "separate kernel" if si is not None else False),
                   "retrieval_window": bool(args.ret_window)},
        "bytes_per_step": bytes_step,
        "bytes_detail": {k: v for k, v in detail.items() if k not in ("sel_tokens", "sel_mass")},
        "sel_tokens_per_head": detail["sel_tokens"],
        "sel_mass_per_head": detail["sel_mass"],
        "roofline": kern[dominant],
        "kernels": kern,
        "phases_us": {k: round(v, 3) for k, v in ph.items()},
    }
    if ceiling is not None:
        res["hbm_read_ceiling"] = ceiling
        res["pct_of_read_ceiling"] = round(100.0 * value / ceiling["value"], 2)
    if not args.skip_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, bytes_step, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
