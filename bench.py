"""Benchmark of the activation-sparse gated FFN forward on one MI355X.

A step is one sparse forward of the whole hot path over one batch of
synthetic tokens: twell_pack (gate GEMM + TwELL epilogue), sparse_ffn_fwd
(fused up*gate -> down over the packed nonzeros) and hybrid_route (routing scan
+ dense fallback of the overflowing rows).  The same-GPU dense gated FFN
(dense_ffn_ref) is timed beside it for the speed-up.  Inputs are resident in
HBM before the timed region starts.

Prints one JSON line (metric, value = sparse FFN tokens/s, roofline of the
dominant kernel, CPU oracle baseline, per-kernel times, speed-up over dense).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="prefill_1pct")
    p.add_argument("--beta", type=float, default=None, help="override the gate bias -beta")
    p.add_argument("--cap", type=int, default=None, help="override the TwELL capacity")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=None,
                   help="rows of the CPU oracle sample (default: whole batch, at most 4096)")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-backward", action="store_true",
                   help="skip timing the sparse backward (sparse_ffn_bwd) and the dense one")
    p.add_argument("--no-l1", action="store_true",
                   help="skip timing twell_pack_l1 (the L1 regulariser fused into the gate epilogue)")
    p.add_argument("--no-conversion", action="store_true",
                   help="skip the separate-conversion baseline (gate GEMM storing z, then "
                        "standalone TwELL and row-ELLPACK conversions)")
    p.add_argument("--cold-steps", type=int, default=10,
                   help="steps of the cold pass (a 512 MiB read between steps evicts the "
                        "Infinity Cache); 0 skips it")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the peak probes (measured HBM bandwidth and bf16 MFMA rate)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run device copies of MIB MiB (reference for the HBM byte "
                        "counters of a profiling run) and exit")
    return p.parse_args()


def measured_peaks() -> dict:
    """Achievable HBM bandwidth and bf16 MFMA rate on this GPU, from the
    library's probe kernels (best of five timed calls each): a read-only pass
    and a copy over 1 GiB buffers (four times the Infinity Cache), and 16
    independent MFMA chains per wave on 16 workgroups per CU."""
    import torch
    from activation_sparse_feed_amd import sffn
    E = torch.cuda.Event

    def best(fn, reps=5):
        fn()
        times = []
        for _ in range(reps):
            a, b = E(enable_timing=True), E(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        return min(times)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    wg_hbm = nbytes // (16 * 4 * 256)  # one pass of four 16-byte chunks per lane
    t_read = best(lambda: sffn.probe_hbm(src, None, workgroups=wg_hbm))
    t_copy = best(lambda: sffn.probe_hbm(src, dst, workgroups=wg_hbm))
    ok_copy = bool(torch.equal(src[:1 << 20], dst[:1 << 20]))
    del src, dst
    wgs, iters = 256 * 16, 1024
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    t_mfma = best(lambda: sffn.probe_mfma(out, iters))
    ok_mfma = bool(torch.all(out == 2048.0 * iters).item())
    flops = wgs * 4 * 16 * iters * 16384.0
    del out
    # cached loads: every workgroup re-reads one 2 MiB window (resident in each
    # XCD's L2), 8 workgroups per CU
    win, reps, cwg = 2 << 20, 24, 2048
    buf = torch.ones(win // 4, dtype=torch.int32, device="cuda")
    t_cached = best(lambda: sffn.probe_cached(buf, win, reps, cwg))
    del buf
    return {"hbm_read_gb_s": nbytes / t_read / 1e9, "hbm_copy_gb_s": 2 * nbytes / t_copy / 1e9,
            "mfma_bf16_tflop_s": flops / t_mfma / 1e12, "checks_passed": ok_copy and ok_mfma,
            "cached_load_gb_s": float(cwg) * reps * win / t_cached / 1e9,
            "probe": "sffn_probe_hbm over 1 GiB, 65536 workgroups (read-only; copy counts read + write), "
                     "sffn_probe_mfma 4096 workgroups x 4 waves x 16 chains x 1024 MFMAs, "
                     "sffn_probe_cached 2048 workgroups x 24 passes over one 2 MiB window, 8 loads in flight per lane"}


def gather_probe(wu, wd, idx_live, flush) -> dict:
    """The bare row gather of the sparse step: the wu_t and wd rows of the
    distinct active columns, read once by sffn_probe_gather with no arithmetic,
    warm (rows cached by a previous pass) and cold (a 512 MiB read in between
    evicts the Infinity Cache)."""
    import torch
    from activation_sparse_feed_amd import sffn
    rows = torch.unique(idx_live.to(torch.int64)).to(torch.int32)
    row_bytes = wu.shape[1] * wu.element_size()
    if rows.numel() == 0 or row_bytes not in (1024, 2048, 4096, 8192, 16384):
        return None
    E = torch.cuda.Event

    def timed(cold):
        ts = []
        for _ in range(5):
            if cold:  # evict, then one gather
                sffn.probe_hbm(flush, None, workgroups=4096)
            a, b = E(enable_timing=True), E(enable_timing=True)
            reps = 1 if cold else 10  # warm: back-to-back gathers of cached rows
            a.record()
            for _ in range(reps):
                sffn.probe_gather(wu, wd, rows, row_bytes, max_row=top)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3 / reps)
        return min(ts)
    nb = 2.0 * rows.numel() * row_bytes
    top = int(rows.max().item())
    tw, tc = timed(False), timed(True)
    return {"rows": int(rows.numel()), "bytes": nb, "warm_us": tw * 1e6, "cold_us": tc * 1e6,
            "warm_gb_s": nb / tw / 1e9, "cold_gb_s": nb / tc / 1e9}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_twell_pack_prefill_1pct.md")
GATE_SOURCES = ("activation_sparse_feed_amd/csrc/twell_gate.hip",
                "activation_sparse_feed_amd/csrc/twell_emit.cuh",
                "activation_sparse_feed_amd/csrc/gemm_v2.cuh",
                "activation_sparse_feed_amd/csrc/exact.cuh",
                "activation_sparse_feed_amd/csrc/common.cuh")


SPARSE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sparse_prefill_1pct.md")
SPARSE_SOURCES = ("activation_sparse_feed_amd/csrc/sparse.hip",
                  "activation_sparse_feed_amd/csrc/common.cuh")


def source_digest(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gate_source_digest() -> str:
    return source_digest(GATE_SOURCES)


def sparse_source_digest() -> str:
    return source_digest(SPARSE_SOURCES)


def measured_traffic(workload: str, path: str = TRAFFIC_FILE, digest=gate_source_digest):
    """HBM bytes per launch of a kernel from its stored counter summary (its
    'key: value' lines), or None when the counters were taken on another
    workload or on different kernel sources."""
    try:
        with open(path) as f:
            kv = dict(line.split(": ", 1) for line in f.read().splitlines()
                      if line.count(": ") == 1 and " " not in line.split(": ", 1)[0])
    except OSError:
        return None
    if kv.get("workload") != workload or kv.get("source_digest") != digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gpu_clocks():
    """Current DPM clock levels of the GPU from sysfs (the entries marked '*'
    in pp_dpm_sclk / pp_dpm_mclk / pp_dpm_fclk); None where unavailable.  Read
    as plain files: no helper program is started from this GPU process."""
    import glob
    out = {}
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_*clk")):
        try:
            with open(path) as f:
                cur = [ln.split(":", 1)[1].strip(" *\n") for ln in f if ln.rstrip().endswith("*")]
        except OSError:
            continue
        if cur:
            card = path.split("/")[4]
            out[f"{card}.{os.path.basename(path)[7:]}"] = cur[0]
    return out or None


def cpu_baseline(inp, rows: int) -> dict:
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    w = inp.workload
    sel = np.arange(min(rows, w.T))
    x = inp.rows_f64("x", sel)
    wg, wu, wd = inp.as_f64("wg_t"), inp.as_f64("wu_t"), inp.as_f64("wd")
    # repeat the whole sample until about 10 s of host time have passed (at most 30
    # passes), so that the rate is not one short measurement
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.sparse_forward(x, wg, inp.b_g, wu, wd, w.tile, w.cap)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 30:
            break
    # the oracle's dense FFN on the same rows (fp64 BLAS), for context
    t1 = time.perf_counter()
    oracle.ffn_dense(x, wg, inp.b_g, wu, wd)
    t_dense = time.perf_counter() - t1
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": passes * len(sel) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(sel)} of {w.T} tokens of {w.name}, {passes} float64 sparse forwards "
                      f"(gate with exact sign, TwELL pack, route, fused sum), {dt:.2f} s",
            "cpu_model": cpu, "os_cpu_count": os.cpu_count(),
            "oracle_dense_tokens_per_s": len(sel) / t_dense}


def training_memory(w, x, wg, b, wu, wd, wg_norms, gy) -> dict:
    """Device-allocator bytes of one forward + backward step, sparse against
    dense.  x, the weights, gy, y and the gradient outputs are allocated first
    (both paths need them) and are not counted.  For each path: the bytes the
    forward keeps for the backward (allocated after the forward, its
    transients freed) and the peak over the step (forward transients,
    workspaces, backward transients).
      sparse: twell_pack, sparse_ffn_fwd, hybrid_route; the forward keeps the
              TwELL arrays and the routed list; sparse_ffn_bwd with its
              workspace sized for the routed rows the forward produced.
      dense:  the gated FFN on hipBLASLt GEMMs keeping h and u ([d_ff, T]
              bf16), then the dense backward (six GEMMs).
    """
    import torch

    from activation_sparse_feed_amd import sffn
    dt = x.dtype
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    y = torch.empty_like(x)
    gx = torch.empty_like(x)
    gw3 = [torch.empty((w.d_ff, w.d_model), device="cuda") for _ in range(3)]
    gbv = torch.empty(w.d_ff, device="cuda")
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()

    def mib(v):
        return v / 2 ** 20

    # sparse
    torch.cuda.reset_peak_memory_stats()
    ffn = sffn.SparseFFN(w.T, w.d_model, w.d_ff, w.cap, dt)
    s = ffn.shape
    sffn.twell_pack(s, x, wg, b, ffn.count, ffn.idx, ffn.val, ffn.ws_pack, wg_norms)
    sffn.sparse_ffn_fwd(s, x, wu, wd, ffn.count, ffn.idx, ffn.val, y, ffn.ws_sparse)
    sffn.hybrid_route(s, x, wg, b, wu, wd, ffn.count, ffn.routed, ffn.n_routed, ffn.ws_hybrid, y)
    saved = {k: getattr(ffn, k) for k in ("count", "idx", "val", "routed", "n_routed")}
    n_r = int(saved["n_routed"].item())
    del ffn
    torch.cuda.synchronize()
    sp_saved = torch.cuda.memory_allocated() - base
    ws = torch.empty(max(sffn.backward_workspace_bytes(s, n_r), 16), dtype=torch.uint8,
                     device="cuda")
    sffn.sparse_ffn_bwd(s, x, wg, b, wu, wd, saved["count"], saved["idx"], saved["val"],
                        saved["routed"], saved["n_routed"], gy, gx, *gw3, gbv, ws, wg_norms,
                        max_routed=n_r)
    torch.cuda.synchronize()
    sp_peak = torch.cuda.max_memory_allocated() - base
    ws_bytes = ws.numel()
    del ws, saved
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # dense
    torch.cuda.reset_peak_memory_stats()
    zT = (torch.nn.functional.linear(x, wg) + b.to(dt)).t().contiguous()
    uT = torch.nn.functional.linear(x, wu).t().contiguous()
    hT = torch.relu(zT)
    del zT
    aT = hT * uT
    torch.mm(aT.t().contiguous(), wd, out=y)
    del aT
    torch.cuda.synchronize()
    de_saved = torch.cuda.memory_allocated() - base
    de_fwd_peak = torch.cuda.max_memory_allocated() - base
    wg_tt, wu_tt = wg.t().contiguous(), wu.t().contiguous()  # prepared weights, not counted
    pre = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    gyT = gy.t().contiguous()
    gaT = torch.mm(wd, gyT)
    gzT = torch.where(hT > 0, gaT * uT, torch.zeros_like(gaT))
    guT = gaT * hT
    del gaT
    gx.copy_((torch.mm(wg_tt, gzT) + torch.mm(wu_tt, guT)).t())
    gw3[0].copy_(torch.mm(gzT, x))
    gw3[1].copy_(torch.mm(guT, x))
    gw3[2].copy_(torch.mm(hT * uT, gy))
    gbv.copy_(gzT.float().sum(1))
    torch.cuda.synchronize()
    de_peak = max(torch.cuda.max_memory_allocated() - pre + de_saved, de_fwd_peak)
    del gzT, guT, gyT, hT, uT, wg_tt, wu_tt
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"sparse_saved_MiB": mib(sp_saved), "sparse_peak_MiB": mib(sp_peak),
            "sparse_backward_workspace_MiB": mib(ws_bytes), "routed_rows": n_r,
            "dense_saved_MiB": mib(de_saved), "dense_peak_MiB": mib(de_peak),
            "saved_reduction": 1.0 - sp_saved / de_saved if de_saved else None,
            "peak_reduction": 1.0 - sp_peak / de_peak if de_peak else None,
            "note": "device allocator (torch.cuda.memory_allocated / max_memory_allocated) over "
                    "one forward + backward; x, weights, gy, y and the gradient outputs excluded"}


def backward_ok(w) -> bool:
    """Shapes sparse_ffn_bwd takes: bf16 up to d_model 4096 (any multiple of
    8), float32 up to 2048."""
    return w.d_model % 8 == 0 and w.d_model <= (4096 if w.dtype == "bf16" else 2048)


def d_model_ok(d_model: int) -> bool:
    """The separate-conversion calls need d_model % 32 == 0."""
    return d_model % 32 == 0


def nnz_live_of(count, cap: int) -> int:
    return int(count.clamp(max=cap).sum().item()) if cap > 0 else 0


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the activation-"
              "sparse FFN path is built and measured for a single MI355X.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from activation_sparse_feed_amd import sffn, workloads as wl

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": max(1, args.steps)}))
        return 0

    w = wl.WORKLOADS[args.workload]
    if args.cap is not None:
        w = w.replace(cap=args.cap)
    inp = wl.generate(w, beta=args.beta)
    beta = w.beta if args.beta is None else args.beta
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, wg, wu, wd = dev(inp.x), dev(inp.wg_t), dev(inp.wu_t), dev(inp.wd)
    b = torch.from_numpy(inp.b_g).cuda()
    ffn = sffn.SparseFFN(w.T, w.d_model, w.d_ff, w.cap, dt)
    dense = sffn.DenseFFN(w.T, w.d_model, w.d_ff, dt)
    s = ffn.shape
    # gate-weight row norms: a property of the weights, computed once (like
    # any weight preparation at load time), outside the timed region
    wg_norms = ffn.weight_norms(wg)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        ffn.forward(x, wg, b, wu, wd, wg_norms)
        if not args.no_dense:
            dense.forward(x, wg, b, wu, wd)
    torch.cuda.synchronize()

    # ---- timed sparse forward: exactly K steps between two synchronisations,
    # nothing else on the stream (the value)
    K = args.steps
    E = torch.cuda.Event
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        sffn.twell_pack(s, x, wg, b, ffn.count, ffn.idx, ffn.val, ffn.ws_pack, wg_norms)
        sffn.sparse_ffn_fwd(s, x, wu, wd, ffn.count, ffn.idx, ffn.val, ffn.y, ffn.ws_sparse)
        sffn.hybrid_route(s, x, wg, b, wu, wd, ffn.count, ffn.routed, ffn.n_routed,
                          ffn.ws_hybrid, ffn.y)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K

    # ---- the same K steps again with HIP events around each call, on the
    # stream the kernels run on (per-call times, roofline, percentiles)
    ev = [[E(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record()
        sffn.twell_pack(s, x, wg, b, ffn.count, ffn.idx, ffn.val, ffn.ws_pack, wg_norms)
        ev[i][1].record()
        sffn.sparse_ffn_fwd(s, x, wu, wd, ffn.count, ffn.idx, ffn.val, ffn.y, ffn.ws_sparse)
        ev[i][2].record()
        sffn.hybrid_route(s, x, wg, b, wu, wd, ffn.count, ffn.routed, ffn.n_routed,
                          ffn.ws_hybrid, ffn.y)
        ev[i][3].record()
    torch.cuda.synchronize()
    t_gate = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]))
    t_sparse = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]))
    t_hybrid = float(np.mean([ev[i][2].elapsed_time(ev[i][3]) for i in range(K)]))
    t_events = float(np.mean([ev[i][0].elapsed_time(ev[i][3]) for i in range(K)]))
    step_ev = np.array([ev[i][0].elapsed_time(ev[i][3]) for i in range(K)])

    # ---- cold pass: the same three calls after reading a 512 MiB buffer, which
    # evicts the 256 MB Infinity Cache with clean lines (a write would leave
    # dirty lines whose write-back lands inside the timed calls), so the weights
    # come from HBM; the dense reference is timed the same way
    cold = None
    if args.cold_steps > 0:
        flush = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
        sink = torch.zeros((), dtype=torch.int64, device="cuda")
        nc = args.cold_steps
        # one event pair around each whole step (as around each dense call) ...
        sev = [[E(enable_timing=True) for _ in range(2)] for _ in range(nc)]
        for i in range(nc):
            sink += flush.sum()
            sev[i][0].record()
            sffn.twell_pack(s, x, wg, b, ffn.count, ffn.idx, ffn.val, ffn.ws_pack, wg_norms)
            sffn.sparse_ffn_fwd(s, x, wu, wd, ffn.count, ffn.idx, ffn.val, ffn.y, ffn.ws_sparse)
            sffn.hybrid_route(s, x, wg, b, wu, wd, ffn.count, ffn.routed, ffn.n_routed,
                              ffn.ws_hybrid, ffn.y)
            sev[i][1].record()
        # ... and a pass with events around each call for the per-call times
        cev = [[E(enable_timing=True) for _ in range(4)] for _ in range(nc)]
        for i in range(nc):
            sink += flush.sum()
            cev[i][0].record()
            sffn.twell_pack(s, x, wg, b, ffn.count, ffn.idx, ffn.val, ffn.ws_pack, wg_norms)
            cev[i][1].record()
            sffn.sparse_ffn_fwd(s, x, wu, wd, ffn.count, ffn.idx, ffn.val, ffn.y, ffn.ws_sparse)
            cev[i][2].record()
            sffn.hybrid_route(s, x, wg, b, wu, wd, ffn.count, ffn.routed, ffn.n_routed,
                              ffn.ws_hybrid, ffn.y)
            cev[i][3].record()
        dev_ = [[E(enable_timing=True) for _ in range(2)] for _ in range(nc)]
        if not args.no_dense:
            for i in range(nc):
                sink += flush.sum()
                dev_[i][0].record()
                dense.forward(x, wg, b, wu, wd)
                dev_[i][1].record()
        torch.cuda.synchronize()
        del flush
        cm = lambda a, z: float(np.median([cev[i][a].elapsed_time(cev[i][z]) for i in range(nc)]))
        cold = {"steps": nc, "twell_pack_ms": cm(0, 1), "sparse_ffn_fwd_ms": cm(1, 2),
                "hybrid_route_ms": cm(2, 3),
                "step_ms": float(np.median([sev[i][0].elapsed_time(sev[i][1]) for i in range(nc)]))}
        if not args.no_dense:
            cold["dense_ffn_ref_ms"] = float(np.median([dev_[i][0].elapsed_time(dev_[i][1])
                                                        for i in range(nc)]))
            cold["speedup_vs_dense"] = cold["dense_ffn_ref_ms"] / cold["step_ms"]

    # ---- dense reference
    t_dense = None
    if not args.no_dense:
        d0, d1 = E(enable_timing=True), E(enable_timing=True)
        torch.cuda.synchronize()
        d0.record()
        for _ in range(K):
            dense.forward(x, wg, b, wu, wd)
        d1.record()
        torch.cuda.synchronize()
        t_dense = d0.elapsed_time(d1) / K

    # ---- sanity line: the same dense FFN from torch's own GEMMs (hipBLASLt)
    t_torch = None
    if not args.no_dense and w.dtype == "bf16":
        def torch_ffn():
            z = torch.nn.functional.linear(x, wg) + b.to(dt)
            u = torch.nn.functional.linear(x, wu)
            return torch.mm(torch.relu(z) * u, wd)
        for _ in range(3):
            torch_ffn()
        t0_, t1_ = E(enable_timing=True), E(enable_timing=True)
        torch.cuda.synchronize()
        t0_.record()
        for _ in range(K):
            torch_ffn()
        t1_.record()
        torch.cuda.synchronize()
        t_torch = t0_.elapsed_time(t1_) / K

    # ---- separate-conversion baseline: the gate GEMM stores the float32
    # pre-activation z, then standalone kernels build TwELL and a classic
    # row-wise ELLPACK padded to the longest row (not part of the step above)
    conversion = None
    # (measured where twell_pack runs the same GEMM, more than 64 tokens)
    if not args.no_conversion and w.dtype == "bf16" and d_model_ok(w.d_model) and w.T > 64:
        eb_ = 2
        z = torch.empty((w.T, w.d_ff), dtype=torch.float32, device="cuda")
        ws_c = sffn.alloc_workspace(s, sffn.WS_CONVERT)
        tw = sffn.alloc_twell(s)
        width = int(ffn.count.to(torch.int64).sum(1).max().item())
        ell = sffn.alloc_ell(s, width)
        def conv_pass():
            sffn.gate_preact(s, x, wg, b, z)
            sffn.twell_from_preact(s, z, x, wg, b, *tw, ws_c, wg_norms)
        for _ in range(2):
            conv_pass()
            sffn.ell_from_preact(s, width, z, x, wg, b, *ell, ws_c, wg_norms)
        torch.cuda.synchronize()
        # K passes back to back (as the step above), then per-call events
        c0, c1 = E(enable_timing=True), E(enable_timing=True)
        c0.record()
        for _ in range(K):
            conv_pass()
        c1.record()
        torch.cuda.synchronize()
        t_two_pass = c0.elapsed_time(c1) / K
        cv = [[E(enable_timing=True) for _ in range(4)] for _ in range(K)]
        for i in range(K):
            cv[i][0].record()
            sffn.gate_preact(s, x, wg, b, z)
            cv[i][1].record()
            sffn.twell_from_preact(s, z, x, wg, b, *tw, ws_c, wg_norms)
            cv[i][2].record()
            sffn.ell_from_preact(s, width, z, x, wg, b, *ell, ws_c, wg_norms)
            cv[i][3].record()
        # the fused call timed the same way, right after
        f0, f1 = E(enable_timing=True), E(enable_timing=True)
        f0.record()
        for _ in range(K):
            sffn.twell_pack(s, x, wg, b, ffn.count, ffn.idx, ffn.val, ffn.ws_pack, wg_norms)
        f1.record()
        torch.cuda.synchronize()
        t_fused = f0.elapsed_time(f1) / K
        cmean = lambda a, e: float(np.mean([cv[i][a].elapsed_time(cv[i][e]) for i in range(K)]))
        t_pre, t_conv, t_ell = cmean(0, 1), cmean(1, 2), cmean(2, 3)
        cnt = ffn.count.to(torch.int64)
        live_c = torch.arange(max(w.cap, 1), device="cuda")[None, None, :] < torch.clamp(cnt, max=w.cap)[:, :, None]
        same = bool(torch.equal(tw[0], ffn.count)) and bool(torch.equal(
            torch.where(live_c, tw[1].to(torch.int64), -1), torch.where(live_c, ffn.idx.to(torch.int64), -1)))
        nnz_all = int(cnt.sum().item())
        nt_ = w.d_ff // w.tile
        z_bytes = 4.0 * w.T * w.d_ff
        conversion = {
            "fused_twell_pack_ms": t_fused,
            "two_pass_ms": t_two_pass,
            "two_pass_over_fused": t_two_pass / t_fused,
            "gate_preact_ms": t_pre, "twell_from_preact_ms": t_conv, "ell_from_preact_ms": t_ell,
            "z_bytes": z_bytes,
            "twell_from_preact_gb_per_s": (z_bytes + w.T * nt_ * 2 + nnz_live_of(cnt, w.cap) * (2 + eb_)) / (t_conv * 1e-3) / 1e9,
            "ell_from_preact_gb_per_s": (z_bytes + w.T * 2 + nnz_all * (2 + eb_)) / (t_ell * 1e-3) / 1e9,
            "twell_matches_fused": same,
            "ell_width": width,
            "storage_bytes": {"live_entries": nnz_all * (2 + eb_),
                              "twell": w.T * nt_ * 2 + w.T * nt_ * w.cap * (2 + eb_),
                              "row_ellpack_padded_to_longest_row": w.T * 2 + w.T * width * (2 + eb_),
                              "dense_h": w.T * w.d_ff * eb_},
        }
        del z, tw, ell, ws_c

    # ---- the column-union organisation of the fused kernel (the token block's
    # distinct columns staged once in LDS) on the same TwELL, against the row
    # walk of sparse_ffn_fwd: K calls each back to back, then y compared
    union = None
    if w.dtype == "bf16" and w.d_model in (512, 1024, 2048, 4096) and w.cap <= 32:
        y_u = torch.empty_like(ffn.y)
        ffn.forward(x, wg, b, wu, wd, wg_norms)
        for _ in range(2):
            sffn.sparse_ffn_fwd_union(s, x, wu, wd, ffn.count, ffn.idx, ffn.val, y_u)
        u0, u1, u2 = E(enable_timing=True), E(enable_timing=True), E(enable_timing=True)
        torch.cuda.synchronize()
        u0.record()
        for _ in range(K):
            sffn.sparse_ffn_fwd_union(s, x, wu, wd, ffn.count, ffn.idx, ffn.val, y_u)
        u1.record()
        for _ in range(K):
            sffn.sparse_ffn_fwd(s, x, wu, wd, ffn.count, ffn.idx, ffn.val, ffn.y, ffn.ws_sparse)
        u2.record()
        torch.cuda.synchronize()
        t_union, t_walk = u0.elapsed_time(u1) / K, u1.elapsed_time(u2) / K
        keep = torch.ones(w.T, dtype=torch.bool, device="cuda")
        keep[ffn.routed[:int(ffn.n_routed.item())].long()] = False
        yu_, yw_ = y_u[keep].float(), ffn.y[keep].float()
        cnt_u = ffn.count.to(torch.int64)
        live_u = nnz_live_of(cnt_u[keep], w.cap)
        union = {"sparse_ffn_fwd_union_ms": t_union, "sparse_ffn_fwd_ms": t_walk,
                 "union_over_row_walk": t_union / t_walk,
                 "union_gflop_per_s": 4.0 * w.d_model * live_u / (t_union * 1e-3) / 1e9,
                 "y_rel_diff_vs_row_walk": float(((yu_ - yw_).norm() / yw_.norm().clamp_min(1e-30)).item())}
        del y_u

    # ---- the L1 regulariser fused into the gate epilogue: twell_pack_l1 against
    # twell_pack, K calls each back to back
    l1 = None
    if not args.no_l1:
        l1_out = torch.empty(1, dtype=torch.float32, device="cuda")
        ws_l1 = sffn.alloc_workspace(s, sffn.WS_PACK_L1)
        tw1 = sffn.alloc_twell(s)
        lam = 1.0
        for _ in range(2):
            sffn.twell_pack_l1(s, x, wg, b, *tw1, lam, l1_out, ws_l1, wg_norms)
        l0, l1e, l2e = E(enable_timing=True), E(enable_timing=True), E(enable_timing=True)
        torch.cuda.synchronize()
        l0.record()
        for _ in range(K):
            sffn.twell_pack_l1(s, x, wg, b, *tw1, lam, l1_out, ws_l1, wg_norms)
        l1e.record()
        for _ in range(K):
            sffn.twell_pack(s, x, wg, b, ffn.count, ffn.idx, ffn.val, ffn.ws_pack, wg_norms)
        l2e.record()
        torch.cuda.synchronize()
        t_l1, t_p = l0.elapsed_time(l1e) / K, l1e.elapsed_time(l2e) / K
        l1 = {"lambda": lam, "value": float(l1_out.item()), "twell_pack_l1_ms": t_l1,
              "twell_pack_ms": t_p, "overhead": t_l1 / t_p - 1.0}
        del ws_l1, tw1

    # ---- backward through TwELL and the routing (sparse_ffn_bwd), against a
    # dense backward from torch's GEMMs (hipBLASLt) given the forward's dense
    # activations; both after the same forward, K calls each
    backward = None
    if not args.no_backward and backward_ok(w):
        gy = dev(wl.upstream_grad(w))
        ws_b = sffn.alloc_workspace(s, sffn.WS_BACKWARD)
        gx = torch.empty_like(x)
        gw3 = [torch.empty((w.d_ff, w.d_model), device="cuda") for _ in range(3)]
        gbv = torch.empty(w.d_ff, device="cuda")
        ffn.forward(x, wg, b, wu, wd, wg_norms)

        def bwd():
            sffn.sparse_ffn_bwd(s, x, wg, b, wu, wd, ffn.count, ffn.idx, ffn.val, ffn.routed,
                                ffn.n_routed, gy, gx, *gw3, gbv, ws_b, wg_norms)
        # dense backward from activations saved in [d_ff, T] layout and weights
        # prepared in [d_model, d_ff] layout (one-time), so that no GEMM
        # operand is a transposed view
        wg_tt, wu_tt = wg.t().contiguous(), wu.t().contiguous()
        zT = (torch.nn.functional.linear(x, wg) + b.to(dt)).t().contiguous()
        uT = torch.nn.functional.linear(x, wu).t().contiguous()
        actT = zT > 0
        hT = torch.where(actT, zT, torch.zeros_like(zT))

        def dense_bwd():
            gyT = gy.t().contiguous()
            gaT = torch.mm(wd, gyT)
            gzT = torch.where(actT, gaT * uT, torch.zeros_like(gaT))
            guT = gaT * hT
            gx_d = (torch.mm(wg_tt, gzT) + torch.mm(wu_tt, guT)).t().contiguous()
            return (gx_d, torch.mm(gzT, x), torch.mm(guT, x), torch.mm(hT * uT, gy),
                    gzT.float().sum(1))
        for _ in range(2):
            bwd()
            dense_bwd()
        b0, b1, b2 = E(enable_timing=True), E(enable_timing=True), E(enable_timing=True)
        torch.cuda.synchronize()
        b0.record()
        for _ in range(K):
            bwd()
        b1.record()
        for _ in range(K):
            dense_bwd()
        b2.record()
        torch.cuda.synchronize()
        t_b, t_db = b0.elapsed_time(b1) / K, b1.elapsed_time(b2) / K
        backward = {"sparse_ffn_bwd_ms": t_b, "torch_dense_backward_ms": t_db,
                    "speedup_vs_torch_dense": t_db / t_b,
                    "weight_grad_bytes": 3.0 * w.d_ff * w.d_model * 4,
                    "note": f"dense: 6 hipBLASLt {w.dtype} GEMMs from saved dense activations"}
        del ws_b, gw3, zT, uT, hT, actT, wg_tt, wu_tt
        # measured memory of a training step: what the forward keeps for the
        # backward and the peak, sparse (TwELL + routed list) against dense (h, u)
        backward["memory"] = training_memory(w, x, wg, b, wu, wd, wg_norms, gy)

    count = ffn.count.to(torch.int64)
    nnz_live = int(torch.clamp(count, max=w.cap).sum().item()) if w.cap > 0 else 0
    n_routed = int(ffn.n_routed.item())
    nnz_total = int(count.sum().item())

    T, d, n = w.T, w.d_model, w.d_ff
    eb = 2 if w.dtype == "bf16" else 4
    gate_flop = 2.0 * T * d * n
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    gate_tflops = gate_flop / (t_gate * 1e-3) / 1e12
    # the gate's algorithmic bytes: x and wg_t once, bias, count, the live TwELL entries
    gate_bytes = (T * d + n * d) * eb + 4.0 * n + T * (n // 128) * 2
    # bound by the matrix cores when its arithmetic intensity is above the
    # machine balance (peak flops / HBM bandwidth), else by the weight stream
    if gate_flop / gate_bytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        roofline = {"kernel": "twell_pack (gate GEMM + TwELL epilogue)", "bound": "mfma",
                    "achieved": gate_tflops, "peak": peak, "unit": "TFLOP/s",
                    "frac": gate_tflops / peak}
    else:
        gbs = gate_bytes / (t_gate * 1e-3) / 1e9
        roofline = {"kernel": "twell_pack (gate weight stream + TwELL epilogue)", "bound": "hbm",
                    "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": gbs / PEAK_HBM_GBS}
    peaks = None if args.no_peaks else measured_peaks()
    if peaks is not None and w.dtype == "bf16":
        mp = peaks["mfma_bf16_tflop_s"] if roofline["bound"] == "mfma" else peaks["hbm_read_gb_s"]
        roofline["measured_peak"] = mp
        roofline["frac_of_measured"] = roofline["achieved"] / mp
    roofline["traffic"] = measured_traffic(w.name)
    roofline["traffic_unit"] = "bytes per launch (HBM, counter-derived)"
    roof_gate = roofline
    # fused kernel: algorithmic bytes = x + y + live TwELL + distinct gathered rows
    routed_mask = torch.zeros(T, dtype=torch.bool, device="cuda")
    routed_mask[ffn.routed[:n_routed].long()] = True
    live = (torch.arange(max(w.cap, 1), device="cuda")[None, None, :]
            < torch.clamp(count, max=w.cap)[:, :, None]) & ~routed_mask[:, None, None]
    uniq = int(torch.unique(ffn.idx.to(torch.int64)[live]).numel()) if w.cap > 0 else 0
    sparse_bytes = 2.0 * T * d * eb + nnz_live * (2 + eb) + T * (n // 128) * 2 + uniq * 2.0 * d * eb
    sparse_flop = 4.0 * d * int(live.sum().item())
    # the fused kernel's own roofline: the larger of its vector-ALU time (packed
    # bf16 dot2 and float32 FMA at the 157.3 TFLOP/s vector peak) and its HBM
    # time on the algorithmic bytes
    t_s = t_sparse * 1e-3
    if sparse_flop / (PEAK_F32_TFLOPS * 1e12) >= sparse_bytes / (PEAK_HBM_GBS * 1e9):
        roof_sparse = {"kernel": "sparse_ffn_fwd (fused up*gate -> down over TwELL)", "bound": "alu",
                       "achieved": sparse_flop / t_s / 1e12, "peak": PEAK_F32_TFLOPS,
                       "unit": "TFLOP/s"}
    else:
        roof_sparse = {"kernel": "sparse_ffn_fwd (fused up*gate -> down over TwELL)", "bound": "hbm",
                       "achieved": sparse_bytes / t_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        if peaks is not None:
            roof_sparse["measured_peak"] = peaks["hbm_read_gb_s"]
            roof_sparse["frac_of_measured"] = roof_sparse["achieved"] / peaks["hbm_read_gb_s"]
    roof_sparse["frac"] = roof_sparse["achieved"] / roof_sparse["peak"]
    roof_sparse["traffic"] = measured_traffic(w.name, SPARSE_TRAFFIC_FILE, sparse_source_digest)
    roof_sparse["traffic_unit"] = "bytes per launch (HBM, counter-derived)"
    # the kernel's own bound: every live entry brings its wu_t and wd rows into
    # the CU; against the measured rate of cached loads (sffn_probe_cached) and
    # the bare gather of the distinct rows (sffn_probe_gather)
    n_live = int(live.sum().item())
    row_bytes_per_call = n_live * 2.0 * d * eb
    roof_sparse["entry_row_bytes"] = row_bytes_per_call
    roof_sparse["entry_row_gb_s"] = row_bytes_per_call / t_s / 1e9
    if peaks is not None:
        roof_sparse["cached_load_ceiling_gb_s"] = peaks["cached_load_gb_s"]
        roof_sparse["frac_of_cached_load_ceiling"] = (row_bytes_per_call / t_s / 1e9
                                                      / peaks["cached_load_gb_s"])
        if w.dtype == "bf16" and w.cap > 0:
            flush = torch.empty(128 << 20, dtype=torch.int32, device="cuda")
            roof_sparse["bare_gather"] = gather_probe(wu, wd, ffn.idx.to(torch.int32)[live], flush)
            del flush
    # the line's roofline is the dominant (longer) kernel's; both are kept
    roofline = roof_sparse if t_sparse > t_gate else roof_gate

    out = {
        # the headline metric as stated for this benchmark; `value` is its
        # tokens/s part, the HBM GB/s and the speed-up are in sparse_ffn_fwd,
        # roofline and speedup_vs_dense of the same line
        "metric": "sparse gated-FFN tokens/s, HBM GB/s and speedup vs dense FFN @1% act density",
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normals, gate bias -beta)",
        "config": {"workload": w.name, "tokens": T, "d_model": d, "d_ff": n, "beta": beta,
                   "tile": w.tile, "cap": w.cap, "rows": w.rows},
        "roofline": roofline,
        "roofline_twell_pack": roof_gate,
        "roofline_sparse_ffn_fwd": roof_sparse,
        "kernels_ms": {"twell_pack": t_gate, "sparse_ffn_fwd": t_sparse,
                       "hybrid_route": t_hybrid, "events_step": t_events,
                       "dense_ffn_ref": t_dense},
        "sparse_ffn_fwd": {"algorithmic_bytes": sparse_bytes, "gb_per_s": sparse_bytes / (t_sparse * 1e-3) / 1e9,
                           "hbm_frac": sparse_bytes / (t_sparse * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           "hbm_frac_of_measured": (sparse_bytes / (t_sparse * 1e-3) / 1e9
                                                    / peaks["hbm_read_gb_s"]) if peaks else None,
                           "flop": sparse_flop, "tflop_per_s": sparse_flop / (t_sparse * 1e-3) / 1e12,
                           "distinct_columns": uniq},
        "step_ms_percentiles": {"p10": float(np.percentile(step_ev, 10)),
                                "p50": float(np.median(step_ev)),
                                "p90": float(np.percentile(step_ev, 90))},
        "cold": cold,
        "torch_dense_ms": t_torch,
        "separate_conversion": conversion,
        "union_variant": union,
        "l1_regulariser": l1,
        "backward": backward,
        "dense_tokens_per_s": (T / (t_dense * 1e-3)) if t_dense else None,
        "speedup_vs_dense": (t_dense / ms_step) if t_dense else None,
        # against torch's dense FFN (hipBLASLt GEMMs) too, and against the
        # faster of the two same-GPU dense FFNs
        "speedup_vs_torch_dense": (t_torch / ms_step) if t_torch else None,
        "speedup_vs_best_dense": (min(t for t in (t_dense, t_torch) if t) / ms_step)
        if (t_dense or t_torch) else None,
        "dense_tflops": (3 * gate_flop / (t_dense * 1e-3) / 1e12) if t_dense else None,
        "measured_peaks": peaks,
        "activity": {"nnz_per_row": nnz_total / T, "density": nnz_total / (T * n),
                     "routed_rows": n_routed},
        "device": torch.cuda.get_device_name(0),
        "clocks": gpu_clocks(),
        "host": platform.node(),
    }
    if not args.no_cpu_baseline:
        rows = args.cpu_rows if args.cpu_rows is not None else min(T, 4096)
        out["cpu_baseline"] = cpu_baseline(inp, rows)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
