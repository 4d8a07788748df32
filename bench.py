"""Benchmark: attention forward TFLOP/s on one MI355X, through the C ABI.

One step = one fa_fwd call (or, with --nsplit > 1, one fa_fwd_splitk call)
over the whole workload (default: the GPT-2 124M
attention layer, B=16 H=12 T=1024 D=64, BNHD, bf16, causal), inputs resident
in HBM. W untimed warm-up steps (default 2000, so the GPU clock has settled),
then K steps timed with HIP events on the stream the kernel is launched on,
bracketed by device synchronisation.

Counted FLOP per step: 4*B*H*T^2*D, halved when causal (the dense-contraction
count; the masked upper triangle is not counted).

Prints ONE JSON line. Extra keys: `roofline` (achieved vs MI355X dense bf16
MFMA peak), `cpu_baseline` (the float64 oracle timed on this host, with the
GPU output compared against it as a by-product), `cold` (per-call times with
the L2s and the 256 MB last-level cache emptied of the step's data before each
call, by reading a 512 MiB buffer; `after_fill` the same after writing it).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MFMA peak (GPT-2 causal bf16 shape)"
PEAK = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X published dense MFMA, TFLOP/s
HBM_PEAK_GBS = 8000.0                                     # MI355X published HBM3E bandwidth
# the forward kernel's sources (its traffic figures are tied to their hash)
KERNEL_SRCS = [os.path.join(ROOT, "exact_attention_91_amd", "csrc", n)
               for n in ("fa_fwd.hip", "fa_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_bf16_gpt2_traffic.json")
_ELEM = {"bf16": "__bf16", "f16": "_Float16"}   # element type of the 16-bit kernel


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # The GPU's clock takes several hundred back-to-back launches (tens of ms)
    # to settle; shorter warm-ups time the ramp, not the kernel.
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="gpt2")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd", "decode"), default="fwd",
                    help="bwd: time fa_bwd (gradients for a seeded dO, from the "
                         "forward's o and lse computed once before timing); decode: time "
                         "fa_fwd_decode on --decode-shape (the workload is not used)")
    ap.add_argument("--decode-shape", default="16,32,8,1,8192,128",
                    help="B,H,H_kv,T_q,T_k,D of the decode step (default: a 32-head "
                         "layer with 8 kv heads, one new token, an 8192-token cache)")
    ap.add_argument("--head-split", type=int, default=0,
                    help="bwd: query-head parts of the dK/dV kernel (0: library choice)")
    ap.add_argument("--nsplit", type=int, default=1,
                    help="> 1: time fa_fwd_splitk (key split into this many parts "
                         "plus the logsumexp combine) instead of fa_fwd")
    ap.add_argument("--no-global-split", action="store_true",
                    help="window backward: workspace without room for the global keys' "
                         "partial sums (each global key tile walks every query tile itself)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle until this much wall time has passed")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before timing, run one device copy of this many MiB "
                         "(a known-size kernel for HBM counter calibration)")
    return ap.parse_args()


def source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def one_thread_rate(orc, x, w, causal, seconds):
    """The oracle on one host thread over evenly spaced query rows of the
    workload (counted FLOP 4*D per visible key of each row), for about
    `seconds`; the thread count is restored afterwards."""
    import numpy as np
    n_all = w.B * w.H * w.T
    keep = orc.num_threads()
    orc.set_num_threads(1)
    try:
        n = 64
        while True:
            rows = np.linspace(0, n_all - 1, n).astype(np.int64)
            t0 = time.perf_counter()
            orc.attention_rows(x.q64, x.k64, x.v64, causal, w.scale, rows)
            el = time.perf_counter() - t0
            if el >= seconds or n >= n_all:
                break
            n = min(n_all, n * max(2, int(seconds / max(el, 1e-3))))
        keys = (rows % w.T + 1) if causal else np.full(rows.shape, w.T)
        flop = float(4 * w.D * np.sum(keys))
    finally:
        orc.set_num_threads(keep)
    return {"value": flop / el / 1e12, "unit": "TFLOP/s", "cores": 1,
            "sample": f"{len(rows)} evenly spaced query rows of {n_all}, {el:.2f} s"}


def traffic_for(workload_name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_hash() or t.get("workload") != workload_name:
        return None
    return t.get("bytes_per_launch")


def bench_decode(a):
    """One decode step per call: fa_fwd_decode (split kernel + combine) on
    seeded bf16 inputs, library split choice. The kernel is bound by reading
    the key/value cache once, so the roofline is HBM: compulsory bytes (q, k,
    v, o once, lse fp32) over the time per step."""
    import numpy as np
    import torch
    from exact_attention_91_amd import fa
    B, H, H_kv, Tq, Tk, D = (int(x) for x in a.decode_shape.split(","))
    torch.cuda.set_device(0)
    rng = np.random.default_rng(2024)
    mk = lambda *sh: torch.from_numpy(rng.standard_normal(sh).astype(np.float32)).to(
        torch.bfloat16).cuda()
    q, k, v = mk(B, Tq, H, D), mk(B, Tk, H_kv, D), mk(B, Tk, H_kv, D)
    nsplit = fa.decode_splits(B, H_kv, H, Tq, Tk)
    nbytes = fa.decode_workspace_bytes(B, H, Tq, D, nsplit)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device="cuda")
    lib = fa._lib()
    stream = torch.cuda.current_stream()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H_kv,
            Tq, Tk, D, 1, D ** -0.5, fa.FA_DTYPE_BF16, nsplit, ws.data_ptr(), nbytes,
            stream.cuda_stream)

    def step():
        rc = lib.fa_fwd_decode(*args)
        if rc:
            raise RuntimeError(fa.status_str(rc))
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    comp = 2 * (B * Tq * H * D * 2) + 2 * (B * Tk * H_kv * D * 2) + 4 * B * H * Tq
    gbs = comp / (ms * 1e-3) / 1e9
    vis = sum(min(Tk, Tk - Tq + i + 1) for i in range(Tq))
    flops = 4.0 * B * H * D * vis
    out = {"metric": f"attention decode GB/s and % of HBM peak (B={B} H={H} H_kv={H_kv} "
                     f"T_q={Tq} T_k={Tk} D={D})",
           "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"decode: B={B} H={H} H_kv={H_kv} T_q={Tq} T_k={Tk} D={D} "
                                  f"bf16 causal, nsplit={nsplit}",
                      "pass": "decode", "nsplit": nsplit, "parallelism": "single GPU"},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                        "kernel": "fa_fwd_half_kernel<__bf16, ..., DECODE> + "
                                  "fa_lse_combine_kernel (rate over the step)"},
           "tflops": flops / (ms * 1e-3) / 1e12, "algorithmic_bytes": comp,
           "cpu_baseline": None, "device": torch.cuda.get_device_name(0)}
    print(json.dumps(out), flush=True)


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention forward is sharded "
              "by batch/head with no exchange, and multi-GPU runs are not part of "
              "this build. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if a.which == "decode":
        return bench_decode(a)

    import numpy as np
    import torch

    from exact_attention_91_amd import fa
    from exact_attention_91_amd.inputs import WORKLOADS, generate_workload, torch_dtype

    w = WORKLOADS[a.workload]
    causal = True if True in w.causal else False
    torch.cuda.set_device(0)
    x = generate_workload(w)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda")
    lib = fa._lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    dcode = fa._dtype_code(q)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            w.B, w.H, w.H_kv, w.T, w.D, int(causal), w.scale, dcode, sp)

    if a.which == "bwd":
        from exact_attention_91_amd.inputs import generate_dout
        if a.nsplit > 1:
            raise SystemExit("--nsplit applies to the forward only")
        bits = None
        if w.window >= 0:
            # o and lse from the window forward; the token bitmap is built once
            bits = (fa.window_bitmap(w.global_tokens, w.T, q.device) if w.global_tokens
                    else None)
            rc = lib.fa_fwd_window(*(args[:-1] + (w.window, None if bits is None
                                                  else bits.data_ptr(), sp)))
        else:
            rc = lib.fa_fwd(*args)
        if rc:
            raise RuntimeError(fa.status_str(rc))
        do = generate_dout(w.B, w.H, w.T, w.D, w.dtype, w.seed)[0].cuda()
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nbytes = fa.bwd_workspace_bytes(w.B, w.H, w.H_kv, w.T, w.D, a.head_split)
        if w.window >= 0 and w.global_tokens and not a.no_global_split:
            # room for the global keys' partial sums: their far queries are split
            nbytes = fa.bwd_window_workspace_bytes(w.B, w.H, w.H_kv, w.T, w.D, w.window,
                                                   len(set(w.global_tokens)), a.head_split)
        ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
        bargs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                 do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.H, w.H_kv,
                 w.T, w.D, int(causal), w.scale, dcode)
        tail = (a.head_split, ws.data_ptr(), nbytes, sp)
        if w.window >= 0:
            wargs = bargs + (w.window, None if bits is None else bits.data_ptr()) + tail

            def step():
                rc = lib.fa_bwd_window(*wargs)
                if rc:
                    raise RuntimeError(fa.status_str(rc))
        else:
            bargs = bargs + tail

            def step():
                rc = lib.fa_bwd(*bargs)
                if rc:
                    raise RuntimeError(fa.status_str(rc))
    elif w.window >= 0:
        if a.nsplit > 1:
            raise SystemExit("--nsplit does not apply to window workloads")
        # the bitmap of the global tokens is built once (it serves every call
        # with the same tokens), like the inputs, outside the timed region
        bits = (fa.window_bitmap(w.global_tokens, w.T, q.device) if w.global_tokens else None)
        wargs = args[:-1] + (w.window, None if bits is None else bits.data_ptr(), sp)

        def step():
            rc = lib.fa_fwd_window(*wargs)
            if rc:
                raise RuntimeError(fa.status_str(rc))
    elif a.nsplit > 1:
        nbytes = fa.splitk_workspace_bytes(w.B, w.H, w.T, w.D, a.nsplit)
        ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
        sargs = args[:-1] + (a.nsplit, ws.data_ptr(), nbytes, sp)

        def step():
            rc = lib.fa_fwd_splitk(*sargs)
            if rc:
                raise RuntimeError(fa.status_str(rc))
    else:
        def step():
            rc = lib.fa_fwd(*args)
            if rc:
                raise RuntimeError(fa.status_str(rc))

    if a.calib_copy_mib:
        n = a.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    # backward: five contractions (S, dP, dV, dK, dQ) against the forward's two
    flops = w.flops(causal) * (2.5 if a.which == "bwd" else 1.0)
    tflops = flops / (ms * 1e-3) / 1e12

    cold = None
    if not a.no_cold:
        # Caches emptied of the step's data before each of 20 calls by touching
        # a 512 MiB buffer (twice the 256 MB MALL, far above the L2s):
        #   "cold": the buffer is read (summed), which leaves clean lines only;
        #   "after_fill": the buffer is written (filled), which leaves 256 MB of
        #   dirty lines whose write-back to HBM competes with the step.
        flush = torch.ones(512 << 18, dtype=torch.int32, device="cuda")
        sink = torch.zeros((), dtype=torch.int64, device="cuda")

        def timed_after(evict):
            times = []
            for _ in range(20):
                evict()
                c0 = torch.cuda.Event(enable_timing=True)
                c1 = torch.cuda.Event(enable_timing=True)
                c0.record(stream)
                step()
                c1.record(stream)
                torch.cuda.synchronize()
                times.append(c0.elapsed_time(c1))
            return times

        times = timed_after(lambda: sink.add_(flush.sum()))
        ftimes = timed_after(lambda: flush.fill_(1))
        del flush
        cms = float(np.median(times))
        fms = float(np.median(ftimes))
        cold = {"ms_median": cms, "tflops": flops / (cms * 1e-3) / 1e12,
                "ms_p10": float(np.percentile(times, 10)),
                "ms_p90": float(np.percentile(times, 90)),
                "after_fill": {"ms_median": fms, "tflops": flops / (fms * 1e-3) / 1e12}}

    peak = PEAK[w.dtype]
    groups = fa.key_groups(w.B, w.H, w.T, w.D, torch_dtype(w.dtype))
    # head pairs: an even number of query heads per kv head with one key group
    pairs = groups == 1 and (w.H // w.H_kv) % 2 == 0
    # Compulsory bytes: q, k, v, o once each in the element type, L in fp32.
    esz = {"f32": 4, "bf16": 2, "f16": 2}[w.dtype]
    nbytes = esz * w.B * w.T * w.D * (2 * w.H + 2 * w.H_kv) + 4 * w.B * w.H * w.T
    # The binding roof of the plain forward: the larger of the MFMA time
    # (counted FLOP at the published dense peak) and the HBM time (compulsory
    # bytes at 8 TB/s). The GPT-2 layer's intensity, 254 FLOP/B, lies below the
    # ridge (2.5 PFLOP/s / 8 TB/s = 312), so there the binding roof is HBM.
    hbm_bound = (a.which == "fwd" and w.window < 0 and a.nsplit == 1 and
                 nbytes / HBM_PEAK_GBS / 1e9 > flops / (peak * 1e12))
    if hbm_bound:
        achieved = nbytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                "frac": tflops / peak}
    roof.update({"traffic": traffic_for(w.name),
                 "mfma_tflops": tflops, "mfma_frac": tflops / peak,
                 "kernel": (f"fa_fwd_half_kernel<{_ELEM[w.dtype]}, {w.D}, {str(causal).lower()}, "
                            f"{str(a.nsplit > 1).lower()}, false, "
                            f"{str(a.nsplit == 1 and groups == 2).lower()}, "
                            f"{str(a.nsplit == 1 and pairs).lower()}, false>"
                            if w.dtype in _ELEM else
                            f"fa_fwd_f32_kernel<{w.D}, {str(causal).lower()}>")})
    if w.window >= 0 and a.which == "fwd":
        roof["kernel"] = (f"fa_fwd_half_kernel<{_ELEM[w.dtype]}, {w.D}, {str(causal).lower()}, "
                          f"false, true, false, false, false> (window)")
        roof["traffic"] = None
    if a.which == "bwd":
        roof["kernel"] = (f"fa_bwd_dq_kernel + fa_bwd_dkdv_kernel<{_ELEM[w.dtype]}, {w.D}, "
                          f"{str(causal).lower()}> (+ fa_bwd_reduce_kernel with a head split; "
                          f"rate over the step)")
        roof["traffic"] = None
    if a.nsplit > 1:
        # one step = the split kernel plus the combine kernel; the rate is over both
        roof["kernel"] += f" + fa_lse_combine_kernel<{_ELEM[w.dtype]}, {w.D}>"
        roof["traffic"] = None

    cpu = None
    if not a.no_cpu_baseline and a.which == "bwd":
        from oracle import oracle as orc
        torch.cuda.synchronize()
        got = [t.to(torch.float64).cpu().numpy() for t in (dq, dk, dv)]
        do64 = generate_dout(w.B, w.H, w.T, w.D, w.dtype, w.seed)[1]
        reps, t0 = 0, time.perf_counter()
        while True:
            if w.window >= 0:
                ref = orc.attention_bwd_masked(x.q64, x.k64, x.v64, do64, causal, w.scale,
                                               w.window, w.global_tokens)
            else:
                ref = orc.attention_bwd(x.q64, x.k64, x.v64, do64, causal, w.scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= a.cpu_seconds:
                break
        sec = el / reps
        cpu = {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(),
               "kind": "oracle",
               "sample": f"the full {w.name} backward (all {w.B * w.H * w.T} query rows), "
                         f"{reps} repeat(s), {sec:.3f} s each",
               "gpu_vs_oracle_max_abs_err": {n: float(np.max(np.abs(g_ - r_)))
                                             for n, g_, r_ in zip(("dQ", "dK", "dV"), got, ref)}}
    elif not a.no_cpu_baseline:
        from oracle import oracle as orc
        torch.cuda.synchronize()
        o_gpu = o.to(torch.float64).cpu().numpy()
        l_gpu = lse.to(torch.float64).cpu().numpy()
        reps, t0 = 0, time.perf_counter()
        while True:
            if w.window >= 0:
                o_ref, l_ref = orc.attention_masked(x.q64, x.k64, x.v64, causal, w.scale,
                                                    w.window, w.global_tokens)
            else:
                o_ref, l_ref = orc.attention(x.q64, x.k64, x.v64, causal, w.scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= a.cpu_seconds:
                break
        sec = el / reps
        cpu = {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(),
               "kind": "oracle",
               "sample": f"the full {w.name} workload (all {w.B * w.H * w.T} query rows), "
                         f"{reps} repeat(s), {sec:.3f} s each",
               "gpu_vs_oracle_max_abs_err": {"O": float(np.max(np.abs(o_gpu - o_ref))),
                                             "L": float(np.max(np.abs(l_gpu - l_ref)))},
               "host_cpu": host_cpu_model()}
        if w.window < 0:
            cpu["one_thread"] = one_thread_rate(orc, x, w, causal, a.cpu_seconds / 4)

    if a.which == "fwd" and w.name == "gpt2" and a.nsplit == 1:
        metric = METRIC
    else:
        metric = (f"attention {a.which} TFLOP/s and % of MFMA peak ({w.name} workload"
                  f"{f', nsplit={a.nsplit}' if a.nsplit > 1 else ''})")
    roofs = None
    if a.which == "fwd" and w.window < 0 and a.nsplit == 1:
        # Times the step could not beat on each unit, against the published
        # peaks (dense MFMA, 8 TB/s HBM over the compulsory bytes) and against
        # the rates the microbenchmarks of include/fa_roofs.h measured on this
        # GPU model (profiles/roofs_mi355x.json): sustained bf16 MFMA, a
        # device-memory copy, and v_exp_f32 with one exponential per visible
        # score.
        from exact_attention_91_amd import roofs as roofs_mod
        meas = roofs_mod.load() or {}
        exps = w.B * w.H * (w.T * (w.T + 1) / 2 if causal else w.T * w.T)
        t = {"mfma_us": flops / (peak * 1e12) * 1e6, "hbm_us": nbytes / (HBM_PEAK_GBS * 1e9) * 1e6}
        if meas.get("exp_per_s"):
            t["exp_us"] = exps / meas["exp_per_s"] * 1e6
        roofs = dict(t, largest=max(t, key=t.get)[:-3], measured_us=ms * 1e3,
                     algorithmic_bytes=nbytes, exps=exps)
        if w.dtype in ("bf16", "f16") and meas.get("mfma_bf16_tflops"):
            roofs["measured_mfma_tflops"] = meas["mfma_bf16_tflops"]
            roofs["frac_of_measured_mfma"] = tflops / meas["mfma_bf16_tflops"]
        if meas.get("copy_gbps"):
            roofs["measured_copy_gbps"] = meas["copy_gbps"]
            roofs["frac_of_measured_copy"] = nbytes / (ms * 1e-3) / 1e9 / meas["copy_gbps"]
        if meas:
            roofs["measured_roofs_file"] = os.path.relpath(roofs_mod.ROOFS_FILE, ROOT)
    out = {
        "metric": metric, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}{' backward' if a.which == 'bwd' else ''}: B={w.B} "
                               f"H={w.H} H_kv={w.H_kv} T={w.T} D={w.D} BNHD {w.dtype} "
                               f"causal={causal}",
                   "B": w.B, "H": w.H, "H_kv": w.H_kv, "T": w.T, "D": w.D,
                   "causal": causal, "layout": "BNHD", "parallelism": "single GPU",
                   "nsplit": a.nsplit, "pass": a.which,
                   **({"window": w.window, "global_tokens": len(w.global_tokens)}
                      if w.window >= 0 else {})},
        "flop_per_step": flops,
        "roofline": roof,
        "roofs": roofs,
        "cpu_baseline": cpu,
        "cold": cold,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
