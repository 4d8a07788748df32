"""Measured roofs of this GPU (the microbenchmarks of include/fa_roofs.h).

Runs each microbenchmark of libfa.so on torch's current stream, times it with
events on that stream, and reports rates: dense bf16 MFMA FLOP/s, v_exp_f32
and fp32 FMA instructions per second, MFMA/VALU overlap on one SIMD, and
device-memory copy and read bandwidth. `python -m exact_attention_91_amd.roofs --write`
stores the result as JSON under profiles/, which bench.py reads to state the
attention kernels' speed against measured as well as published peaks.
"""
import argparse
import ctypes
import datetime
import json
import os
import statistics
import sys

import torch

from exact_attention_91_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROOFS_FILE = os.path.join(ROOT, "profiles", "roofs_mi355x.json")
FA_ROOF_FMA, FA_ROOF_EXP = 0, 1
_VP, _I, _LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
MFMA_FLOP = 2 * 32 * 32 * 16     # one v_mfma_f32_32x32x16_bf16
NUM_CU = 256


def _lib():
    lib = fa._lib()
    if not getattr(lib, "_roofs_typed", False):
        lib.fa_roof_mfma.argtypes = [_I, _I, _VP, _VP]
        lib.fa_roof_valu.argtypes = [_I, _I, _I, _VP, _VP]
        lib.fa_roof_overlap.argtypes = [_I, _I, _I, _I, _I, _VP, _VP]
        lib.fa_roof_copy.argtypes = [_VP, _VP, _LL, _VP]
        lib.fa_roof_read.argtypes = [_VP, _LL, _VP, _VP]
        for f in (lib.fa_roof_mfma, lib.fa_roof_valu, lib.fa_roof_overlap, lib.fa_roof_copy,
                  lib.fa_roof_read):
            f.restype = _I
        lib._roofs_typed = True
    return lib


def _time(launch, reps=10, warm=3):
    """Median milliseconds of `launch()` over `reps` timed calls."""
    st = torch.cuda.current_stream()
    for _ in range(warm):
        launch()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        launch()
        e1.record(st)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return statistics.median(ts)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} failed with status {rc}")


def measure(copy_mib: int = 1024):
    lib = _lib()
    sp = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(NUM_CU * 16, dtype=torch.float32, device="cuda")
    out = {}

    # MFMA: 2 waves per SIMD (grid of 2 four-wave blocks per CU), 4 chains each
    grid, n = 2 * NUM_CU, 20000
    ms = _time(lambda: _check(lib.fa_roof_mfma(grid, n, sink.data_ptr(), sp), "fa_roof_mfma"))
    out["mfma_bf16_tflops"] = grid * 4 * n * 4 * MFMA_FLOP / (ms * 1e-3) / 1e12
    out["mfma_bf16_ms"] = ms

    # VALU: 4 waves per SIMD, 16 independent chains each
    grid, n = 4 * NUM_CU, 4000
    for name, op in (("exp", FA_ROOF_EXP), ("fma", FA_ROOF_FMA)):
        ms = _time(lambda: _check(lib.fa_roof_valu(grid, n, op, sink.data_ptr(), sp),
                                  "fa_roof_valu"))
        rate = grid * 4 * n * 16 / (ms * 1e-3)          # wave64 instructions per second
        out[f"{name}_wave_instr_per_s"] = rate
        out[f"{name}_per_s"] = rate * 64                 # lane operations per second
        out[f"{name}_ms"] = ms

    # Overlap: one 8-wave block per CU; waves 0-3 MFMA, waves 4-7 VALU, same SIMDs
    ov = {}
    for name, op, n_valu in (("fma", FA_ROOF_FMA, 12000), ("exp", FA_ROOF_EXP, 4500)):
        n_mfma = 6000
        t = {}
        for mask in (1, 2, 3):
            t[mask] = _time(lambda: _check(lib.fa_roof_overlap(NUM_CU, n_mfma, n_valu, op, mask,
                                                               sink.data_ptr(), sp),
                                           "fa_roof_overlap"))
        hidden = (t[1] + t[2] - t[3]) / min(t[1], t[2])
        ov[name] = {"mfma_alone_ms": t[1], "valu_alone_ms": t[2], "both_ms": t[3],
                    "mfma_per_wave": 4 * n_mfma, "valu_per_wave": 16 * n_valu,
                    "hidden_fraction_of_shorter": hidden}
    out["overlap"] = ov

    # Device-memory copy
    nbytes = copy_mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = _time(lambda: _check(lib.fa_roof_copy(src.data_ptr(), dst.data_ptr(), nbytes, sp),
                              "fa_roof_copy"))
    if not torch.equal(src, dst):
        raise RuntimeError("fa_roof_copy: copy mismatch")
    out["copy_bytes"] = nbytes
    out["copy_gbps"] = 2 * nbytes / (ms * 1e-3) / 1e9   # read + write
    out["copy_ms"] = ms
    del dst
    big = torch.zeros(8192, dtype=torch.float32, device="cuda")   # one per work-group
    ms = _time(lambda: _check(lib.fa_roof_read(src.data_ptr(), nbytes, big.data_ptr(), sp),
                              "fa_roof_read"))
    out["read_gbps"] = nbytes / (ms * 1e-3) / 1e9
    out["read_ms"] = ms
    del src
    out["device"] = torch.cuda.get_device_name(0)
    return out


def load():
    """The committed measurement (dict), or None."""
    try:
        with open(ROOFS_FILE) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--write", action="store_true", help=f"store the result in {ROOFS_FILE}")
    ap.add_argument("--copy-mib", type=int, default=1024)
    a = ap.parse_args()
    if not torch.cuda.is_available():
        sys.exit("roofs: needs a GPU")
    torch.cuda.set_device(0)
    r = measure(a.copy_mib)
    r["command"] = "python -m exact_attention_91_amd.roofs --write"
    r["date"] = datetime.date.today().isoformat()
    print(json.dumps(r), flush=True)
    if a.write:
        with open(ROOFS_FILE, "w") as f:
            json.dump(r, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
