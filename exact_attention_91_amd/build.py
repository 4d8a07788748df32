"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", n) for n in ("fa_fwd.hip", "fa_bwd.hip", "fa_roofs.hip")]
LIB = os.path.join(HERE, "libfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are disabled for all device code. MFMA accumulators are
# kept in ordinary VGPRs (the softmax rescales them every tile; AGPR
# accumulators would need a copy to VGPRs and back each time).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         # NaN inputs are unsupported (documented in fa.h); without this every
         # fmaxf on an MFMA result gets an extra NaN-quieting copy.
         "-fno-honor-nans",
         # Keep the hand-interleaved MFMA/VALU phases in source order: do not
         # hoist instructions common to both arms of a branch above it.
         "-mllvm", "-simplifycfg-hoist-common=false"]


def build(verbose: bool = False, extra=(), out: str = None) -> str:
    """Compile each source to an object in parallel, then link the library
    (libfa.so, or `out`)."""
    out = out or LIB
    tag = os.path.splitext(os.path.basename(out))[0]
    objs = [os.path.join(HERE, "csrc", f"{os.path.basename(src)}.{tag}.o") for src in SRCS]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    procs = []
    for src, obj in zip(SRCS, objs):
        cmd = [HIPCC, *compile_flags, *extra, "-I", os.path.join(ROOT, "include"), "-c",
               "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
    failed = [p.args for p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    cmd = [HIPCC, *FLAGS, *extra, "-o", out + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    for obj in objs:
        os.remove(obj)
    os.replace(out + ".tmp", out)
    return out


POISON_LIB = os.path.join(HERE, "libfa_poison.so")


def build_poison(verbose: bool = False) -> str:
    """The debug build of the same library in which every staged LDS buffer
    reads as NaN between its last reader and its refill (FA_LDS_POISON): the
    GPU tests run a set of parity cases through it, so a read that races a
    refill shows up as NaN instead of stale data. Slower; not for use."""
    return build(verbose, extra=("-DFA_LDS_POISON",), out=POISON_LIB)


def build_host_sanitized(out_dir: str, verbose: bool = False) -> str:
    """The library with its host code (argument validation, dispatch, the C
    ABI) built with AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU
    sanitizer tests; device code is compiled as usual, without sanitizers (the
    -fsanitize flags apply to the host pass only). Load it with the clang ASan
    runtime preloaded (host_sanitizer_runtime())."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libfa_host_asan.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-g",
           "-fno-omit-frame-pointer", "-shared-libsan"]
    objs = [os.path.join(out_dir, os.path.basename(src) + ".o") for src in SRCS]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    procs = []
    for src, obj in zip(SRCS, objs):
        cmd = [HIPCC, *compile_flags, *san, "-I", os.path.join(ROOT, "include"), "-c", "-o", obj,
               src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
    failed = [p.args for p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    subprocess.run([HIPCC, *FLAGS, *san, "-o", out, *objs], check=True)
    return out


def host_sanitizer_runtime() -> str:
    """Path of the clang ASan runtime that build_host_sanitized() links against."""
    res = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "lib", "llvm", "bin", "clang"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.isabs(res) or not os.path.exists(res):
        import glob
        found = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not found:
            raise FileNotFoundError("clang ASan runtime not found")
        res = found[0]
    return res


if __name__ == "__main__":
    print(build(verbose=True))
