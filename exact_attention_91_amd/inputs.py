"""Seeded synthetic inputs for the attention forward (no attention arithmetic here).

Both the GPU path's tests/benchmark and the CPU oracle take their inputs from
this module, so the two sides see bit-identical values.

Recipe: numpy PCG64 seeded with SeedSequence(seed); spawn(3) children draw q, k,
v with standard_normal in float64, shaped and drawn in memory order: q is
[B, T, H, D], k and v are [B, T, H_kv, D]. q and k are multiplied by `qk_sigma`
(4 for the multi-query workload, which pushes scores to large magnitude). The
draws are rounded to float32 (round to nearest even) and, for bf16 or f16, on to
bfloat16 or IEEE half (round to nearest even, by torch on the CPU). The float64 arrays handed
to the oracle are the exact values of those rounded device tensors.

Workloads (shapes from the yelogs.com Flash Attention2-in-Triton article,
"基準測試設置" sweep and "多查詢注意力（MQA）" variant, and the GPT-2 124M
attention layer of "Flash Attention Memory Optimization Explained"):
  single_head_fp32  B=1  H=1  T=256  D=64  fp32, non-causal and causal
  batched_d{16,32,64,128}  B=64 H=1 T=1024 bf16 causal
  gpt2              B=16 H=12 T=1024 D=64  bf16 causal, scale 1/8
  long              B=8  H=1  T=8192 D=128 bf16 causal (oracle checks sampled rows)
  mqa               B=8  H=12 H_kv=1 T=4096 D=64 bf16 causal, q,k ~ N(0, 4^2)
  gpt2_f16          the gpt2 workload in IEEE half (seed 1006)
  gpt2_b2, long_b1  gpt2 at B=2 and long at B=1 (one GPU's share of a batch
                    split over 8 GPUs), seeds 1007 and 1008
  window            B=2 H=12 T=8192 D=64 bf16 causal, window 256 and global
                    tokens 0..15 (seed 1009); window_dense: the same without
                    the mask
Seeds: 1001, 1020+D, 1003, 1004, 1005 respectively. The backward pass takes an
upstream gradient dO drawn the same way from the fourth child of the same seed.
"""
from dataclasses import dataclass
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    H_kv: int
    T: int
    D: int
    dtype: str          # "bf16", "f16" or "f32"
    causal: tuple       # mask settings this workload is run with
    seed: int
    qk_sigma: float = 1.0
    window: int = -1            # >= 0: sliding-window / local-global mask
    global_tokens: tuple = ()   # global key positions of that mask

    @property
    def scale(self) -> float:
        return default_scale(self.D)

    def flops(self, causal: bool) -> float:
        """Counted FLOP: 4*B*H*T^2*D, halved when causal; under a window mask,
        4*D per visible (query, key) pair."""
        if self.window >= 0:
            return 4.0 * self.B * self.H * self.D * visible_pairs(
                self.T, self.window, self.global_tokens, causal)
        f = 4.0 * self.B * self.H * self.T * self.T * self.D
        return f / 2.0 if causal else f


def visible_pairs(T: int, window: int, global_tokens, causal: bool) -> int:
    """Number of (i, j) with |i - j| <= window or j global, and j <= i if causal."""
    i = np.arange(T, dtype=np.int64)
    lo = np.maximum(0, i - window)
    hi = i if causal else np.minimum(T - 1, i + window)
    hi = np.minimum(hi, i + window)
    n = int(np.sum(hi - lo + 1))
    for g in sorted(set(int(x) for x in global_tokens if 0 <= int(x) < T)):
        rows = i[(np.abs(i - g) > window) & ((g <= i) if causal else True)]
        n += len(rows)
    return n


def default_scale(D: int) -> float:
    """1/sqrt(D) as the float32 value the kernel receives."""
    return float(np.float32(1.0 / math.sqrt(D)))


WORKLOADS = {
    "single_head_fp32": Workload("single_head_fp32", 1, 1, 1, 256, 64, "f32", (False, True), 1001),
    **{f"batched_d{D}": Workload(f"batched_d{D}", 64, 1, 1, 1024, D, "bf16", (True,), 1020 + D)
       for D in (16, 32, 64, 128)},
    "gpt2": Workload("gpt2", 16, 12, 12, 1024, 64, "bf16", (True,), 1003),
    "long": Workload("long", 8, 1, 1, 8192, 128, "bf16", (True,), 1004),
    "mqa": Workload("mqa", 8, 12, 1, 4096, 64, "bf16", (True,), 1005, qk_sigma=4.0),
    "gpt2_f16": Workload("gpt2_f16", 16, 12, 12, 1024, 64, "f16", (True,), 1006),
    # One GPU's share when the gpt2 and long workloads are split by batch over
    # 8 GPUs: fewer work-groups than compute units (the key-split regime).
    "gpt2_b2": Workload("gpt2_b2", 2, 12, 12, 1024, 64, "bf16", (True,), 1007),
    "long_b1": Workload("long_b1", 1, 1, 1, 8192, 128, "bf16", (True,), 1008),
    # Sliding window of 256 plus the first 16 tokens global, over an 8192-token
    # sequence (the local-global pattern of the sparse-attention variants).
    "window": Workload("window", 2, 12, 12, 8192, 64, "bf16", (True,), 1009, window=256,
                       global_tokens=tuple(range(16))),
    # the window workload's shape without the mask (plain causal attention)
    "window_dense": Workload("window_dense", 2, 12, 12, 8192, 64, "bf16", (True,), 1009),
}


@dataclass
class Inputs:
    q64: np.ndarray     # float64 exact values, [B, T, H, D]
    k64: np.ndarray     # [B, T, H_kv, D]
    v64: np.ndarray
    q: torch.Tensor     # CPU tensors in the device dtype
    k: torch.Tensor
    v: torch.Tensor


def torch_dtype(dtype: str):
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f16":
        return torch.float16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def _round(a64: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32))
    t = t.to(torch_dtype(dtype))
    exact = t.to(torch.float64).numpy()
    return t, exact


def generate(B, H, H_kv, T, D, dtype="bf16", seed=0, qk_sigma=1.0) -> Inputs:
    ss = np.random.SeedSequence(seed)
    gq, gk, gv = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3))
    q = gq.standard_normal((B, T, H, D))
    k = gk.standard_normal((B, T, H_kv, D))
    v = gv.standard_normal((B, T, H_kv, D))
    if qk_sigma != 1.0:
        q *= qk_sigma
        k *= qk_sigma
    qt, q64 = _round(q, dtype)
    kt, k64 = _round(k, dtype)
    vt, v64 = _round(v, dtype)
    return Inputs(q64, k64, v64, qt, kt, vt)


def generate_dout(B, H, T, D, dtype="bf16", seed=0):
    """Upstream gradient dO [B, T, H, D] for the backward pass: standard
    normals from the fourth child of SeedSequence(seed) (q, k, v use the
    first three), rounded like the inputs. Returns (CPU tensor, float64)."""
    gd = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(4)[3]))
    return _round(gd.standard_normal((B, T, H, D)), dtype)


def generate_workload(w: Workload) -> Inputs:
    return generate(w.B, w.H, w.H_kv, w.T, w.D, w.dtype, w.seed, w.qk_sigma)


def sample_rows(B, H, T, per_batch, seed, fixed=(0, 1, 63, 64, 127, 128)):
    """Flat row ids (b*H + h)*T + i: for each batch, `per_batch` distinct
    (h, i) pairs -- the fixed query positions (plus the last two rows) at
    head 0, then seeded uniform draws without replacement."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    out = []
    for b in range(B):
        fixed_i = sorted({i for i in list(fixed) + [T // 2 - 1, T // 2, T - 2, T - 1]
                          if 0 <= i < T})
        chosen = {(0, i) for i in fixed_i}
        pool = H * T
        need = min(per_batch, pool) - len(chosen)
        while need > 0:
            draw = rng.choice(pool, size=need, replace=False)
            for x in draw:
                hi = (int(x) // T, int(x) % T)
                if hi not in chosen and len(chosen) < min(per_batch, pool):
                    chosen.add(hi)
            need = min(per_batch, pool) - len(chosen)
        out.extend((b * H + h) * T + i for h, i in sorted(chosen))
    return np.asarray(out, dtype=np.int64)
