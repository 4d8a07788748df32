"""The measured-roof microbenchmarks of libfa.so (include/fa_roofs.h) on the
GPU: the copy is exact, the streaming read visits every vector, and the rates
that roofs.measure() reports are positive and below the chip's published
peaks (dense bf16 MFMA 2.5 PFLOP/s, HBM 8 TB/s)."""
import ctypes

import pytest
import torch

from exact_attention_91_amd import roofs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48])
def test_copy_is_exact(nbytes):
    lib = roofs._lib()
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    assert lib.fa_roof_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0        # nothing past the end


@pytest.mark.parametrize("n16", [1, 5000, 8192 * 256 * 8 + 17])
def test_read_folds_every_vector_of_its_thread(n16):
    """Work-group g of G = 8192 reads its own chunk [n16 g / G, n16 (g+1) / G)
    of 16-byte vectors; its thread 0 XORs the vectors lo, lo + 256, ... of the
    chunk, and the sink entry g is set iff that fold equals 0x9e3779b9. Put
    that word, split in two, in the first and the last vector thread 0 of the
    work-group owning vector 0 reads: only that entry is set, and only if the
    loop reached both."""
    lib = roofs._lib()
    G = 8192
    import numpy as np
    g = next(b for b in range(G) if n16 * (b + 1) // G > 0)   # owner of vector 0
    lo, hi = n16 * g // G, n16 * (g + 1) // G
    assert lo == 0
    last = lo + ((hi - 1 - lo) // 256) * 256
    words = np.zeros(n16 * 4, dtype=np.uint32)
    if last == lo:
        words[0] = 0x9E3779B9
    else:
        words[0] = 0x9E370000
        words[4 * last] = 0x000079B9
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(G, dtype=torch.float32, device="cuda")
    assert lib.fa_roof_read(src.data_ptr(), n16 * 16, sink.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert float(sink[g]) == 1.0
    assert int(sink.count_nonzero()) == 1


def test_measured_rates_are_plausible():
    r = roofs.measure(copy_mib=64)
    assert 500 < r["mfma_bf16_tflops"] < 2500
    assert 0 < r["exp_per_s"] < r["fma_per_s"]
    # a 64 MiB buffer may be served from the 256 MB last-level cache, above HBM's 8 TB/s
    assert 100 < r["copy_gbps"] < 30000
    assert 100 < r["read_gbps"] < 30000
    for k in ("fma", "exp"):
        assert -0.1 < r["overlap"][k]["hidden_fraction_of_shorter"] < 1.2
