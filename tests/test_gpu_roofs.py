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


@pytest.mark.parametrize("n16", [1, 5000, 2048 * 256 * 8 + 17])
def test_read_folds_every_vector_of_its_thread(n16):
    """Thread 0 of the grid XORs the vectors i = 0, N, 2N, ... (N threads);
    the sink is set iff the fold equals 0x9e3779b9. Put that word, split in
    two, in the first and the last vector thread 0 reads: the sink is set only
    if the loop reached both."""
    lib = roofs._lib()
    nthreads = 256 * 8 * 256
    import numpy as np
    words = np.zeros(n16 * 4, dtype=np.uint32)
    last = ((n16 - 1) // nthreads) * nthreads
    if last == 0:
        words[0] = 0x9E3779B9
    else:
        words[0] = 0x9E370000
        words[4 * last] = 0x000079B9
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(2048, dtype=torch.float32, device="cuda")
    assert lib.fa_roof_read(src.data_ptr(), n16 * 16, sink.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert float(sink[0]) == 1.0
    assert int(sink[1:].count_nonzero()) == 0


def test_measured_rates_are_plausible():
    r = roofs.measure(copy_mib=64)
    assert 500 < r["mfma_bf16_tflops"] < 2500
    assert 0 < r["exp_per_s"] < r["fma_per_s"]
    assert 100 < r["copy_gbps"] < 8000
    assert 100 < r["read_gbps"] < 8000
    for k in ("fma", "exp"):
        assert -0.1 < r["overlap"][k]["hidden_fraction_of_shorter"] < 1.2
