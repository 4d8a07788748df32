"""C-ABI checks that need no GPU: libfa.so loads, exports every function that
include/fa.h declares, and rejects every invalid argument before any HIP call
(validation is pure host code, so these calls never reach the device)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
HEADERS = sorted(os.path.join(ROOT, "include", n) for n in os.listdir(os.path.join(ROOT, "include"))
                 if n.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    from exact_attention_91_amd import fa
    if not os.path.exists(fa.lib_path()):
        from exact_attention_91_amd import build
        build.build()
    return fa._lib()


def _declared_functions(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?(?:\w+\s+)*\w+\s*\*?\s*(fa_\w+)\s*\(",
                                text, re.M))
    return sorted(names)


def _enum_values(name):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef enum \{([^}]*)\}\s*" + name, text).group(1)
    return dict((k, int(v)) for k, v in re.findall(r"(FA_\w+)\s*=\s*(\d+)", body))


ST = _enum_values("fa_status_t")
DT = _enum_values("fa_dtype_t")


def test_header_declares_the_entry_points():
    assert _declared_functions([os.path.join(ROOT, "include", "fa_roofs.h")]) == [
        "fa_roof_copy", "fa_roof_mfma", "fa_roof_overlap", "fa_roof_read", "fa_roof_valu"]
    assert _declared_functions([HEADER]) == ["fa_bwd", "fa_bwd_window", "fa_bwd_window_workspace_bytes",
                                     "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_decode", "fa_fwd_decode_workspace_bytes", "fa_fwd_key_groups",
                                     "fa_fwd_splitk", "fa_fwd_splitk_noalloc",
                                     "fa_fwd_splitk_scratch_bytes", "fa_fwd_splitk_workspace_bytes",
                                     "fa_fwd_strided", "fa_fwd_window", "fa_lse_combine",
                                     "fa_status_str", "fa_version", "fa_window_bitmap",
                                     "fa_window_bitmap_bytes"]


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # and nothing else with the fa_ prefix escapes the library
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "exact_attention_91_amd",
                          "libfa.so")], capture_output=True, text=True, check=True).stdout
    exported = sorted(set(re.findall(r"\bT (fa_\w+)", out)))
    assert exported == _declared_functions()


def test_version_and_status_strings(lib):
    assert lib.fa_version() == 100
    seen = set()
    for code in ST.values():
        s = lib.fa_status_str(code).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == len(ST)
    assert lib.fa_status_str(12345).decode() == "unknown status"
    assert lib.fa_status_str(-1).decode() == "unknown status"


# A fake, 16-byte aligned, never-dereferenced device address: every call below
# is meant to fail validation, which runs entirely on the host before any HIP
# call. Where a GPU is visible these calls are skipped, so that a case that
# wrongly passed validation could never launch a kernel on a fake address.
P = 4096


def _host_only():
    from tests.conftest import gpu_available
    if gpu_available():
        pytest.skip("fake-pointer validation tests run only where no GPU is visible")


def call(lib, **kw):
    _host_only()
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=4, H_kv=2, T=100, D=64, causal=1,
             scale=0.125, dtype=DT["FA_DTYPE_BF16"], stream=None)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"],
                      a["T"], a["D"], a["causal"], a["scale"], a["dtype"], a["stream"])


def call_strided(lib, qs=(0, 0, 0), ks=(0, 0, 0), vs=(0, 0, 0), os_=(0, 0, 0), **kw):
    _host_only()
    from exact_attention_91_amd.fa import _LL3
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=4, H_kv=2, T=100, D=64, causal=0,
             scale=0.125, dtype=DT["FA_DTYPE_BF16"])
    a.update(kw)
    return lib.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                              a["H_kv"], a["T"], a["D"], a["causal"], a["scale"], a["dtype"],
                              _LL3(*qs), _LL3(*ks), _LL3(*vs), _LL3(*os_), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), "FA_ERR_DTYPE"),
    (dict(dtype=-1), "FA_ERR_DTYPE"),
    (dict(B=-1), "FA_ERR_BAD_SHAPE"),
    (dict(T=-5), "FA_ERR_BAD_SHAPE"),
    (dict(H=0), "FA_ERR_BAD_SHAPE"),
    (dict(H_kv=0), "FA_ERR_BAD_SHAPE"),
    (dict(H=6, H_kv=4), "FA_ERR_HEADS"),
    (dict(H=2, H_kv=4), "FA_ERR_HEADS"),
    (dict(D=8), "FA_ERR_HEAD_DIM"),
    (dict(D=48), "FA_ERR_HEAD_DIM"),
    (dict(D=256), "FA_ERR_HEAD_DIM"),
    (dict(scale=math.nan), "FA_ERR_SCALE"),
    (dict(scale=math.inf), "FA_ERR_SCALE"),
    (dict(scale=-math.inf), "FA_ERR_SCALE"),
    (dict(scale=3.0e38), "FA_ERR_SCALE"),        # |scale| * log2(e) overflows fp32
    (dict(q=None), "FA_ERR_NULL_PTR"),
    (dict(lse=None), "FA_ERR_NULL_PTR"),
    (dict(o=None), "FA_ERR_NULL_PTR"),
    (dict(q=P + 8), "FA_ERR_ALIGN"),
    (dict(v=P + 2), "FA_ERR_ALIGN"),
    (dict(lse=P + 2), "FA_ERR_ALIGN"),
    (dict(B=1 << 20, H=1 << 10, H_kv=1, T=1 << 12), "FA_ERR_OVERFLOW"),   # grid > 2^24-1
])
def test_fa_fwd_rejects(lib, kw, code):
    assert call(lib, **kw) == ST[code]


def test_fp32_alignment_rule(lib):
    # fp32 rows need 16-byte alignment too
    assert call(lib, dtype=DT["FA_DTYPE_F32"], k=P + 4) == ST["FA_ERR_ALIGN"]


@pytest.mark.parametrize("kw", [dict(B=0), dict(T=0), dict(B=0, q=None, k=None, v=None, o=None,
                                                            lse=None)])
def test_empty_call_is_a_noop(lib, kw):
    # nothing to compute: success without a launch (null pointers allowed)
    assert call(lib, **kw) == ST["FA_OK"]


def test_strided_rejects(lib):
    good = (100 * 4 * 64, 4 * 64, 64)
    kvs = (100 * 2 * 64, 2 * 64, 64)
    base = dict(qs=good, ks=kvs, vs=kvs, os_=good)
    bad_neg = dict(base, ks=(-64, 128, 64))
    assert call_strided(lib, **bad_neg) == ST["FA_ERR_STRIDE"]
    bad_mult = dict(base, vs=(100 * 2 * 64, 2 * 64 + 4, 64))
    assert call_strided(lib, **bad_mult) == ST["FA_ERR_ALIGN"]
    huge = dict(base, qs=(1 << 62, 4 * 64, 64))
    assert call_strided(lib, **huge) == ST["FA_ERR_OVERFLOW"]
    wrap = dict(base, os_=((1 << 62) + 8, 4 * 64, 64))
    assert call_strided(lib, **wrap) == ST["FA_ERR_OVERFLOW"]
    # 64 rows of q (or k, v) at this row stride span more than 2 GiB: the
    # kernel's 32-bit tile offsets would wrap
    for key in ("qs", "ks"):
        far = dict(base, **{key: (100 << 24, 1 << 24, 64)})
        assert call_strided(lib, **far) == ST["FA_ERR_OVERFLOW"]
    from exact_attention_91_amd.fa import _LL3
    _host_only()
    rc = lib.fa_fwd_strided(P, P, P, P, P, 2, 4, 2, 100, 64, 0, 0.125, 1,
                            None, _LL3(*kvs), _LL3(*kvs), _LL3(*good), None)
    assert rc == ST["FA_ERR_NULL_PTR"]


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from exact_attention_91_amd import fa
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "_LIB_PATH", str(tmp_path / "missing" / "libfa.so"))
    with pytest.raises(RuntimeError, match="libfa.so not found"):
        fa.version()


def test_no_unresolved_kernel_stubs(lib):
    """Every kernel the host code launches has its launch stub in the library
    (a kernel template the host pass silently failed to instantiate would leave
    an undefined stub symbol and make dlopen fail at first use)."""
    import subprocess
    out = subprocess.run(["nm", "-D", os.path.join(ROOT, "exact_attention_91_amd", "libfa.so")],
                         capture_output=True, text=True, check=True).stdout
    assert not re.findall(r"\bU \S*device_stub\S*", out)


def call_splitk(lib, **kw):
    _host_only()
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=4, H_kv=2, T=100, D=64, causal=1,
             scale=0.125, dtype=DT["FA_DTYPE_BF16"], nsplit=3, ws=P, ws_bytes=1 << 40)
    a.update(kw)
    return lib.fa_fwd_splitk(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                             a["H_kv"], a["T"], a["D"], a["causal"], a["scale"], a["dtype"],
                             a["nsplit"], a["ws"], a["ws_bytes"], None)


def test_splitk_workspace_bytes(lib):
    f = lib.fa_fwd_splitk_workspace_bytes
    assert f(2, 4, 100, 64, 3) == 3 * 2 * 4 * 100 * 65 * 4
    assert f(16, 12, 1024, 128, 1) == 16 * 12 * 1024 * 129 * 4
    assert f(0, 4, 100, 64, 2) == 0
    assert f(2, 4, 100, 48, 2) == -1      # bad head dim
    assert f(2, 4, 100, 64, 0) == -1      # bad split count
    assert f(2, 0, 100, 64, 2) == -1
    assert f(1 << 30, 1 << 30, 1 << 30, 128, 1 << 30) == -1   # overflow


@pytest.mark.parametrize("kw,code", [
    (dict(nsplit=0), "FA_ERR_BAD_SHAPE"),
    (dict(dtype=DT["FA_DTYPE_F32"]), "FA_ERR_DTYPE"),      # split-K runs the 16-bit kernel
    (dict(dtype=7), "FA_ERR_DTYPE"),
    (dict(D=48), "FA_ERR_HEAD_DIM"),
    (dict(H=6, H_kv=4), "FA_ERR_HEADS"),
    (dict(scale=math.nan), "FA_ERR_SCALE"),
    (dict(q=None), "FA_ERR_NULL_PTR"),
    (dict(ws=None), "FA_ERR_NULL_PTR"),
    (dict(ws_bytes=3 * 2 * 4 * 100 * 65 * 4 - 1), "FA_ERR_WORKSPACE"),
    (dict(ws=P + 4), "FA_ERR_ALIGN"),
    (dict(o=P + 8), "FA_ERR_ALIGN"),
])
def test_splitk_rejects(lib, kw, code):
    assert call_splitk(lib, **kw) == ST[code]


def test_splitk_empty_call_is_a_noop(lib):
    assert call_splitk(lib, B=0, q=None, k=None, v=None, o=None, lse=None, ws=None,
                       ws_bytes=0) == ST["FA_OK"]


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), "FA_ERR_BAD_SHAPE"),
    (dict(H=0), "FA_ERR_BAD_SHAPE"),
    (dict(D=40), "FA_ERR_HEAD_DIM"),
    (dict(dtype=9), "FA_ERR_DTYPE"),
    (dict(op=None), "FA_ERR_NULL_PTR"),
    (dict(lp=None), "FA_ERR_NULL_PTR"),
    (dict(op=P + 4), "FA_ERR_ALIGN"),
    (dict(o=P + 2), "FA_ERR_ALIGN"),
    (dict(B=0, op=None, lp=None, o=None, lse=None), "FA_OK"),
])
def test_lse_combine_rejects(lib, kw, code):
    _host_only()
    a = dict(op=P, lp=P, n=2, B=2, H=4, T=100, D=64, o=P, lse=P, dtype=DT["FA_DTYPE_BF16"])
    a.update(kw)
    rc = lib.fa_lse_combine(a["op"], a["lp"], a["n"], a["B"], a["H"], a["T"], a["D"], a["o"],
                            a["lse"], a["dtype"], None)
    assert rc == ST[code]


def call_bwd(lib, **kw):
    _host_only()
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=2, H=4, H_kv=2, T=100,
             D=64, causal=1, scale=0.125, dtype=DT["FA_DTYPE_BF16"], hsplit=1, ws=P,
             ws_bytes=1 << 40)
    a.update(kw)
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                      a["dv"], a["B"], a["H"], a["H_kv"], a["T"], a["D"], a["causal"],
                      a["scale"], a["dtype"], a["hsplit"], a["ws"], a["ws_bytes"], None)


def test_bwd_workspace_bytes(lib):
    f = lib.fa_bwd_workspace_bytes
    stat = (2 * 4 * 100 * 8 + 15) // 16 * 16
    assert f(2, 4, 2, 100, 64, 1) == stat                    # no head split
    assert f(2, 4, 4, 100, 64, 0) == stat                    # one query head per kv head
    # one query head per kv head, rows of >= 4096 keys and at most 128 key-tile
    # work-groups: the library splits each key tile's query tiles into
    # min(8, ceil(1024 / work-groups)) parts
    # At D = 128 with rows of >= 4096 keys and at most 128 query tiles, dQ's keys
    # are split too: floor(256 / query tiles) parts (at most 8) of fp32 B*T*H*D.
    st = lambda B, H, T: (B * H * T * 8 + 15) // 16 * 16
    assert f(1, 1, 1, 8192, 128, 0) == st(1, 1, 8192) + 8 * 1 * 8192 * 1 * 128 * 8 + \
        4 * 1 * 8192 * 1 * 128 * 4                              # 64 tiles: 8 + 4 parts
    # (at D = 128 the runs also stop at 512 dK/dV work-groups: 128 tiles take 4)
    assert f(2, 1, 1, 8192, 128, 0) == st(2, 1, 8192) + 4 * 2 * 8192 * 1 * 128 * 8 + \
        2 * 2 * 8192 * 1 * 128 * 4                              # 128 tiles: 4 + 2 parts
    assert f(2, 1, 1, 8192, 64, 0) == st(2, 1, 8192) + 8 * 2 * 8192 * 1 * 64 * 8 + \
        2 * 2 * 8192 * 1 * 64 * 4                               # D = 64: 8 + 2 parts
    # query heads at D = 128: 128 key-tile work-groups take 4 head parts, not 8
    assert f(4, 16, 1, 4096, 128, 0) == st(4, 16, 4096) + 4 * 4 * 4096 * 1 * 128 * 8
    assert f(1, 2, 2, 4096, 64, 0) == st(1, 2, 4096) + 8 * 1 * 4096 * 2 * 64 * 8 + \
        4 * 1 * 4096 * 2 * 64 * 4                               # D = 64, 64 tiles: 8 + 4 parts
    assert f(3, 1, 1, 8192, 128, 0) == st(3, 1, 8192)        # 192 tiles: no split
    assert f(1, 1, 1, 4095, 128, 0) == st(1, 1, 4095)        # shorter rows: no split
    # explicit head_split: dK/dV capped at the group; dQ's parts do not depend on it
    assert f(1, 1, 1, 8192, 128, 5) == st(1, 1, 8192) + 4 * 1 * 8192 * 1 * 128 * 4
    assert f(1, 1, 1, 8192, 64, 1) == st(1, 1, 8192) + 4 * 1 * 8192 * 1 * 64 * 4
    assert f(1, 1, 1, 8192, 32, 1) == st(1, 1, 8192)         # D < 64: one dQ group, no parts
    assert f(1, 3, 3, 8192, 64, 1) == st(1, 3, 8192)         # 192 tiles: one dQ part

    # two parts: plus fp32 dK and dV parts of [2][B][T][H_kv][D]
    assert f(2, 4, 2, 100, 64, 2) == stat + 2 * 2 * 100 * 2 * 64 * 8
    assert f(2, 4, 2, 100, 64, 9) == f(2, 4, 2, 100, 64, 2)  # capped at the group size
    # the library's choice for 2 key tiles x 2 kv heads x B=2: 8 work-groups -> all 2 parts
    assert f(2, 4, 2, 200, 64, 0) == f(2, 4, 2, 200, 64, 2)
    assert f(0, 4, 2, 100, 64, 0) == 0
    assert f(2, 0, 1, 100, 64, 0) == -1
    assert f(2, 4, 3, 100, 64, 0) == -1                      # H % H_kv
    assert f(2, 4, 2, 100, 48, 0) == -1                      # head dim
    assert f(2, 4, 2, 100, 64, -1) == -1
    assert f(-1, 4, 2, 100, 64, 0) == -1
    assert f(1 << 30, 1 << 30, 1, 1 << 30, 64, 1) == -1


def test_bwd_window_workspace_bytes(lib):
    f = lib.fa_bwd_window_workspace_bytes
    base = lib.fa_bwd_workspace_bytes
    assert f(1, 2, 2, 2000, 64, 40, 0, 0) == base(1, 2, 2, 2000, 64, 0)
    # 3 slots: 16-byte header, slot map (12 -> 16 bytes), then fp32 dK and dV
    # sums of [slots][parts][B][H_kv][D]; parts = 1 head part + 7 far chunks
    # (32 query tiles of 64 in runs of the band's 5)
    assert f(1, 2, 2, 2000, 64, 40, 3, 0) == base(1, 2, 2, 2000, 64, 0) + 16 + 16 + \
        3 * 8 * 1 * 2 * 64 * 8
    # slots 1..4 share a 16-byte map; each slot adds parts x B x H_kv x D x 8
    # bytes with parts = 3 head parts + at least one far chunk
    extra = [f(2, 6, 1, 1800, 64, 50, n, 3) - base(2, 6, 1, 1800, 64, 3) for n in (1, 2, 4)]
    per = extra[1] - extra[0]
    assert per > 0 and per % (2 * 1 * 64 * 8) == 0 and (per // (2 * 64 * 8)) >= 3 + 1
    assert extra[2] - extra[0] == 3 * per and extra[0] == 32 + per
    assert f(1, 1, 1, 100, 64, 5, 500, 1) == f(1, 1, 1, 100, 64, 5, 100, 1)   # slots <= T
    # where fa_bwd splits query tiles (H == H_kv, long rows, few key tiles) the
    # window keeps one part -- the same split sums as with head_split = 1 --
    # but they still start past fa_bwd's (larger) size
    extra0 = f(1, 1, 1, 8192, 128, 64, 2, 0) - base(1, 1, 1, 8192, 128, 0)
    extra1 = f(1, 1, 1, 8192, 128, 64, 2, 1) - base(1, 1, 1, 8192, 128, 1)
    assert base(1, 1, 1, 8192, 128, 0) > base(1, 1, 1, 8192, 128, 1)
    assert extra0 == extra1 and extra0 > 32 and (extra0 - 32) % (2 * 1 * 1 * 128 * 8) == 0
    assert f(0, 1, 1, 100, 64, 5, 3, 1) == 0
    assert f(1, 1, 1, 100, 64, -1, 3, 1) == -1
    assert f(1, 1, 1, 100, 64, 5, -1, 1) == -1
    assert f(1, 1, 1, 100, 48, 5, 3, 1) == -1
    assert f(1 << 20, 1 << 10, 1 << 10, 1 << 20, 128, 5, 1 << 20, 1) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=DT["FA_DTYPE_F32"]), "FA_ERR_DTYPE"),     # 16-bit MFMA kernels only
    (dict(dtype=5), "FA_ERR_DTYPE"),
    (dict(B=-1), "FA_ERR_BAD_SHAPE"),
    (dict(H_kv=0), "FA_ERR_BAD_SHAPE"),
    (dict(hsplit=-1), "FA_ERR_BAD_SHAPE"),
    (dict(H=6, H_kv=4), "FA_ERR_HEADS"),
    (dict(D=48), "FA_ERR_HEAD_DIM"),
    (dict(scale=math.inf), "FA_ERR_SCALE"),
    (dict(scale=3.0e38), "FA_ERR_SCALE"),
    (dict(o=None), "FA_ERR_NULL_PTR"),
    (dict(do=None), "FA_ERR_NULL_PTR"),
    (dict(dv=None), "FA_ERR_NULL_PTR"),
    (dict(ws=None), "FA_ERR_NULL_PTR"),
    (dict(dq=P + 8), "FA_ERR_ALIGN"),
    (dict(do=P + 2), "FA_ERR_ALIGN"),
    (dict(ws=P + 4), "FA_ERR_ALIGN"),
    (dict(lse=P + 2), "FA_ERR_ALIGN"),
    (dict(ws_bytes=2 * 2 * 4 * 100 * 4 - 1), "FA_ERR_WORKSPACE"),
    (dict(hsplit=2, ws_bytes=2 * 2 * 4 * 100 * 4 + 1000), "FA_ERR_WORKSPACE"),
    (dict(B=1 << 20, H=1 << 10, H_kv=1, T=1 << 12, ws_bytes=1 << 62), "FA_ERR_OVERFLOW"),
    (dict(B=1, H=1 << 18, H_kv=1, T=64, D=128), "FA_ERR_OVERFLOW"),   # 64-row tile > 2 GiB
])
def test_bwd_rejects(lib, kw, code):
    assert call_bwd(lib, **kw) == ST[code]


@pytest.mark.parametrize("kw", [dict(B=0), dict(T=0),
                                dict(B=0, q=None, k=None, v=None, o=None, lse=None, do=None,
                                     dq=None, dk=None, dv=None, ws=None, ws_bytes=0)])
def test_bwd_empty_call_is_a_noop(lib, kw):
    assert call_bwd(lib, **kw) == ST["FA_OK"]


def call_window(lib, **kw):
    _host_only()
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=4, H_kv=2, T=100, D=64, causal=1, scale=0.125,
             dtype=DT["FA_DTYPE_BF16"], window=16, bits=P)
    a.update(kw)
    return lib.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"],
                             a["T"], a["D"], a["causal"], a["scale"], a["dtype"], a["window"],
                             a["bits"], None)


def test_window_bitmap_bytes(lib):
    f = lib.fa_window_bitmap_bytes
    assert f(100) == 16 and f(64) == 8 and f(65) == 16 and f(0) == 0 and f(-1) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), "FA_ERR_BAD_SHAPE"),
    (dict(dtype=DT["FA_DTYPE_F32"]), "FA_ERR_DTYPE"),
    (dict(D=40), "FA_ERR_HEAD_DIM"),
    (dict(H=3, H_kv=2), "FA_ERR_HEADS"),
    (dict(scale=math.nan), "FA_ERR_SCALE"),
    (dict(q=None), "FA_ERR_NULL_PTR"),
    (dict(bits=P + 4), "FA_ERR_ALIGN"),
    (dict(o=P + 8), "FA_ERR_ALIGN"),
])
def test_window_rejects(lib, kw, code):
    assert call_window(lib, **kw) == ST[code]


def test_window_empty_call_is_a_noop(lib):
    assert call_window(lib, T=0, q=None, k=None, v=None, o=None, lse=None,
                       bits=None) == ST["FA_OK"]


@pytest.mark.parametrize("args,code", [
    ((P, -1, 100, P, 16), "FA_ERR_BAD_SHAPE"),
    ((P, 3, -1, P, 16), "FA_ERR_BAD_SHAPE"),
    ((None, 3, 100, P, 16), "FA_ERR_NULL_PTR"),
    ((P, 3, 100, None, 16), "FA_ERR_NULL_PTR"),
    ((P, 3, 100, P + 4, 16), "FA_ERR_ALIGN"),
    ((P + 2, 3, 100, P, 16), "FA_ERR_ALIGN"),
    ((P, 3, 100, P, 15), "FA_ERR_WORKSPACE"),
    ((None, 0, 0, None, 0), "FA_OK"),
])
def test_window_bitmap_rejects(lib, args, code):
    _host_only()
    assert lib.fa_window_bitmap(*args, None) == ST[code]


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), "FA_ERR_BAD_SHAPE"),
    (dict(bits=P + 4), "FA_ERR_ALIGN"),
    (dict(dtype=DT["FA_DTYPE_F32"]), "FA_ERR_DTYPE"),
    (dict(dq=None), "FA_ERR_NULL_PTR"),
    (dict(ws_bytes=10), "FA_ERR_WORKSPACE"),
    (dict(B=0), "FA_OK"),
])
def test_bwd_window_rejects(lib, kw, code):
    _host_only()
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=2, H=4, H_kv=2, T=100,
             D=64, causal=1, scale=0.125, dtype=DT["FA_DTYPE_BF16"], window=8, bits=P, hsplit=1,
             ws=P, ws_bytes=1 << 40)
    a.update(kw)
    rc = lib.fa_bwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                           a["dv"], a["B"], a["H"], a["H_kv"], a["T"], a["D"], a["causal"],
                           a["scale"], a["dtype"], a["window"], a["bits"], a["hsplit"], a["ws"],
                           a["ws_bytes"], None)
    assert rc == ST[code]


@pytest.mark.parametrize("B,H,T,D,dtype,expect", [
    (16, 12, 1024, 64, "BF16", 1),    # GPT-2 layer: 1536 query tiles
    (8, 1, 8192, 128, "BF16", 2),     # long rows, 512 tiles = every work-group resident
    (8, 12, 4096, 64, "BF16", 1),     # MQA workload: 3072 tiles
    (64, 1, 1024, 64, "BF16", 1),     # 512 tiles of short rows
    (64, 1, 1024, 128, "F16", 1),     # 512 tiles of short rows at D = 128
    (2, 12, 1024, 64, "BF16", 2),     # 192 tiles: under a quarter of 1024
    (32, 1, 1024, 64, "F16", 2),      # 256 tiles: exactly a quarter
    (33, 1, 1024, 64, "BF16", 1),     # 264 tiles, short rows
    (2, 12, 4096, 64, "BF16", 2),     # 768 tiles of 4096-key rows
    (4, 16, 4096, 64, "BF16", 1),     # 2048 tiles: more than the GPU holds
    (1, 128, 128, 128, "BF16", 2),    # 128 tiles: a quarter of 512
    (1, 129, 128, 128, "BF16", 1),
    (1, 1, 2048, 128, "BF16", 2),
    (8, 4, 4096, 128, "BF16", 1),     # 1024 tiles at D = 128
    (1, 1, 1, 64, "BF16", 2),
    (1, 1, 300, 32, "BF16", 1),       # D < 64: one group
    (1, 1, 300, 16, "F16", 1),
    (1, 1, 8192, 128, "F32", 1),      # the fp32 kernel has one group
    (0, 4, 100, 64, "BF16", 2),       # empty launch: nothing runs
])
def test_key_groups_rule(lib, B, H, T, D, dtype, expect):
    """The launch-shape rule fa_fwd_key_groups reports (pure host code)."""
    assert lib.fa_fwd_key_groups(B, H, T, D, DT["FA_DTYPE_" + dtype]) == expect


@pytest.mark.parametrize("args", [(-1, 1, 10, 64, 1), (1, 0, 10, 64, 1), (1, 1, -1, 64, 1),
                                  (1, 1, 10, 48, 1), (1, 1, 10, 64, 3), (1, 1, 10, 64, -1)])
def test_key_groups_invalid(lib, args):
    assert lib.fa_fwd_key_groups(*args) == -1


# The binding reads B, T and D from q alone, so k and v of another shape would
# be read (and, in the backward, dk/dv written) past their allocations. Every
# entry point must reject them before any device check or library call; CPU
# tensors are enough to show the order.
_BAD_KV = [
    ((2, 64, 4, 32), (2, 64, 2, 32), (2, 64, 1, 32)),   # k and v differ in heads
    ((2, 64, 4, 32), (1, 64, 2, 32), (1, 64, 2, 32)),   # batch
    ((2, 64, 4, 32), (2, 63, 2, 32), (2, 63, 2, 32)),   # tokens
    ((2, 64, 4, 32), (2, 64, 2, 16), (2, 64, 2, 16)),   # head dim
    ((2, 64, 4, 32), (2, 64, 2, 32), (2, 65, 2, 32)),   # v alone longer
    ((2, 64, 4, 32), (2, 64, 2, 32, 1), (2, 64, 2, 32)),  # k not 4-D
]


@pytest.mark.parametrize("qs,ks,vs", _BAD_KV)
def test_binding_rejects_mismatched_kv(qs, ks, vs):
    import torch
    from exact_attention_91_amd import fa
    q = torch.zeros(qs, dtype=torch.bfloat16)
    k = torch.zeros(ks, dtype=torch.bfloat16)
    v = torch.zeros(vs, dtype=torch.bfloat16)
    o = torch.zeros(qs, dtype=torch.bfloat16)
    lse = torch.zeros((qs[0], qs[2], qs[1]), dtype=torch.float32)
    calls = [
        lambda: fa.fwd(q, k, v, causal=True),
        lambda: fa.fwd_strided(q, k, v, causal=True),
        lambda: fa.fwd_splitk(q, k, v, causal=True, nsplit=2),
        lambda: fa.fwd_window(q, k, v, 8, causal=True),
        lambda: fa.bwd(q, k, v, o, lse, o, causal=True),
        lambda: fa.bwd_window(q, k, v, o, lse, o, 8, causal=True),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="k/v|k and v|4-D"):
            call()


def test_binding_shape_check_accepts_grouped_heads():
    import torch
    from exact_attention_91_amd import fa
    q = torch.zeros((2, 64, 4, 32))
    kv = torch.zeros((2, 64, 2, 32))
    fa.check_shapes(q, kv, kv)   # H_kv = 2 divides H = 4: the library checks the rest


def test_roof_entry_points_reject_bad_arguments(lib):
    """The microbenchmarks validate their arguments before any HIP call."""
    _host_only()
    VP, I, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.fa_roof_mfma.argtypes = [I, I, VP, VP]
    lib.fa_roof_valu.argtypes = [I, I, I, VP, VP]
    lib.fa_roof_overlap.argtypes = [I, I, I, I, I, VP, VP]
    lib.fa_roof_copy.argtypes = [VP, VP, LL, VP]
    assert lib.fa_roof_mfma(0, 10, P, None) == 2
    assert lib.fa_roof_mfma(4, 0, P, None) == 2
    assert lib.fa_roof_mfma(4, 10, None, None) == 1
    assert lib.fa_roof_valu(4, 10, 2, P, None) == 2
    assert lib.fa_roof_valu(4, 10, 0, None, None) == 1
    assert lib.fa_roof_overlap(4, 10, 10, 0, 0, P, None) == 2
    assert lib.fa_roof_overlap(4, 10, 10, 0, 4, P, None) == 2
    assert lib.fa_roof_overlap(4, 10, 10, 5, 3, P, None) == 2
    assert lib.fa_roof_overlap(4, 10, 10, 1, 3, None, None) == 1
    assert lib.fa_roof_copy(P, P, 0, None) == 2
    assert lib.fa_roof_copy(None, P, 64, None) == 1
    assert lib.fa_roof_copy(P, P, 40, None) == 7
    assert lib.fa_roof_copy(P + 4, P, 64, None) == 7
    lib.fa_roof_read.argtypes = [VP, LL, VP, VP]
    assert lib.fa_roof_read(P, 0, P, None) == 2
    assert lib.fa_roof_read(None, 64, P, None) == 1
    assert lib.fa_roof_read(P, 64, None, None) == 1
    assert lib.fa_roof_read(P, 40, P, None) == 7


def test_splitk_noalloc_rejects_before_any_hip_call(lib):
    """The allocation-free key split validates everything, including that its
    partials fit the fixed scratch, before its first HIP call (the scratch
    address lookup)."""
    _host_only()
    VP, I = ctypes.c_void_p, ctypes.c_int
    lib.fa_fwd_splitk_noalloc.argtypes = [VP] * 5 + [I] * 6 + [ctypes.c_float, I, I, VP]
    lib.fa_fwd_splitk_scratch_bytes.restype = ctypes.c_longlong
    lib.fa_fwd_splitk_workspace_bytes.restype = ctypes.c_longlong
    assert lib.fa_fwd_splitk_scratch_bytes() == 64 << 20

    def run(B=2, H=4, H_kv=2, T=1000, D=64, nsplit=4, dtype=DT["FA_DTYPE_BF16"], q=P):
        return lib.fa_fwd_splitk_noalloc(q, P, P, P, P, B, H, H_kv, T, D, 1, 0.125, dtype,
                                         nsplit, None)
    assert run(nsplit=0) == ST["FA_ERR_BAD_SHAPE"]
    assert run(dtype=DT["FA_DTYPE_F32"]) == ST["FA_ERR_DTYPE"]
    assert run(q=None) == ST["FA_ERR_NULL_PTR"]
    assert run(D=48) == ST["FA_ERR_HEAD_DIM"]
    assert run(B=0) == ST["FA_OK"]          # empty call: nothing launched
    big = dict(B=4, H=8, T=8192, D=128, nsplit=8)
    assert lib.fa_fwd_splitk_workspace_bytes(4, 8, 8192, 128, 8) > 64 << 20
    assert run(H_kv=8, **big) == ST["FA_ERR_SCRATCH"]


def test_size_heuristics_saturate(lib):
    """The kernel-variant choice for absurd sizes: the unit count saturates
    instead of overflowing (found by the UndefinedBehaviorSanitizer leg)."""
    lib.fa_fwd_key_groups.argtypes = [ctypes.c_int] * 5
    assert lib.fa_fwd_key_groups(1 << 30, 1 << 30, 1 << 30, 64, DT["FA_DTYPE_BF16"]) == 1
    assert lib.fa_fwd_key_groups((1 << 31) - 1, (1 << 31) - 1, (1 << 31) - 1, 128,
                                 DT["FA_DTYPE_F16"]) == 1
    lib.fa_bwd_workspace_bytes.argtypes = [ctypes.c_int] * 6
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_longlong
    assert lib.fa_bwd_workspace_bytes((1 << 31) - 1, (1 << 31) - 1, 1, (1 << 31) - 1, 128, 0) == -1


def test_sequence_length_limit(lib):
    """T above 2^30 is rejected (the kernels use 32-bit row arithmetic)."""
    _host_only()
    assert call(lib, B=1, H=1, H_kv=1, T=(1 << 30) + 1) == ST["FA_ERR_OVERFLOW"]


def test_decode_rejects_and_workspace(lib):
    """fa_fwd_decode validates before any HIP call; its workspace size."""
    _host_only()
    VP, I = ctypes.c_void_p, ctypes.c_int
    lib.fa_fwd_decode.argtypes = [VP] * 5 + [I] * 7 + [ctypes.c_float, I, I, VP,
                                                        ctypes.c_longlong, VP]
    lib.fa_fwd_decode_workspace_bytes.argtypes = [I] * 5
    lib.fa_fwd_decode_workspace_bytes.restype = ctypes.c_longlong
    ws = lib.fa_fwd_decode_workspace_bytes
    assert ws(2, 8, 3, 64, 4) == 4 * 2 * 8 * 3 * 65 * 4
    assert ws(2, 8, 3, 48, 4) == -1 and ws(2, 8, 3, 64, 0) == -1 and ws(-1, 8, 3, 64, 1) == -1

    def run(B=2, H=8, H_kv=2, Tq=3, Tk=500, D=64, dtype=DT["FA_DTYPE_BF16"], nsplit=4,
            wsb=1 << 20, q=P, scale=0.125):
        return lib.fa_fwd_decode(q, P, P, P, P, B, H, H_kv, Tq, Tk, D, 1, scale, dtype, nsplit,
                                 P, wsb, None)
    assert run(dtype=DT["FA_DTYPE_F32"]) == ST["FA_ERR_DTYPE"]
    assert run(Tk=0) == ST["FA_ERR_BAD_SHAPE"]
    assert run(nsplit=0) == ST["FA_ERR_BAD_SHAPE"]
    assert run(H_kv=3) == ST["FA_ERR_HEADS"]
    assert run(D=48) == ST["FA_ERR_HEAD_DIM"]
    assert run(scale=float("inf")) == ST["FA_ERR_SCALE"]
    assert run(q=None) == ST["FA_ERR_NULL_PTR"]
    assert run(q=P + 8) == ST["FA_ERR_ALIGN"]
    assert run(wsb=100) == ST["FA_ERR_WORKSPACE"]
    assert run(Tq=(1 << 30) + 1) == ST["FA_ERR_OVERFLOW"]
    assert run(B=0) == ST["FA_OK"] and run(Tq=0) == ST["FA_OK"]
