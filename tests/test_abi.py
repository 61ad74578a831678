"""CPU tests of the C ABI: the library loads without a GPU, exports every
function that include/fa.h declares, and rejects invalid arguments on the
host before any HIP call (null device pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

from io_aware_exact_flashattention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from io_aware_exact_flashattention_amd import build
        build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(5):
        assert lib.fa_status_string(s).decode().startswith(
            ["FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP",
             "FA_ERR_NO_SPACE"][s])
    assert lib.fa_version() >= 100


P = 16  # a fake, 16-byte aligned non-null address; never dereferenced on the error paths


def fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Nq=8, Nk=8, Hq=2, Hkv=1, d=64, dt=2, scale=0.125,
             causal=0, stream=None)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Nq"], a["Nk"], a["Hq"],
                      a["Hkv"], a["d"], a["dt"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), 1), (dict(lse=None), 1), (dict(B=0), 1), (dict(Nq=-1), 1), (dict(Nk=0), 1),
    (dict(Hq=3, Hkv=2), 1), (dict(Hkv=0), 1), (dict(dt=7), 1), (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(scale=-0.1), 1),
    (dict(q=18), 1), (dict(d=96), 2), (dict(d=256), 2),
])
def test_fwd_rejects(lib, kw, expect):
    assert fwd(lib, **kw) == expect


def varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, B=2, mq=8, mk=8, Tq=16, Tk=16, Hq=2, Hkv=2,
             d=128, dt=1, scale=0.1, causal=1, stream=None)
    a.update(kw)
    return lib.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["B"],
                             a["mq"], a["mk"], a["Tq"], a["Tk"], a["Hq"], a["Hkv"], a["d"], a["dt"],
                             a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(cq=None), 1), (dict(ck=None), 1), (dict(B=0), 1), (dict(mq=-1), 1), (dict(Tq=-1), 1),
    (dict(mq=17), 1), (dict(d=32), 2),
])
def test_varlen_rejects(lib, kw, expect):
    assert varlen(lib, **kw) == expect


def test_varlen_empty_is_noop(lib):
    # no query rows: success without touching any pointer or the GPU
    assert varlen(lib, Tq=0, mq=0) == 0


def decode(lib, **kw):
    a = dict(q=P, kp=P, vp=P, o=P, lse=P, pt=P, sl=P, B=2, mp=4, npg=8, ps=16, Hq=4, Hkv=1, d=128,
             dt=2, scale=0.1, ns=0, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.fa_decode_paged(a["q"], a["kp"], a["vp"], a["o"], a["lse"], a["pt"], a["sl"], a["B"],
                               a["mp"], a["npg"], a["ps"], a["Hq"], a["Hkv"], a["d"], a["dt"],
                               a["scale"], a["ns"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(pt=None), 1), (dict(sl=None), 1), (dict(ws=None), 1), (dict(wsb=16), 1),
    (dict(ns=-1), 1), (dict(ns=5), 1), (dict(mp=0), 1), (dict(ps=8), 2), (dict(dt=0), 2),
    (dict(Hq=4, Hkv=3), 1), (dict(d=80), 2), (dict(ws=24), 1),
])
def test_decode_rejects(lib, kw, expect):
    assert decode(lib, **kw) == expect


def decode_noalloc(lib, **kw):
    a = dict(q=P, kp=P, vp=P, o=P, lse=P, pt=P, sl=P, B=2, mp=4, npg=8, ps=16, Hq=4, Hkv=1, d=128,
             dt=2, scale=0.1, ns=0, stream=None)
    a.update(kw)
    return lib.fa_decode_paged_noalloc(a["q"], a["kp"], a["vp"], a["o"], a["lse"], a["pt"], a["sl"],
                                       a["B"], a["mp"], a["npg"], a["ps"], a["Hq"], a["Hkv"], a["d"],
                                       a["dt"], a["scale"], a["ns"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(pt=None), 1), (dict(sl=None), 1), (dict(ns=-1), 1), (dict(ns=5), 1), (dict(mp=0), 1),
    (dict(ps=8), 2), (dict(dt=0), 2), (dict(Hq=4, Hkv=3), 1), (dict(d=80), 2),
    # more partials than the fixed device buffer holds: 128 x 64 heads x 43 splits x 129 floats
    (dict(B=128, Hq=64, Hkv=8, mp=2017, npg=75219), 4),
])
def test_decode_noalloc_rejects(lib, kw, expect):
    assert decode_noalloc(lib, **kw) == expect


def test_workspace_size(lib):
    f = lib.fa_decode_paged_workspace_size
    # auto split: 48 pages per split
    assert f(64, 32, 128, 2017, 16, 0) == 64 * 32 * 43 * 129 * 4
    assert f(2, 4, 64, 10, 16, 3) == 2 * 4 * 3 * 65 * 4        # ceil(10/3)=4 pages -> 3 splits
    assert f(2, 4, 64, 10, 16, 1) == 2 * 4 * 1 * 65 * 4
    # a split holds at most 64 pages: one split over 200 pages becomes 4
    assert f(1, 1, 128, 200, 16, 1) == 1 * 1 * 4 * 129 * 4
    assert f(0, 4, 64, 10, 16, 1) == 0 and f(2, 4, 64, 10, 16, 11) == 0


def fwd_paged(lib, **kw):
    a = dict(q=P, kp=P, vp=P, o=P, lse=P, cq=P, pt=P, sl=P, B=2, mq=8, Tq=16, mp=4, npg=8, ps=16,
             Hq=4, Hkv=2, d=128, dt=2, scale=0.1, causal=1, stream=None)
    a.update(kw)
    return lib.fa_fwd_paged(a["q"], a["kp"], a["vp"], a["o"], a["lse"], a["cq"], a["pt"], a["sl"],
                            a["B"], a["mq"], a["Tq"], a["mp"], a["npg"], a["ps"], a["Hq"], a["Hkv"],
                            a["d"], a["dt"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(cq=None), 1), (dict(pt=None), 1), (dict(sl=None), 1), (dict(B=0), 1), (dict(mq=17), 1),
    (dict(Tq=-1), 1), (dict(mp=0), 1), (dict(npg=0), 1), (dict(ps=8), 2), (dict(dt=0), 2),
    (dict(d=96), 2), (dict(Hq=4, Hkv=3), 1), (dict(mp=8193), 2), (dict(scale=0.0), 1),
])
def test_fwd_paged_rejects(lib, kw, expect):
    assert fwd_paged(lib, **kw) == expect


def test_fwd_paged_empty_is_noop(lib):
    assert fwd_paged(lib, Tq=0, mq=0) == 0


def kv_append(lib, **kw):
    a = dict(kn=P, vn=P, kp=P, vp=P, cu=P, pt=P, lb=P, B=2, T=4, mp=4, npg=8, ps=16, Hkv=2, d=128,
             dt=2, stream=None)
    a.update(kw)
    return lib.fa_kv_append(a["kn"], a["vn"], a["kp"], a["vp"], a["cu"], a["pt"], a["lb"], a["B"],
                            a["T"], a["mp"], a["npg"], a["ps"], a["Hkv"], a["d"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(kn=None), 1), (dict(vp=None), 1), (dict(cu=None), 1), (dict(pt=None), 1), (dict(lb=None), 1),
    (dict(B=0), 1), (dict(T=-1), 1), (dict(mp=0), 1), (dict(npg=0), 1), (dict(Hkv=0), 1),
    (dict(dt=5), 1), (dict(kp=24), 1), (dict(ps=32), 2), (dict(d=80), 2),
])
def test_kv_append_rejects(lib, kw, expect):
    assert kv_append(lib, **kw) == expect


def test_kv_append_empty_is_noop(lib):
    assert kv_append(lib, T=0) == 0


def cascade(lib, **kw):
    a = dict(q=P, kp=P, vp=P, o=P, lse=P, pp=P, pl=100, pt=P, sl=P, B=2, mp=4, npg=8, ps=16, Hq=4,
             Hkv=1, d=128, dt=2, scale=0.1, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.fa_decode_cascade(a["q"], a["kp"], a["vp"], a["o"], a["lse"], a["pp"], a["pl"], a["pt"],
                                 a["sl"], a["B"], a["mp"], a["npg"], a["ps"], a["Hq"], a["Hkv"], a["d"],
                                 a["dt"], a["scale"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(pp=None), 1), (dict(pl=-1), 1), (dict(pt=None), 1), (dict(ws=None), 1), (dict(wsb=16), 1),
    (dict(B=0), 1), (dict(mp=0), 1), (dict(ps=8), 2), (dict(dt=0), 2), (dict(d=80), 2),
])
def test_cascade_rejects(lib, kw, expect):
    assert cascade(lib, **kw) == expect


def test_cascade_workspace_size(lib):
    f = lib.fa_decode_cascade_workspace_size
    # prefix 100 tokens = 7 pages -> 1 split of <= 32 pages; suffix 4 pages
    # -> 1 split of <= 8 pages
    assert f(2, 4, 128, 100, 4, 16) == 2 * 4 * 2 * 129 * 4
    assert f(2, 4, 128, 0, 4, 16) == 2 * 4 * 1 * 129 * 4
    assert f(1, 1, 64, 16384, 70, 16) == 1 * 1 * (32 + 9) * 65 * 4
    assert f(0, 4, 128, 1, 4, 16) == 0


def bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Nq=8, Nk=8, Hq=2, Hkv=1,
             d=64, dt=2, scale=0.125, causal=1, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                      a["B"], a["Nq"], a["Nk"], a["Hq"], a["Hkv"], a["d"], a["dt"], a["scale"],
                      a["causal"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(do=None), 1), (dict(dq=None), 1), (dict(dk=None), 1), (dict(dv=None), 1),
    (dict(ws=None), 1), (dict(wsb=2 * 2 * 64 * 4 - 1), 1), (dict(o=None), 1), (dict(dq=40), 1),
    (dict(B=0), 1), (dict(Nk=0), 1), (dict(Hq=3, Hkv=2), 1), (dict(dt=0), 2), (dict(d=96), 2),
    (dict(scale=float("nan")), 1),
])
def test_bwd_rejects(lib, kw, expect):
    assert bwd(lib, **kw) == expect


def test_bwd_workspace_size(lib):
    assert lib.fa_bwd_workspace_size(4, 2048, 16) == 2 * 4 * 2048 * 16 * 4
    assert lib.fa_bwd_workspace_size(1, 65, 3) == 2 * 1 * 128 * 3 * 4  # rows padded to 64
    assert lib.fa_bwd_workspace_size(0, 2048, 16) == 0
