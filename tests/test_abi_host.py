"""C ABI on the host (no GPU): the library loads, exports every entry point that
include/fastar.h declares, and rejects bad arguments with the documented
status before launching anything.  Fake device pointers used here are never
dereferenced: each call below fails validation first."""
import ctypes
import os
import re

import pytest

from sparse_attention_autoregressive_amd import _lib
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fastar.h")
FAKE = 0x100000          # 16-byte aligned, never dereferenced
MISALIGNED = 0x100008


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fastar_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"


def test_status_strings_and_version(lib):
    assert lib.fastar_abi_version() == _lib.FASTAR_ABI_VERSION == 3
    for code, name in [(0, "FASTAR_OK"), (-1, "FASTAR_EINVAL"), (-2, "FASTAR_EDTYPE"),
                       (-3, "FASTAR_ESHAPE"), (-4, "FASTAR_EWORKSPACE"), (-5, "FASTAR_ECAPACITY"),
                       (-6, "FASTAR_EHIP"), (-7, "FASTAR_ESCRATCH")]:
        assert lib.fastar_status_string(code).decode() == name
    assert lib.fastar_status_string(99).decode() == "FASTAR_UNKNOWN"


def test_hash_validation(lib):
    h = lib.fastar_ann_hash
    assert h(FAKE, 7, 1, 4, 64, FAKE, 4, FAKE, None, None) == _lib.FASTAR_EDTYPE
    assert h(FAKE, 0, 1, 4, 96, FAKE, 4, FAKE, None, None) == _lib.FASTAR_ESHAPE
    assert h(FAKE, 0, 1, 4, 64, FAKE, 17, FAKE, None, None) == _lib.FASTAR_ESHAPE
    assert h(FAKE, 0, 1, -1, 64, FAKE, 4, FAKE, None, None) == _lib.FASTAR_EINVAL
    assert h(None, 0, 1, 4, 64, FAKE, 4, FAKE, None, None) == _lib.FASTAR_EINVAL
    assert h(MISALIGNED, 0, 1, 4, 64, FAKE, 4, FAKE, None, None) == _lib.FASTAR_EINVAL
    assert h(FAKE, 0, 1, 4, 64, None, 4, FAKE, None, None) == _lib.FASTAR_EINVAL
    assert h(FAKE, 1, 1, 4, 128, FAKE, 4, None, None, None) == _lib.FASTAR_EINVAL
    # empty work is a no-op that succeeds without touching the device
    assert h(None, 0, 0, 4, 64, None, 4, None, None, None) == _lib.FASTAR_OK
    assert h(None, 1, 3, 0, 128, None, 4, None, None, None) == _lib.FASTAR_OK


def test_workspace_queries(lib):
    a = lib.fastar_annsa_workspace(12, 4680, 32760, 4680, 7)
    assert a > 12 * (4680 + 32760 + 4680) * 4
    assert lib.fastar_annsa_workspace(12, 4680, 32760, 4680, 8) > a
    assert lib.fastar_annsa_workspace(1, 10, 0, 0, 11) == 0          # P out of range
    assert lib.fastar_tempcache_workspace(12, 4680, 32760, 7) > 12 * 32760 * 4
    assert lib.fastar_annca_workspace(12, 4680, 1560, 512, 7) == 0      # selection inside the blocks
    assert lib.fastar_annca_workspace(12, 4680, 1560, 1024, 7) == 0
    assert lib.fastar_annca_workspace(12, 4680, 1560, 1025, 7) >= 12 * 3 * 1025 * 4
    assert lib.fastar_bucket_sort_workspace(2, 1000, 5) > 0
    assert lib.fastar_bucket_sort_workspace(2, 0, 5) == 0


def _cache(H=1, cap=64, d=64, dtype=0, knorm=FAKE, count=None):
    return _lib.FastarCache(H, cap, d, dtype, FAKE, FAKE, FAKE, FAKE, FAKE, knorm, count)


def test_annsa_validation(lib):
    f = lib.fastar_annsa_forward
    need = lib.fastar_annsa_workspace(1, 32, 64, 16, 4)
    c = _cache()
    args = lambda **kw: [kw.get("q", FAKE), FAKE, 1, 32, kw.get("d", 64), kw.get("dt", 0),
                         kw.get("cache", ctypes.byref(c)), FAKE, FAKE, FAKE, 16, kw.get("P", 4),
                         kw.get("scale", 0.125), FAKE, kw.get("odt", 0), None,
                         kw.get("best", None), kw.get("bcos", None), FAKE,
                         kw.get("ws", need), None]
    assert f(*args(ws=need - 1)) == _lib.FASTAR_EWORKSPACE
    assert f(*args(P=11)) == _lib.FASTAR_ESHAPE
    assert f(*args(d=80)) == _lib.FASTAR_ESHAPE
    assert f(*args(dt=1)) == _lib.FASTAR_EDTYPE          # cache is fp32
    assert f(*args(odt=5)) == _lib.FASTAR_EDTYPE
    assert f(*args(scale=float("nan"))) == _lib.FASTAR_EINVAL
    assert f(*args(scale=0.0)) == _lib.FASTAR_EINVAL
    assert f(*args(scale=-0.5)) == _lib.FASTAR_EINVAL
    assert f(*args(q=MISALIGNED)) == _lib.FASTAR_EINVAL
    c2 = _cache(H=2)
    assert f(*args(cache=ctypes.byref(c2))) == _lib.FASTAR_ESHAPE
    assert f(*args(best=FAKE)) == _lib.FASTAR_EINVAL                 # best without cos
    c3 = _cache(knorm=None)
    assert f(*args(best=FAKE, bcos=FAKE, cache=ctypes.byref(c3))) == _lib.FASTAR_EINVAL


def test_annsa_multi_validation(lib):
    f = lib.fastar_annsa_multi_forward
    wq = lib.fastar_annsa_multi_workspace
    assert wq(1, 32, 64, 16, 64, 4, 2) > lib.fastar_annsa_workspace(1, 32, 64, 16, 4)
    assert wq(1, 32, 64, 16, 64, 4, 1) == lib.fastar_annsa_workspace(1, 32, 64, 16, 4)
    assert wq(1, 32, 64, 16, 64, 6, 3) == 0               # 18 id bits
    assert wq(1, 32, 64, 16, 64, 2, 9) == 0               # above FASTAR_MAX_TABLES
    assert wq(1, 32, 64, 16, 64, 4, 0) == 0
    assert wq(1, 32, 64, 16, 80, 4, 2) == 0               # d
    need = wq(1, 32, 64, 16, 64, 4, 2)
    c = _cache()
    args = lambda **kw: [FAKE, FAKE, 1, 32, 64, 0, ctypes.byref(c), FAKE, FAKE, FAKE, 16,
                         kw.get("P", 4), kw.get("T", 2), 0.125, FAKE, 0, None, None, None, FAKE,
                         kw.get("ws", need), None]
    assert f(*args(ws=need - 1)) == _lib.FASTAR_EWORKSPACE
    assert f(*args(T=0)) == _lib.FASTAR_ESHAPE
    assert f(*args(P=6, T=3)) == _lib.FASTAR_ESHAPE
    assert f(*args(P=11, T=1)) == _lib.FASTAR_ESHAPE
    assert _lib.FASTAR_MAX_TABLES == 8


def test_hash_batch_validation(lib):
    f = lib.fastar_ann_hash_batch
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    ns = lambda *v: (ctypes.c_int32 * len(v))(*v)
    ok = lambda c, **kw: f(c, arr(*([FAKE] * c)), ns(*([10] * c)), arr(*([FAKE] * c)), None,
                           kw.get("dt", 0), 2, kw.get("d", 64), FAKE, kw.get("P", 4), None)
    assert ok(0) == _lib.FASTAR_EINVAL
    assert ok(5) == _lib.FASTAR_EINVAL
    assert ok(2, d=96) == _lib.FASTAR_ESHAPE
    assert ok(2, P=17) == _lib.FASTAR_ESHAPE
    assert ok(2, dt=3) == _lib.FASTAR_EDTYPE
    assert f(2, arr(FAKE, MISALIGNED), ns(10, 10), arr(FAKE, FAKE), None, 0, 2, 64, FAKE, 4,
             None) == _lib.FASTAR_EINVAL
    assert f(2, arr(FAKE, FAKE), ns(10, -1), arr(FAKE, FAKE), None, 0, 2, 64, FAKE, 4,
             None) == _lib.FASTAR_EINVAL
    assert _lib.FASTAR_HASH_BATCH == 4


def test_quantize_validation(lib):
    f = lib.fastar_ann_quantize
    base = lambda **kw: [FAKE, kw.get("dt", 0), 2, 10, kw.get("d", 64), FAKE, kw.get("B", 16), FAKE,
                         None, None]
    assert f(*base(B=0)) == _lib.FASTAR_ESHAPE
    assert f(*base(B=65537)) == _lib.FASTAR_ESHAPE
    assert f(*base(d=96)) == _lib.FASTAR_ESHAPE
    assert f(*base(dt=7)) == _lib.FASTAR_EDTYPE
    args = base()
    args[5] = MISALIGNED
    assert f(*args) == _lib.FASTAR_EINVAL
    assert _lib.FASTAR_MAX_CODEWORDS == 65536


def test_annca_validation(lib):
    f = lib.fastar_annca_forward
    need = lib.fastar_annca_workspace(1, 30, 10, 1100, 4)     # a prompt long enough to need it
    assert need > 0
    base = [FAKE, FAKE, 1, 30, 10, 64, 0, FAKE, FAKE, FAKE, 1100, 4, 0.125, FAKE, 0, None, None]
    assert f(*(base + [FAKE, need - 1, None])) == _lib.FASTAR_EWORKSPACE
    bad = list(base); bad[4] = 7                         # 7 does not divide 30
    assert f(*(bad + [FAKE, need, None])) == _lib.FASTAR_ESHAPE
    bad = list(base); bad[4] = 0
    assert f(*(bad + [FAKE, need, None])) == _lib.FASTAR_ESHAPE
    bad = list(base); bad[7] = None                      # prompt keys missing
    assert f(*(bad + [FAKE, need, None])) == _lib.FASTAR_EINVAL


def test_tempcache_validation(lib):
    f = lib.fastar_tempcache_update
    c = _cache(cap=64)
    need = lib.fastar_tempcache_workspace(1, 32, 64, 4)
    def call(N=32, cache=c, tau=0.9, best_in=None, cos_in=None, ws=need, P=4):
        return f(ctypes.byref(cache) if cache is not None else None, FAKE, FAKE, FAKE, FAKE, FAKE,
                 N, P, tau, 3, best_in, cos_in, None, None, None, None, None, None, FAKE, ws, None)
    assert call(ws=need - 1) == _lib.FASTAR_EWORKSPACE
    assert call(N=65) == _lib.FASTAR_ECAPACITY
    assert call(tau=float("nan")) == _lib.FASTAR_EINVAL
    assert call(best_in=FAKE) == _lib.FASTAR_EINVAL      # best without cos
    assert call(cache=None) == _lib.FASTAR_EINVAL
    assert call(P=12) == _lib.FASTAR_ESHAPE
    bad = _cache(cap=64, dtype=3)
    assert call(cache=bad) == _lib.FASTAR_EDTYPE
    assert call(cache=_cache(cap=64, knorm=None)) == _lib.FASTAR_EINVAL   # norms are needed


def test_tempcache_order_validation(lib):
    f = lib.fastar_tempcache_order
    c = _cache(cap=64)
    assert f(None, 32, FAKE, None) == _lib.FASTAR_EINVAL
    assert f(ctypes.byref(c), 65, FAKE, None) == _lib.FASTAR_ECAPACITY
    assert f(ctypes.byref(c), -1, FAKE, None) == _lib.FASTAR_EINVAL
    assert f(ctypes.byref(c), 32, None, None) == _lib.FASTAR_EINVAL      # no output buffer
    assert f(ctypes.byref(c), 0, None, None) == _lib.FASTAR_OK           # nothing to list
    no_ts = _cache(cap=64)
    no_ts.ts = None
    assert f(ctypes.byref(no_ts), 32, FAKE, None) == _lib.FASTAR_EINVAL


def test_bucket_sort_validation(lib):
    f = lib.fastar_bucket_sort
    need = lib.fastar_bucket_sort_workspace(2, 100, 5)
    assert f(FAKE, 2, 100, 5, FAKE, FAKE, FAKE, need - 1, None) == _lib.FASTAR_EWORKSPACE
    assert f(FAKE, 2, 100, 11, FAKE, FAKE, FAKE, need, None) == _lib.FASTAR_ESHAPE
    assert f(None, 2, 100, 5, FAKE, FAKE, FAKE, need, None) == _lib.FASTAR_EINVAL


def test_timer_without_launches(lib):
    assert lib.fastar_timer_start() == 0
    buf = (_lib.FastarKernelTime * 4)()
    assert lib.fastar_timer_stop(buf, 4) == 0


def test_cache_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of fastar_cache has the header's size and offsets
    (a C program built from include/fastar.h prints them)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = tmp_path / "layout.c"
    names = [n for n, _ in _lib.FastarCache._fields_]
    body = "".join(f'    printf("%zu\\n", offsetof(fastar_cache, {n}));\n' for n in names)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "fastar.h"\n'
                   'int main(void) {\n    printf("%zu\\n", sizeof(fastar_cache));\n' + body +
                   '    return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-I", os.path.join(root, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(_lib.FastarCache)
    assert out[1:] == [getattr(_lib.FastarCache, n).offset for n in names]


def test_static_scratch_entry_validates_before_touching_the_device(lib):
    """fastar_annsa_forward_static rejects bad arguments like
    fastar_annsa_forward, and a call whose workspace exceeds the static array
    with FASTAR_ESCRATCH -- all before resolving the array or launching."""
    f = lib.fastar_annsa_forward_static
    c = _cache(H=1, cap=64, d=64)
    args = lambda **kw: dict(dict(q=FAKE, q_ids=FAKE, H=1, Nq=32, d=64, dt=0, cache=c, kc=FAKE, vc=FAKE,
                                  kid=FAKE, Ncur=16, P=4, scale=0.125, out=FAKE, odt=0), **kw)
    call = lambda a: f(a["q"], a["q_ids"], a["H"], a["Nq"], a["d"], a["dt"], ctypes.byref(a["cache"]),
                       a["kc"], a["vc"], a["kid"], a["Ncur"], a["P"], a["scale"], a["out"], a["odt"],
                       None, None, None, None)
    assert call(args(d=96)) == _lib.FASTAR_ESHAPE
    assert call(args(dt=5)) == _lib.FASTAR_EDTYPE
    assert call(args(q=None)) == _lib.FASTAR_EINVAL
    assert call(args(scale=-1.0)) == _lib.FASTAR_EINVAL
    big = _cache(H=8, cap=1_000_000, d=128, dtype=1)
    need = lib.fastar_annsa_workspace(8, 4680, 1_000_000, 4680, 10)
    assert need > _lib.FASTAR_STATIC_SCRATCH_BYTES
    assert call(args(H=8, Nq=4680, d=128, dt=1, cache=big, Ncur=4680, P=10)) == _lib.FASTAR_ESCRATCH
    # empty work succeeds without touching the device
    assert call(args(Nq=0, q=None, out=None, q_ids=None)) == _lib.FASTAR_OK
