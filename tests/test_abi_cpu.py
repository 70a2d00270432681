"""The C-ABI library on the CPU: it loads, exports every function that
include/fusednorm.h declares, reports its version, and rejects every invalid or
unsupported argument before touching the HIP runtime.

The calls below use made-up (aligned, never dereferenced) device addresses and
are all either rejected by validation or empty (T = 0), so nothing is launched.
Where a GPU is visible these cases run with real buffers in the GPU suite
instead, so that a validation bug could never launch on fake addresses.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fusednorm.h")

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake-address validation runs only where no GPU is visible")


@pytest.fixture(scope="module")
def lib():
    from residual_add_rmsnorm_amd import _build
    srcs = _build.SOURCES + [HEADER, os.path.join(_build.CSRC, "fusednorm_internal.h")]
    if not os.path.exists(_build.LIB) or any(
            os.path.getmtime(s) > os.path.getmtime(_build.LIB) for s in srcs):
        _build.build()
    from residual_add_rmsnorm_amd import fusednorm
    return fusednorm._lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:FUSEDNORM_API\s+)?(?:const\s+)?(?:int|char\s*\*|const char\s*\*)"
                      r"\s*\**\s*(\w+)\s*\(", text, re.M)


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    assert {"fused_add_rmsnorm", "fused_add_rmsnorm_quant_fp8",
            "fused_add_rmsnorm_quant_fp8_block", "qk_rmsnorm", "qk_rmsnorm_var",
            "fusednorm_e4m3_encode", "fusednorm_status_string", "fusednorm_last_error",
            "fusednorm_version", "sharded_rmsnorm", "sharded_rmsnorm_var",
            "fused_add_rmsnorm_quant_fp8_static", "fused_rs_epilogue", "ag_dual_rmsnorm"} <= names


def test_library_exports_exactly_the_declared_functions(lib):
    """The dynamic symbol table holds the header's functions and nothing else:
    no internal C++ helper, no compiler data symbol."""
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    declared = set(declared_functions())
    assert exported == declared, (sorted(exported - declared), sorted(declared - exported))
    for n in declared:
        assert getattr(lib, n) is not None


def test_every_declaration_carries_the_export_macro():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decls = re.findall(r"^(.*?)\b(\w+)\s*\([^;{]*\)\s*;", text, re.M)
    assert decls
    for prefix, name in decls:
        assert prefix.startswith("FUSEDNORM_API "), name


def test_version_and_status_strings(lib):
    v = int(re.search(r"#define FUSEDNORM_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.fusednorm_version() == v
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported input"),
                       (3, b"HIP runtime error"), (99, b"unknown status")]:
        assert lib.fusednorm_status_string(code) == text


A = 0x7F0000000000          # fake, 16-byte aligned device addresses, far apart
MB = 1 << 24


def addr(k, off=0):
    return ctypes.c_void_p(A + k * MB * 64 + off)


def parts(P, off=0):
    return (ctypes.c_void_p * P)(*[A + (10 + p) * MB * 64 + off for p in range(P)])


def call_norm(lib, P=2, T=4, H=64, eps=1e-6, res=None, w=None, norm=None, rout=None,
              partials=None):
    return lib.fused_add_rmsnorm(parts(P) if partials is None else partials, P,
                                 res or addr(1), w or addr(2), T, H, eps,
                                 addr(3) if norm is None else norm,
                                 addr(4) if rout is None else rout, None)


def last(lib):
    return lib.fusednorm_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(P=0), 1, "P = 0"),
    (dict(P=17), 1, "P = 17"),
    (dict(T=-1), 1, "T = -1"),
    (dict(H=0), 1, "H = 0"),
    (dict(eps=-1.0), 1, "eps"),
    (dict(eps=float("inf")), 1, "eps"),
    (dict(eps=float("nan")), 1, "eps"),
    (dict(H=12), 2, "multiple of 8"),
    (dict(H=16392), 2, "above 16384"),
    (dict(res=addr(1, 8)), 2, "residual_in not 16-byte aligned"),
    (dict(w=addr(2, 2)), 2, "weight not 16-byte aligned"),
    (dict(norm=addr(3, 4)), 2, "norm_out not 16-byte aligned"),
    (dict(partials=parts(2, 8)), 2, "partials[0] not 16-byte aligned"),
])
def test_norm_validation(lib, kw, code, msg):
    assert call_norm(lib, **kw) == code
    assert msg in last(lib)


def test_null_pointers(lib):
    null = ctypes.c_void_p(0)
    assert lib.fused_add_rmsnorm(None, 1, addr(1), addr(2), 4, 64, 1e-6, addr(3), addr(4),
                                 None) == 1
    pp = (ctypes.c_void_p * 2)(A + 10 * MB * 64, 0)
    assert call_norm(lib, partials=pp) == 1 and "partials[1] is NULL" in last(lib)
    assert lib.fused_add_rmsnorm(parts(1), 1, null, addr(2), 4, 64, 1e-6, addr(3), addr(4),
                                 None) == 1
    assert lib.fused_add_rmsnorm(parts(1), 1, addr(1), null, 4, 64, 1e-6, addr(3), addr(4),
                                 None) == 1
    assert lib.fused_add_rmsnorm(parts(1), 1, addr(1), addr(2), 4, 64, 1e-6, null, addr(4),
                                 None) == 1
    assert lib.fused_add_rmsnorm(parts(1), 1, addr(1), addr(2), 4, 64, 1e-6, addr(3), null,
                                 None) == 1


def test_overlaps(lib):
    T, H = 4, 64
    row = H * 2
    # residual_out partially overlapping residual_in
    assert call_norm(lib, T=T, H=H, rout=addr(1, 16)) == 2 and "overlaps" in last(lib)
    # norm_out overlapping a partial
    assert call_norm(lib, T=T, H=H, norm=ctypes.c_void_p(A + 10 * MB * 64 + row)) == 2
    # norm_out == residual_out
    assert call_norm(lib, T=T, H=H, norm=addr(4), rout=addr(4)) == 2
    # in-place residual is allowed: exactly the same buffer (T = 0: nothing launched)
    assert call_norm(lib, T=0, H=H, rout=addr(1)) == 0
    # norm_out equal to residual_in is not
    assert call_norm(lib, T=T, H=H, norm=addr(1)) == 2


def test_empty_batch_is_ok_and_clears_the_error(lib):
    assert call_norm(lib, P=0) == 1 and last(lib)
    assert call_norm(lib, T=0) == 0
    assert last(lib) == ""


def test_quant_validation(lib):
    f8 = lib.fused_add_rmsnorm_quant_fp8
    fb = lib.fused_add_rmsnorm_quant_fp8_block
    sc = ctypes.cast(addr(6), ctypes.c_void_p)
    assert f8(parts(2), 2, addr(1), addr(2), 0, 64, 1e-6, None, addr(4), addr(5), sc, None) == 0
    assert f8(parts(2), 2, addr(1), addr(2), 4, 64, 1e-6, None, addr(4), None, sc, None) == 1
    assert f8(parts(2), 2, addr(1), addr(2), 4, 64, 1e-6, None, addr(4), addr(5), None, None) == 1
    assert f8(parts(2), 2, addr(1), addr(2), 4, 64, 1e-6, None, addr(4), addr(5, 8), sc,
              None) == 2
    assert f8(parts(2), 2, addr(1), addr(2), 4, 64, 1e-6, None, addr(4), addr(5),
              ctypes.c_void_p(A + 6 * MB * 64 + 2), None) == 2
    # scale_out overlapping quant_out
    assert f8(parts(2), 2, addr(1), addr(2), 4, 64, 1e-6, None, addr(4), addr(5),
              ctypes.c_void_p(A + 5 * MB * 64 + 64), None) == 2
    assert fb(parts(2), 2, addr(1), addr(2), 4, 256, 1e-6, 64, None, addr(4), addr(5), sc,
              None) == 2 and "group_size" in last(lib)
    assert fb(parts(2), 2, addr(1), addr(2), 4, 192, 1e-6, 128, None, addr(4), addr(5), sc,
              None) == 2 and "multiple of 128" in last(lib)
    assert fb(parts(2), 2, addr(1), addr(2), 0, 256, 1e-6, 128, None, addr(4), addr(5), sc,
              None) == 0


def test_qk_validation(lib):
    qk = lib.qk_rmsnorm
    v = ctypes.cast(addr(5), ctypes.c_void_p)

    def call(T=4, stride=96, q=48, k=16, eps=1e-6, tp=1, var=None, qkv=None, qo=None):
        return qk(qkv or addr(1), T, stride, q, k, addr(2), addr(3), eps, tp, var,
                  qo or addr(6), addr(7), None)

    assert call(T=0) == 0
    assert call(tp=4) == 1 and "needs var_in" in last(lib)
    assert call(tp=0, var=v) == 1
    assert call(q=0) == 1
    assert call(q=44) == 2
    assert call(stride=100) == 2
    assert call(stride=56) == 2 and "row_stride" in last(lib)
    assert call(q=16384, k=8, stride=16400) == 2
    assert call(eps=-1.0) == 1
    assert call(qkv=addr(1, 4)) == 2
    assert call(var=ctypes.c_void_p(A + 5 * MB * 64 + 4), tp=2) == 2
    assert call(qo=addr(1, 64)) == 2 and "overlaps" in last(lib)
    assert call(T=0, var=v, tp=4) == 0
    qv = lib.qk_rmsnorm_var
    assert qv(addr(1), 4, 96, 48, 16, None, None) == 1
    assert qv(addr(1), 4, 96, 48, 16, ctypes.cast(addr(1), ctypes.c_void_p), None) == 2
    assert qv(addr(1), 0, 96, 48, 16, ctypes.cast(addr(5), ctypes.c_void_p), None) == 0


def test_e4m3_encode_validation(lib):
    enc = lib.fusednorm_e4m3_encode
    assert enc(None, addr(2), 8, None) == 1
    assert enc(None, None, 0, None) == 0
    assert enc(addr(1), addr(2), -1, None) == 1
    assert enc(addr(1, 4), addr(2), 8, None) == 2
    assert enc(addr(1), addr(1, 16), 64, None) == 2
    assert enc(addr(1), addr(2), 0, None) == 0


def test_binding_fails_loudly_without_the_library(tmp_path):
    # A copy of the binding module next to no library must refuse to import.
    src = os.path.join(ROOT, "residual_add_rmsnorm_amd", "fusednorm.py")
    pkg = tmp_path / "lonely_pkg"
    pkg.mkdir()
    (pkg / "__init__.py").write_text("")
    (pkg / "fusednorm.py").write_text(open(src).read())
    r = subprocess.run([sys.executable, "-c", "import lonely_pkg.fusednorm"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0
    assert "FusedNormLibraryMissing" in r.stderr


def test_sharded_validation(lib):
    sr, sv = lib.sharded_rmsnorm, lib.sharded_rmsnorm_var
    v = ctypes.cast(addr(5), ctypes.c_void_p)

    def call(T=4, stride=64, H=64, eps=1e-6, tp=1, var=None, x=None, out=None):
        return sr(x or addr(1), T, stride, H, addr(2), eps, tp, var, out or addr(6), None)

    assert call(T=0) == 0
    assert call(tp=2) == 1 and "needs var_in" in last(lib)
    assert call(H=0) == 1
    assert call(H=60, stride=64) == 2
    assert call(H=72, stride=64) == 2 and "row_stride" in last(lib)
    assert call(H=16392, stride=16392) == 2
    assert call(eps=float("nan")) == 1
    assert call(x=addr(1, 8)) == 2
    assert call(out=addr(1, 32)) == 2 and "overlaps" in last(lib)
    assert call(var=ctypes.c_void_p(A + 5 * MB * 64 + 2), tp=2) == 2
    assert call(T=0, var=v, tp=4) == 0
    assert sv(addr(1), 4, 64, 64, None, None) == 1
    assert sv(addr(1), 4, 64, 64, ctypes.cast(addr(1), ctypes.c_void_p), None) == 2
    assert sv(addr(1), 0, 64, 64, None, None) == 0


def test_static_quant_validation(lib):
    fs = lib.fused_add_rmsnorm_quant_fp8_static
    sc = ctypes.cast(addr(6), ctypes.c_void_p)
    assert fs(parts(2), 2, addr(1), addr(2), 0, 64, 1e-6, sc, None, addr(4), addr(5), None) == 0
    assert fs(parts(2), 2, addr(1), addr(2), 4, 64, 1e-6, None, None, addr(4), addr(5), None) == 1
    assert "scale_factor" in last(lib)
    assert fs(parts(2), 2, addr(1), addr(2), 4, 64, 1e-6, sc, None, addr(4), None, None) == 1
    assert fs(parts(2), 2, addr(1), addr(2), 4, 64, 1e-6, ctypes.c_void_p(A + 6 * MB * 64 + 2),
              None, addr(4), addr(5), None) == 2
    # the scale may not sit inside an output
    assert fs(parts(2), 2, addr(1), addr(2), 4, 64, 1e-6, ctypes.c_void_p(A + 5 * MB * 64 + 64),
              None, addr(4), addr(5), None) == 2


def test_rs_epilogue_validation(lib):
    rs = lib.fused_rs_epilogue
    sc = ctypes.cast(addr(6), ctypes.c_void_p)

    def call(pattern, add=None, P=2, T=4, off=0, norm=None, q=None, scale=None, factor=None):
        return rs(pattern, parts(P), P, off, add, addr(1), addr(2), T, 256, 1e-6, factor, norm,
                  addr(4), q, scale, None)

    for pattern in (0, 3, 5):
        assert call(pattern) == 2 and "not implemented" in last(lib)
    assert call(9) == 1 and call(-1) == 1
    assert call(8) == 1 and "needs add_in" in last(lib)
    assert call(1, add=addr(7)) == 1 and "takes no add_in" in last(lib)
    assert call(7, add=addr(7), P=16) == 1 and "no room for add_in" in last(lib)
    assert call(1, off=-1) == 1
    assert call(2, q=addr(5), norm=addr(3), factor=sc) == 1          # 2 writes no norm_out
    assert call(4, q=addr(5), factor=sc) == 1                        # 4 needs norm_out
    assert call(2, q=addr(5)) == 1 and "scale_factor" in last(lib)
    assert call(6, q=addr(5)) == 1 and "scale_out" in last(lib)
    assert call(7, add=addr(4), q=addr(5), scale=sc) == 2            # add_in inside residual_out
    assert "add_in" in last(lib)
    assert call(8, add=addr(7), T=0) == 0


def test_ag_dual_validation(lib):
    ag = lib.ag_dual_rmsnorm
    sc = ctypes.cast(addr(6), ctypes.c_void_p)

    def call(pattern=1, T=4, stride=336, q=256, kv=64, xe=1e-6, ye=1e-6, rows=None, x="d",
             y="d", codes=None, scale=None):
        x = addr(3) if x == "d" else x
        y = addr(4) if y == "d" else y
        return ag(pattern, rows or addr(1), T, stride, q, kv, addr(2), addr(7), xe, ye, x, y,
                  codes, scale, None)

    assert call(T=0) == 0 and call(2, T=0) == 0
    assert call(0) == 2 and "not implemented" in last(lib)
    assert call(3) == 1 and call(-1) == 1
    assert call(q=0) == 1 and call(kv=0) == 1
    assert call(T=-1) == 1
    assert call(ye=-1.0) == 1 and call(xe=float("inf")) == 1
    assert call(q=252) == 2
    assert call(2, q=264, stride=336, codes=addr(5), scale=sc) == 2 and "128" in last(lib)
    assert call(stride=312) == 2 and "row_stride" in last(lib)
    assert call(q=16384, kv=8, stride=16392) == 2
    assert call(x=None) == 1 and "x_norm_out" in last(lib)
    assert call(y=None) == 1
    assert call(codes=addr(5), scale=sc) == 1 and "pattern 1" in last(lib)
    assert call(2, codes=addr(5)) == 1 and "scale_out" in last(lib)
    assert call(2, scale=sc) == 1
    assert call(rows=addr(1, 8)) == 2
    assert call(2, x=None, codes=addr(5, 4), scale=sc) == 2
    assert call(y=addr(1, 64)) == 2 and "overlaps" in last(lib)
    assert call(2, x=None, codes=addr(4, 64), scale=sc) == 2 and "overlaps" in last(lib)


def test_stream_aid_validation(lib):
    rd, cp = lib.fusednorm_stream_read, lib.fusednorm_stream_copy
    K16 = 16 * 1024
    assert rd(None, K16, addr(2), None) == 1
    assert rd(addr(1), 0, addr(2), None) == 1
    assert rd(addr(1), K16 + 16, addr(2), None) == 2
    assert rd(addr(1, 8), K16, addr(2), None) == 2
    assert cp(addr(1), None, K16, None) == 1
    assert cp(addr(1), addr(1, K16 // 2), K16, None) == 2      # overlapping
    assert cp(addr(1), addr(2, 4), K16, None) == 2


def test_stream_mix_validation(lib):
    mix = lib.fusednorm_stream_mix
    vp, i64 = ctypes.c_void_p, ctypes.c_int64

    def call(srcs=(1, 2), dsts=(5,), widths=(1024,), row=1024, stride=None, rows=8):
        sp = (vp * max(len(srcs), 1))(*[None if s is None else addr(s) for s in srcs])
        dp = (vp * max(len(dsts), 1))(*[None if d is None else addr(d) for d in dsts])
        wb = (i64 * max(len(widths), 1))(*widths)
        return mix(sp, len(srcs), row, row if stride is None else stride, dp, wb, len(dsts),
                   rows, None)

    assert call(rows=0) == 0                                  # nothing to move
    assert call(srcs=()) == 1
    assert call(srcs=tuple(range(1, 18))) == 1                # 17 sources
    assert call(dsts=(), widths=()) == 1
    assert call(dsts=(5, 6, 7, 8, 9), widths=(16,) * 5) == 1
    assert call(srcs=(1, None)) == 1
    assert call(dsts=(None,)) == 1
    assert call(rows=-1) == 1
    assert call(widths=(0,)) == 1
    assert call(row=1000, widths=(992,)) == 2                 # not a multiple of 16
    assert call(row=32768 + 16, widths=(16,)) == 2            # row above 32 KiB
    assert call(stride=512) == 2                              # stride below the row
    assert call(widths=(2048,)) == 2                          # destination wider than the row
    assert call(dsts=(1,)) == 2                               # destination over a source
    assert call(dsts=(5, 5), widths=(1024, 1024)) == 2        # destinations overlap


def test_c_client_compiles_as_c_and_runs(lib, tmp_path):
    """The header is plain C and the library links from C; the client makes only
    calls that return before any HIP work."""
    from residual_add_rmsnorm_amd import _build
    exe = tmp_path / "abi_check"
    src = os.path.join(ROOT, "residual_add_rmsnorm_amd", "examples", "abi_check.c")
    libdir = os.path.dirname(_build.LIB)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I",
                    os.path.join(ROOT, "include"), src, "-L", libdir, "-lfusednorm",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
