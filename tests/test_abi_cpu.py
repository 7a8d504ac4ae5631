"""C-ABI checks that run without a GPU.

* the shared library loads and exports every function include/mxfp4spec.h declares;
* host-detected errors come back before any HIP call (NULL, shape, alignment,
  workspace), so they are testable here with fake, never-dereferenced pointers;
* with valid arguments and no usable device the library answers MXS_ERR_DEVICE;
* the Python binding fails loudly when the library is missing (no fallback).
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import mx_fp4_weight_amd as mxs
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mxfp4spec.h")
P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text)
    keep = [n for n in names if n.startswith(("mxs_", "mx_", "mxfp4_", "nvfp4_", "spec_accept", "spec_sampling"))]
    return sorted(set(keep))


def test_header_functions_exported():
    names = declared_functions()
    assert set(names) == set(mxs.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", mxs.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n


def test_status_strings_and_version():
    lib = mxs.get_lib()
    assert lib.mxs_abi_version() == 1
    for s in range(8):
        assert mxs.status_string(s).startswith("MXS_")
    assert mxs.status_string(99) == "unknown mxs_status"


def test_workspace_query():
    lib = mxs.get_lib()
    assert lib.spec_accept_workspace_bytes(0, 4, 1024) == 0
    assert lib.spec_accept_workspace_bytes(1, -1, 1024) == 0
    assert lib.spec_accept_workspace_bytes(1, 33, 1024) == 0
    assert lib.spec_accept_workspace_bytes(1, 4, 1) == 0
    a = lib.spec_accept_workspace_bytes(1, 4, 128256)
    b = lib.spec_accept_workspace_bytes(64, 4, 128256)
    assert 0 < a < b
    # per (row, chunk): fp32 max + fp64 sum + int32 flag; per (seq, chunk): two fp64 totals
    rows, chunks = 64 * 9, (128256 + 4095) // 4096
    assert b >= rows * chunks * 16 + 64 * chunks * 16


def _q(w=0x1000, n=4, k=64, codes=0x2000, scales=0x3000, flags=None):
    return mxs.get_lib().mxfp4_quantize(P(w) if w else None, n, k, P(codes) if codes else None,
                                        P(scales) if scales else None, P(flags) if flags else None, None)


def test_quantize_host_errors():
    assert _q(w=0) == mxs.MXS_ERR_NULL
    assert _q(codes=0) == mxs.MXS_ERR_NULL
    assert _q(scales=0) == mxs.MXS_ERR_NULL
    assert _q(k=48) == mxs.MXS_ERR_SHAPE
    assert _q(k=0) == mxs.MXS_ERR_SHAPE
    assert _q(n=0) == mxs.MXS_ERR_SHAPE
    assert _q(w=0x1004) == mxs.MXS_ERR_ALIGN
    assert _q(codes=0x2008) == mxs.MXS_ERR_ALIGN
    assert _q(flags=0x5002) == mxs.MXS_ERR_ALIGN
    assert _q(scales=0x3001) == mxs.MXS_ERR_DEVICE     # scales may have any alignment
    assert _q() == mxs.MXS_ERR_DEVICE                  # valid call, no GPU in this container


def _g(codes=0x1000, scales=0x2000, n=4, k=64, x=0x3000, m=5, y=0x4000):
    return mxs.get_lib().mxfp4_verify_gemm(P(codes) if codes else None, P(scales) if scales else None, n, k,
                                           P(x) if x else None, m, P(y) if y else None, None)


def test_gemm_host_errors():
    for kw in [dict(codes=0), dict(scales=0), dict(x=0), dict(y=0)]:
        assert _g(**kw) == mxs.MXS_ERR_NULL
    for kw in [dict(k=40), dict(k=16), dict(n=0), dict(m=0), dict(m=65537), dict(n=-3)]:
        assert _g(**kw) == mxs.MXS_ERR_SHAPE
    for kw in [dict(codes=0x1004), dict(x=0x3002), dict(y=0x4002)]:
        assert _g(**kw) == mxs.MXS_ERR_ALIGN
    assert _g(m=65536) == mxs.MXS_ERR_DEVICE
    assert _g() == mxs.MXS_ERR_DEVICE


def _a(t=0x1000, d=0x2000, tok=0x3000, u=0x4000, b=1, kd=4, v=1024, ot=0x5000, on=0x6000,
       ws=0x7000, wsb=None, flags=None):
    lib = mxs.get_lib()
    if wsb is None:
        wsb = lib.spec_accept_workspace_bytes(max(b, 1), max(kd, 0), max(v, 2))
    f = lambda a: P(a) if a else None
    return lib.spec_accept(f(t), f(d), f(tok), f(u), b, kd, v, f(ot), f(on), f(ws), wsb, f(flags), None)


def test_accept_host_errors():
    for kw in [dict(t=0), dict(d=0), dict(tok=0), dict(u=0), dict(ot=0), dict(on=0), dict(ws=0)]:
        assert _a(**kw) == mxs.MXS_ERR_NULL
    assert _a(d=0, tok=0, kd=0) == mxs.MXS_ERR_DEVICE   # kd = 0 needs no draft inputs
    for kw in [dict(b=0), dict(kd=-1), dict(kd=33), dict(v=1), dict(v=(1 << 26) + 1)]:
        assert _a(**kw) == mxs.MXS_ERR_SHAPE
    for kw in [dict(t=0x1002), dict(tok=0x3001), dict(ws=0x7008), dict(flags=0x8001)]:
        assert _a(**kw) == mxs.MXS_ERR_ALIGN
    need = mxs.get_lib().spec_accept_workspace_bytes(1, 4, 1024)
    assert _a(wsb=need - 1) == mxs.MXS_ERR_WORKSPACE
    assert _a(wsb=need) == mxs.MXS_ERR_DEVICE


def _na(t=0x1000, d=0x2000, tok=0x3000, u=0x4000, b=1, kd=4, v=1024, ot=0x5000, on=0x6000, flags=None):
    f = lambda a: P(a) if a else None
    return mxs.get_lib().spec_accept_noalloc(f(t), f(d), f(tok), f(u), b, kd, v, f(ot), f(on), f(flags), None)


def test_accept_noalloc_host_errors():
    for kw in [dict(t=0), dict(d=0), dict(tok=0), dict(u=0), dict(ot=0), dict(on=0)]:
        assert _na(**kw) == mxs.MXS_ERR_NULL
    assert _na(d=0, tok=0, kd=0) == mxs.MXS_ERR_DEVICE
    for kw in [dict(b=0), dict(kd=-1), dict(kd=33), dict(v=1), dict(v=(1 << 26) + 1)]:
        assert _na(**kw) == mxs.MXS_ERR_SHAPE
    for kw in [dict(t=0x1002), dict(tok=0x3001), dict(ot=0x5002), dict(flags=0x8001)]:
        assert _na(**kw) == mxs.MXS_ERR_ALIGN
    # the built-in workspace bounds the size: past it the call is refused before any HIP call
    lib = mxs.get_lib()
    assert lib.spec_accept_workspace_bytes(64, 4, 128256) <= mxs.NOALLOC_SCRATCH_BYTES
    assert _na(b=64, kd=4, v=128256) == mxs.MXS_ERR_DEVICE
    big = (4096, 8, 131072)
    assert lib.spec_accept_workspace_bytes(*big) > mxs.NOALLOC_SCRATCH_BYTES
    assert _na(b=big[0], kd=big[1], v=big[2]) == mxs.MXS_ERR_WORKSPACE


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MXS_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mxs.NOALLOC_SCRATCH_BYTES


def test_tree_host_errors():
    lib = mxs.get_lib()
    f = lambda a: P(a) if a else None
    arr = lambda ps: (ctypes.c_int32 * max(1, len(ps)))(*ps)
    par = [-1, -1, 0, 0, 1]
    need = lib.spec_accept_tree_workspace_bytes(arr(par), len(par), 2, 1024)
    assert need > 0
    assert lib.spec_accept_tree_workspace_bytes(arr([0]), 1, 2, 1024) == 0          # a node its own parent
    assert lib.spec_accept_tree_workspace_bytes(arr([-1] * 17), 17, 2, 1024) == 0   # 17 children
    assert lib.spec_accept_tree_workspace_bytes(arr(par), len(par), 0, 1024) == 0

    def call(t=0x1000, d=0x2000, ps=par, nn=None, tok=0x3000, u=0x4000, b=2, v=1024, ot=0x5000, on=0x6000,
             onum=0x7000, ws=0x8000, wsb=None, fl=None):
        nn = len(ps) if nn is None else nn
        wsb = need if wsb is None else wsb
        return lib.spec_accept_tree(f(t), f(d), arr(ps), nn, f(tok), f(u), b, v, f(ot), f(on), f(onum), f(ws), wsb,
                                    f(fl), None)
    for a in [dict(t=0), dict(d=0), dict(tok=0), dict(u=0), dict(ot=0), dict(on=0), dict(onum=0), dict(ws=0)]:
        assert call(**a) == mxs.MXS_ERR_NULL
    assert call(ps=[], nn=0, tok=0, on=0, wsb=lib.spec_accept_tree_workspace_bytes(arr([]), 0, 2, 1024)) == \
        mxs.MXS_ERR_DEVICE
    for a in [dict(b=0), dict(v=1), dict(nn=65, ps=[-1] * 65)]:
        assert call(**a) == mxs.MXS_ERR_SHAPE
    for a in [dict(ps=[-1, 1]), dict(ps=[-1] * 17), dict(ps=[-2])]:
        assert call(**a) == mxs.MXS_ERR_VALUE
    for a in [dict(t=0x1002), dict(tok=0x3001), dict(ws=0x8008), dict(fl=0x9001)]:
        assert call(**a) == mxs.MXS_ERR_ALIGN
    assert call(wsb=need - 1) == mxs.MXS_ERR_WORKSPACE
    assert call() == mxs.MXS_ERR_DEVICE


def test_kv_attention_host_errors():
    lib = mxs.get_lib()
    f = lambda a: P(a) if a else None
    need = lib.mxfp4_kv_attention_workspace_bytes(1, 5, 32, 8, 4096)
    assert need > 0 and lib.mxfp4_kv_attention_workspace_bytes(1, 5, 32, 7, 4096) == 0

    def call(q=0x1000, kc=0x2000, ks=0x3000, vc=0x4000, vs=0x5000, cl=0x6000, b=1, t=5, hq=32, hkv=8, d=128,
             cap=4096, ml=4096, masks=None, scale=0.088, out=0x7000, ws=0x8000, wsb=None, fl=None):
        m = (ctypes.c_uint64 * 5)(*(masks or mxs.chain_masks(5)))
        return lib.mxfp4_kv_attention(f(q), f(kc), f(ks), f(vc), f(vs), f(cl), b, t, hq, hkv, d, cap, ml, m, scale,
                                      f(out), f(ws), need if wsb is None else wsb, f(fl), None)
    for a in [dict(q=0), dict(kc=0), dict(vs=0), dict(cl=0), dict(out=0), dict(ws=0)]:
        assert call(**a) == mxs.MXS_ERR_NULL
    for a in [dict(d=64), dict(hkv=7), dict(t=0), dict(ml=4097), dict(ml=4), dict(hq=64, hkv=2)]:
        assert call(**a) == mxs.MXS_ERR_SHAPE
    for a in [dict(scale=0.0), dict(scale=float("inf")), dict(masks=[1, 3, 7, 15, 32])]:
        assert call(**a) == mxs.MXS_ERR_VALUE
    for a in [dict(q=0x1008), dict(kc=0x2004), dict(out=0x7002), dict(ws=0x8008)]:
        assert call(**a) == mxs.MXS_ERR_ALIGN
    assert call(wsb=need - 1) == mxs.MXS_ERR_WORKSPACE
    assert call() == mxs.MXS_ERR_DEVICE
    # T = 64 (every bit of a mask may be set): the masks are valid, the call reaches the device
    # check; one bit past t is refused for t < 64
    need64 = lib.mxfp4_kv_attention_workspace_bytes(1, 64, 1, 1, 4096)
    m64 = (ctypes.c_uint64 * 64)(*mxs.chain_masks(64))
    assert m64[63] == (1 << 64) - 1
    assert lib.mxfp4_kv_attention(f(0x1000), f(0x2000), f(0x3000), f(0x4000), f(0x5000), f(0x6000), 1, 64, 1, 1,
                                  128, 4096, 4096, m64, 0.088, f(0x7000), f(0x8000), need64, None,
                                  None) == mxs.MXS_ERR_DEVICE
    m63 = (ctypes.c_uint64 * 63)(*(mxs.chain_masks(62) + [1 << 63]))
    assert lib.mxfp4_kv_attention(f(0x1000), f(0x2000), f(0x3000), f(0x4000), f(0x5000), f(0x6000), 1, 63, 1, 1,
                                  128, 4096, 4096, m63, 0.088, f(0x7000), f(0x8000), need64, None,
                                  None) == mxs.MXS_ERR_VALUE


def test_kv_slot_flag_is_the_token_range_bit():
    from oracle import kvcache
    assert kvcache.FLAG_SLOT_RANGE == mxs.FLAG_TOKEN_RANGE and kvcache.FLAG_NONFINITE == mxs.FLAG_NONFINITE


def test_kv_append_host_errors():
    lib = mxs.get_lib()
    f = lambda a: P(a) if a else None
    kv = lambda kv=0x1000, t=4, h=8, d=128, sl=0x2000, cap=64, c=0x3000, s=0x4000, fl=None: lib.mxfp4_kv_append(
        f(kv), t, h, d, f(sl), cap, f(c), f(s), f(fl), None)
    for a in [dict(kv=0), dict(sl=0), dict(c=0), dict(s=0)]:
        assert kv(**a) == mxs.MXS_ERR_NULL
    for a in [dict(t=0), dict(h=0), dict(d=16), dict(d=48), dict(cap=0)]:
        assert kv(**a) == mxs.MXS_ERR_SHAPE
    for a in [dict(kv=0x1008), dict(sl=0x2002), dict(c=0x3002), dict(fl=0x5001)]:
        assert kv(**a) == mxs.MXS_ERR_ALIGN
    assert kv(s=0x4001) == mxs.MXS_ERR_DEVICE   # scales: any alignment
    assert kv() == mxs.MXS_ERR_DEVICE


def test_stream_read_host_errors():
    lib = mxs.get_lib()
    f = lambda a: P(a) if a else None
    sr = lambda buf=0x1000, nb=1 << 20, sink=0x2000: lib.mxs_stream_read(f(buf), nb, f(sink), None)
    assert sr(buf=0) == mxs.MXS_ERR_NULL and sr(sink=0) == mxs.MXS_ERR_NULL
    assert sr(nb=0) == mxs.MXS_ERR_SHAPE and sr(nb=8) == mxs.MXS_ERR_SHAPE and sr(nb=(1 << 20) + 4) == mxs.MXS_ERR_SHAPE
    assert sr(buf=0x1008) == mxs.MXS_ERR_ALIGN and sr(sink=0x2002) == mxs.MXS_ERR_ALIGN
    assert sr() == mxs.MXS_ERR_DEVICE


def test_binding_fails_loudly_without_library(tmp_path):
    code = (
        "import mx_fp4_weight_amd as m\n"
        f"m.LIB_PATH = {str(tmp_path / 'missing.so')!r}\n"
        "m._LIB = None\n"
        "try:\n"
        "    m.get_lib()\n"
        "except ImportError as e:\n"
        "    print('IMPORT_ERROR', 'no fallback' in str(e))\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "IMPORT_ERROR True" in r.stdout, r.stderr


def test_product_never_imports_oracle():
    """The product package and its sources name neither the oracle nor the input generator."""
    pkg = os.path.join(ROOT, "mx_fp4_weight_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "import synth" not in text and "from synth" not in text, fn


def test_grouped_gemm_host_errors():
    lib = mxs.get_lib()
    arr = (mxs.GemmProblem * 3)()
    for i in range(3):
        arr[i] = mxs.GemmProblem(0x1000 * (i + 1), 0x20000, 0x30000, 0x40000, 64)
    assert lib.mxfp4_verify_gemm_grouped(None, 3, 64, 5, None) == mxs.MXS_ERR_NULL
    assert lib.mxfp4_verify_gemm_grouped(arr, 0, 64, 5, None) == mxs.MXS_ERR_SHAPE
    assert lib.mxfp4_verify_gemm_grouped(arr, 3, 48, 5, None) == mxs.MXS_ERR_SHAPE
    assert lib.mxfp4_verify_gemm_grouped(arr, 3, 64, 0, None) == mxs.MXS_ERR_SHAPE
    assert lib.mxfp4_verify_gemm_grouped(arr, 3, 64, 5, None) == mxs.MXS_ERR_DEVICE
    arr[1].x = 0
    assert lib.mxfp4_verify_gemm_grouped(arr, 3, 64, 5, None) == mxs.MXS_ERR_NULL
    arr[1].x = 0x30008
    assert lib.mxfp4_verify_gemm_grouped(arr, 3, 64, 5, None) == mxs.MXS_ERR_ALIGN
    arr[1].x = 0x30000
    arr[2].n = 0
    assert lib.mxfp4_verify_gemm_grouped(arr, 3, 64, 5, None) == mxs.MXS_ERR_SHAPE


def _as(t=0x1000, d=0x2000, tok=0x3000, u=0x4000, b=1, kd=4, v=1024, tau=1.0, k=0, p=1.0, mask=None,
        ot=0x5000, on=0x6000, ws=0x7000, wsb=None, flags=None):
    lib = mxs.get_lib()
    if wsb is None:
        wsb = lib.spec_accept_sampled_workspace_bytes(max(b, 1), max(kd, 0), max(v, 2))
    f = lambda a: P(a) if a else None
    return lib.spec_accept_sampled(f(t), f(d), f(tok), f(u), b, kd, v, tau, k, p, f(mask), f(ot), f(on),
                                   f(ws), wsb, f(flags), None)


def test_sampled_host_errors():
    lib = mxs.get_lib()
    plain = lib.spec_accept_workspace_bytes(2, 4, 128256)
    sampled = lib.spec_accept_sampled_workspace_bytes(2, 4, 128256)
    # per logit row: a 4096-bucket count + mass histogram and an 8192-key candidate list
    assert sampled >= plain + 2 * 9 * (4096 * 12 + 8192 * 4)
    assert lib.spec_accept_sampled_workspace_bytes(0, 4, 1024) == 0
    for kw in [dict(t=0), dict(u=0), dict(ot=0), dict(on=0), dict(ws=0), dict(d=0), dict(tok=0)]:
        assert _as(**kw) == mxs.MXS_ERR_NULL
    for kw in [dict(b=0), dict(kd=33), dict(v=1)]:
        assert _as(**kw) == mxs.MXS_ERR_SHAPE
    for kw in [dict(tau=0.0), dict(tau=-1.0), dict(tau=float("inf")), dict(tau=float("nan")),
               dict(k=-1), dict(p=0.0), dict(p=1.5), dict(p=float("nan"))]:
        assert _as(**kw) == mxs.MXS_ERR_VALUE, kw
    assert _as(mask=0x8002) == mxs.MXS_ERR_ALIGN
    need = lib.spec_accept_sampled_workspace_bytes(1, 4, 1024)
    assert _as(wsb=need - 1) == mxs.MXS_ERR_WORKSPACE
    assert _as(wsb=need, tau=0.7, k=50, p=0.9, mask=0x8000) == mxs.MXS_ERR_DEVICE


def _th(z=0x1000, rows=3, v=1024, tau=1.0, k=50, p=0.9, mask=None, out=0x2000, ws=0x3000, wsb=None):
    lib = mxs.get_lib()
    if wsb is None:
        wsb = lib.spec_sampling_thresholds_workspace_bytes(max(rows, 1), max(v, 2))
    f = lambda a: P(a) if a else None
    return lib.spec_sampling_thresholds(f(z), rows, v, tau, k, p, f(mask), f(out), f(ws), wsb, None)


def test_sampling_thresholds_host_errors():
    lib = mxs.get_lib()
    need = lib.spec_sampling_thresholds_workspace_bytes(3, 1024)
    assert need >= 3 * (4096 * 12 + 8192 * 4)
    assert lib.spec_sampling_thresholds_workspace_bytes(0, 1024) == 0
    assert lib.spec_sampling_thresholds_workspace_bytes(3, 1) == 0
    assert lib.spec_sampling_thresholds_workspace_bytes((1 << 22) + 1, 1024) == 0
    for kw in [dict(z=0), dict(out=0), dict(ws=0)]:
        assert _th(**kw) == mxs.MXS_ERR_NULL, kw
    for kw in [dict(rows=0), dict(v=1), dict(v=(1 << 26) + 1)]:
        assert _th(**kw) == mxs.MXS_ERR_SHAPE, kw
    for kw in [dict(tau=0.0), dict(tau=float("inf")), dict(tau=float("nan")), dict(k=-1), dict(p=0.0),
               dict(p=1.01), dict(p=float("nan"))]:
        assert _th(**kw) == mxs.MXS_ERR_VALUE, kw
    for kw in [dict(z=0x1002), dict(out=0x2001), dict(ws=0x3008), dict(mask=0x4002)]:
        assert _th(**kw) == mxs.MXS_ERR_ALIGN, kw
    assert _th(wsb=need - 1) == mxs.MXS_ERR_WORKSPACE
    assert _th(wsb=need, mask=0x4000) == mxs.MXS_ERR_DEVICE
    assert _th(k=0, p=1.0) == mxs.MXS_ERR_DEVICE   # both off: still a device call (zero fill)


def _nq(w=0x1000, n=4, k=64, codes=0x2000, scales=0x3000, g=0x4000, flags=None):
    f = lambda a: P(a) if a else None
    return mxs.get_lib().nvfp4_quantize(f(w), n, k, f(codes), f(scales), f(g), f(flags), None)


def test_nvfp4_quantize_host_errors():
    for kw in [dict(w=0), dict(codes=0), dict(scales=0), dict(g=0)]:
        assert _nq(**kw) == mxs.MXS_ERR_NULL
    for kw in [dict(k=24), dict(k=0), dict(n=0), dict(k=8)]:
        assert _nq(**kw) == mxs.MXS_ERR_SHAPE
    for kw in [dict(w=0x1008), dict(codes=0x2001), dict(g=0x4002), dict(flags=0x5001)]:
        assert _nq(**kw) == mxs.MXS_ERR_ALIGN
    assert _nq(scales=0x3001, k=16) == mxs.MXS_ERR_DEVICE   # scales may have any alignment
    assert _nq() == mxs.MXS_ERR_DEVICE


def _ng(codes=0x1000, scales=0x2000, g=0x3000, n=4, k=512, x=0x4000, m=5, y=0x5000):
    f = lambda a: P(a) if a else None
    return mxs.get_lib().nvfp4_verify_gemm(f(codes), f(scales), f(g), n, k, f(x), m, f(y), None)


def test_nvfp4_gemm_host_errors():
    for kw in [dict(codes=0), dict(scales=0), dict(g=0), dict(x=0), dict(y=0)]:
        assert _ng(**kw) == mxs.MXS_ERR_NULL
    for kw in [dict(k=256), dict(k=768), dict(k=0), dict(n=0), dict(m=0), dict(m=65537)]:
        assert _ng(**kw) == mxs.MXS_ERR_SHAPE
    for kw in [dict(codes=0x1008), dict(scales=0x2004), dict(g=0x3002), dict(x=0x4008), dict(y=0x5002)]:
        assert _ng(**kw) == mxs.MXS_ERR_ALIGN
    assert _ng(m=65536, k=1024) == mxs.MXS_ERR_DEVICE
    assert _ng() == mxs.MXS_ERR_DEVICE


def _qa(x=0x1000, m=4, k=64, fmt=0, codes=0x2000, scales=0x3000, flags=None):
    f = lambda a: P(a) if a else None
    return mxs.get_lib().mx_quantize_act(f(x), m, k, fmt, f(codes), f(scales), f(flags), None)


def test_act_quantize_host_errors():
    for kw in [dict(x=0), dict(codes=0), dict(scales=0)]:
        assert _qa(**kw) == mxs.MXS_ERR_NULL
    for kw in [dict(fmt=1), dict(fmt=2), dict(fmt=-1), dict(fmt=8)]:
        assert _qa(**kw) == mxs.MXS_ERR_VALUE
    for kw in [dict(k=48), dict(k=16), dict(m=0), dict(k=0)]:
        assert _qa(**kw) == mxs.MXS_ERR_SHAPE
    for kw in [dict(x=0x1008), dict(codes=0x2004), dict(codes=0x2002, fmt=4), dict(flags=0x5002)]:
        assert _qa(**kw) == mxs.MXS_ERR_ALIGN
    assert _qa(codes=0x2004, fmt=4) == mxs.MXS_ERR_DEVICE
    assert _qa(scales=0x3001) == mxs.MXS_ERR_DEVICE


def _ga(codes=0x1000, scales=0x2000, n=4, k=256, ac=0x3000, asc=0x4000, fmt=0, m=5, y=0x5000):
    f = lambda a: P(a) if a else None
    return mxs.get_lib().mx_verify_gemm_act(f(codes), f(scales), n, k, f(ac), f(asc), fmt, m, f(y), None)


def test_act_gemm_host_errors():
    for kw in [dict(codes=0), dict(scales=0), dict(ac=0), dict(asc=0), dict(y=0)]:
        assert _ga(**kw) == mxs.MXS_ERR_NULL
    assert _ga(fmt=3) == mxs.MXS_ERR_VALUE
    for kw in [dict(k=96), dict(k=64), dict(n=0), dict(m=0), dict(m=65537), dict(k=(1 << 24) + 128)]:
        assert _ga(**kw) == mxs.MXS_ERR_SHAPE
    for kw in [dict(codes=0x1008), dict(ac=0x3004), dict(y=0x5002), dict(scales=0x2001), dict(asc=0x4002)]:
        assert _ga(**kw) == mxs.MXS_ERR_ALIGN
    assert _ga(scales=0x2004, asc=0x400C, fmt=4) == mxs.MXS_ERR_DEVICE
    assert _ga() == mxs.MXS_ERR_DEVICE


def test_nvfp4_grouped_host_errors():
    lib = mxs.get_lib()
    arr = (mxs.NvProblem * 2)()
    for i in range(2):
        arr[i] = mxs.NvProblem(0x10000 * (i + 1), 0x200000, 0x300000, 0x400000, 0x500000, 64)
    assert lib.nvfp4_verify_gemm_grouped(None, 2, 512, 5, None) == mxs.MXS_ERR_NULL
    assert lib.nvfp4_verify_gemm_grouped(arr, 0, 512, 5, None) == mxs.MXS_ERR_SHAPE
    assert lib.nvfp4_verify_gemm_grouped(arr, 2, 256, 5, None) == mxs.MXS_ERR_SHAPE
    assert lib.nvfp4_verify_gemm_grouped(arr, 2, 512, 0, None) == mxs.MXS_ERR_SHAPE
    assert lib.nvfp4_verify_gemm_grouped(arr, 2, 512, 5, None) == mxs.MXS_ERR_DEVICE
    arr[1].global_scale = 0
    assert lib.nvfp4_verify_gemm_grouped(arr, 2, 512, 5, None) == mxs.MXS_ERR_NULL
    arr[1].global_scale = 0x300002
    assert lib.nvfp4_verify_gemm_grouped(arr, 2, 512, 5, None) == mxs.MXS_ERR_ALIGN
    arr[1].global_scale = 0x300000
    arr[0].scales = 0x200008
    assert lib.nvfp4_verify_gemm_grouped(arr, 2, 512, 5, None) == mxs.MXS_ERR_ALIGN


def test_tiled_host_errors():
    """mxfp4_tile_codes / mx_verify_gemm_act_tiled refuse malformed calls before any HIP call."""
    lib = mxs.get_lib()
    assert lib.mxfp4_tiled_bytes(17, 256) == 32 * 128
    assert lib.mxfp4_tiled_bytes(16, 256) == 16 * 128
    assert lib.mxfp4_tiled_bytes(16, 192) == 0 and lib.mxfp4_tiled_bytes(0, 256) == 0
    a, b = P(0x100000), P(0x200000)
    assert lib.mxfp4_tile_codes(None, 16, 256, b, None) == mxs.MXS_ERR_NULL
    assert lib.mxfp4_tile_codes(a, 16, 192, b, None) == mxs.MXS_ERR_SHAPE
    assert lib.mxfp4_tile_codes(a, 0, 256, b, None) == mxs.MXS_ERR_SHAPE
    assert lib.mxfp4_tile_codes(P(0x100008), 16, 256, b, None) == mxs.MXS_ERR_ALIGN
    assert lib.mxfp4_tile_codes(a, 16, 256, b, None) == mxs.MXS_ERR_DEVICE
    assert lib.mxfp4_tiled_scale_bytes(129, 640) == 2 * 2 * 2048
    assert lib.mxfp4_tiled_scale_bytes(128, 192) == 0
    assert lib.mxfp4_tile_scales(None, 16, 256, b, None) == mxs.MXS_ERR_NULL
    assert lib.mxfp4_tile_scales(a, 16, 192, b, None) == mxs.MXS_ERR_SHAPE
    assert lib.mxfp4_tile_scales(P(0x100002), 16, 256, b, None) == mxs.MXS_ERR_ALIGN
    assert lib.mxfp4_tile_scales(a, 16, 256, P(0x200004), None) == mxs.MXS_ERR_ALIGN
    assert lib.mxfp4_tile_scales(a, 16, 256, b, None) == mxs.MXS_ERR_DEVICE
    call = lambda tc=0x100000, ts=0x300000, fmt=0, n=64, k=256, m=5: lib.mx_verify_gemm_act_tiled(
        P(tc) if tc else None, P(ts), n, k, P(0x400000), P(0x500000), fmt, m, P(0x600000), None)
    assert call(ts=0x300004) == mxs.MXS_ERR_ALIGN
    assert call(tc=0) == mxs.MXS_ERR_NULL
    assert call(fmt=3) == mxs.MXS_ERR_VALUE
    assert call(k=192) == mxs.MXS_ERR_SHAPE and call(m=0) == mxs.MXS_ERR_SHAPE and call(n=0) == mxs.MXS_ERR_SHAPE
    assert call(tc=0x100004) == mxs.MXS_ERR_ALIGN
    assert call() == mxs.MXS_ERR_DEVICE


def test_verify_gemm_tiled_host_errors():
    """mxfp4_verify_gemm_tiled refuses malformed calls before any HIP call."""
    lib = mxs.get_lib()
    call = lambda tc=0x100000, ts=0x300000, x=0x400000, n=64, k=256, m=40: lib.mxfp4_verify_gemm_tiled(
        P(tc) if tc else None, P(ts) if ts else None, n, k, P(x), m, P(0x600000), None)
    assert call(tc=0) == mxs.MXS_ERR_NULL and call(ts=0) == mxs.MXS_ERR_NULL
    assert call(k=192) == mxs.MXS_ERR_SHAPE and call(k=64) == mxs.MXS_ERR_SHAPE
    assert call(k=(1 << 23) + 128) == mxs.MXS_ERR_SHAPE
    assert call(m=0) == mxs.MXS_ERR_SHAPE and call(m=65537) == mxs.MXS_ERR_SHAPE and call(n=0) == mxs.MXS_ERR_SHAPE
    # launch grid beyond 32 bits of threads: 2^21 rows at m = 65536
    assert call(n=1 << 21, m=65536) == mxs.MXS_ERR_SHAPE
    assert call(tc=0x100004) == mxs.MXS_ERR_ALIGN and call(ts=0x300004) == mxs.MXS_ERR_ALIGN
    assert call(x=0x400008) == mxs.MXS_ERR_ALIGN
    assert call() == mxs.MXS_ERR_DEVICE
    assert call(n=1 << 20, m=65536) == mxs.MXS_ERR_DEVICE


def test_grouped_tiled_host_errors():
    """mxfp4_verify_gemm_grouped_tiled refuses malformed calls before any HIP call."""
    lib = mxs.get_lib()

    def call(count=2, k=512, m=5, **kw):
        arr = (mxs.GemmProblem * 2)()
        for i in range(2):
            arr[i] = mxs.GemmProblem(0x100000, 0x200000, 0x300000, 0x400000, 64)
        for name, v in kw.items():
            setattr(arr[1], name, v)
        return lib.mxfp4_verify_gemm_grouped_tiled(arr, count, k, m, None)
    assert lib.mxfp4_verify_gemm_grouped_tiled(None, 1, 512, 5, None) == mxs.MXS_ERR_NULL
    assert call(codes=0) == mxs.MXS_ERR_NULL and call(scales=0) == mxs.MXS_ERR_NULL
    assert call(count=0) == mxs.MXS_ERR_SHAPE and call(k=192) == mxs.MXS_ERR_SHAPE
    assert call(m=0) == mxs.MXS_ERR_SHAPE and call(n=0) == mxs.MXS_ERR_SHAPE
    assert call(n=1 << 21, m=65536) == mxs.MXS_ERR_SHAPE
    assert call(scales=0x200004) == mxs.MXS_ERR_ALIGN and call(codes=0x100008) == mxs.MXS_ERR_ALIGN
    assert call() == mxs.MXS_ERR_DEVICE and call(k=640) == mxs.MXS_ERR_DEVICE


def test_nvfp4_grouped_tiled_host_errors():
    """nvfp4_verify_gemm_grouped_tiled refuses malformed calls before any HIP call."""
    lib = mxs.get_lib()

    def call(count=2, k=512, m=5, **kw):
        arr = (mxs.NvProblem * 2)()
        for i in range(2):
            arr[i] = mxs.NvProblem(0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 64)
        for name, v in kw.items():
            setattr(arr[1], name, v)
        return lib.nvfp4_verify_gemm_grouped_tiled(arr, count, k, m, None)
    assert lib.nvfp4_verify_gemm_grouped_tiled(None, 1, 512, 5, None) == mxs.MXS_ERR_NULL
    assert call(codes=0) == mxs.MXS_ERR_NULL and call(global_scale=0) == mxs.MXS_ERR_NULL
    assert call(count=0) == mxs.MXS_ERR_SHAPE and call(k=640) == mxs.MXS_ERR_SHAPE
    assert call(m=0) == mxs.MXS_ERR_SHAPE and call(n=0) == mxs.MXS_ERR_SHAPE
    assert call(codes=0x100008) == mxs.MXS_ERR_ALIGN and call(scales=0x200004) == mxs.MXS_ERR_ALIGN
    assert call() == mxs.MXS_ERR_DEVICE
