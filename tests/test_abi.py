"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments before touching the GPU.  Pointer
arguments here are fake addresses that the library never dereferences,
because argument checks run on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from sparse_moe_layer_wave_amd import hy3moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hy3moe.h")

A = ctypes.c_void_p(0x10000)       # aligned fake device address
MIS = ctypes.c_void_p(0x10004)     # misaligned
NUL = None


@pytest.fixture(scope="module")
def L():
    return hy3moe.lib()


def test_every_declared_function_is_exported(L):
    decl = set(re.findall(r"\b(hy3moe_\w+)\s*\(", open(HEADER).read()))
    assert decl == set(hy3moe.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert len(L.hy3moe_status_string(code)) > 0
    assert L.hy3moe_status_string(-99) == b"unknown status"
    assert L.hy3moe_last_hip_error() == 0


def _ws(L, T, d=4096, E=192, k=8, F=1536, dt=0):
    n = ctypes.c_size_t(0)
    st = L.hy3moe_workspace_size(T, d, E, k, F, dt, ctypes.byref(n))
    return st, n.value


def test_workspace_size_monotone_and_checked(L):
    prev = -1
    for T in (1, 2, 63, 64, 65, 1000, 8192, 65536):
        for dt in (0, 1):
            st, n = _ws(L, T, dt=dt)
            assert st == 0 and n > 0
        st, n = _ws(L, T)
        assert n > prev
        prev = n
    # bf16 y [T*k, d] alone is part of the requirement
    assert _ws(L, 65536)[1] >= 65536 * 8 * 4096 * 2
    assert _ws(L, 8, dt=2)[0] == hy3moe.ERR_UNSUPPORTED
    assert L.hy3moe_workspace_size(8, 4096, 192, 8, 1536, 0, None) == hy3moe.ERR_NULL


def _fwd(L, T=16, d=512, E=32, k=8, F=128, x=A, wg=A, gu=A, dn=A, out=A, ws=A, nws=1 << 40,
         bias=NUL, idx=NUL, w=NUL):
    return L.hy3moe_forward(x, wg, gu, dn, out, T, d, E, k, F, 2.826, NUL, bias, idx, w, ws, nws)


def test_forward_argument_checks(L):
    assert _fwd(L, T=-1) == hy3moe.ERR_SHAPE
    assert _fwd(L, k=0) == hy3moe.ERR_SHAPE
    assert _fwd(L, k=33, E=32) == hy3moe.ERR_SHAPE
    assert _fwd(L, d=0) == hy3moe.ERR_SHAPE
    assert _fwd(L, k=17, E=64) == hy3moe.ERR_UNSUPPORTED
    assert _fwd(L, E=1025) == hy3moe.ERR_UNSUPPORTED
    assert _fwd(L, d=520) == hy3moe.ERR_UNSUPPORTED
    assert _fwd(L, F=100) == hy3moe.ERR_UNSUPPORTED
    assert _fwd(L, T=(1 << 24) + 1) == hy3moe.ERR_UNSUPPORTED
    assert _fwd(L, x=NUL) == hy3moe.ERR_NULL
    assert _fwd(L, dn=NUL) == hy3moe.ERR_NULL
    assert _fwd(L, ws=NUL) == hy3moe.ERR_NULL
    assert _fwd(L, x=MIS) == hy3moe.ERR_ALIGN
    assert _fwd(L, out=MIS) == hy3moe.ERR_ALIGN
    assert _fwd(L, bias=MIS) == hy3moe.ERR_ALIGN
    assert _fwd(L, idx=MIS) == hy3moe.ERR_ALIGN
    st, need = _ws(L, 16, 512, 32, 8, 128)
    assert _fwd(L, nws=need - 1) == hy3moe.ERR_WORKSPACE
    # T == 0 is a no-op that needs no pointers at all
    assert _fwd(L, T=0, x=NUL, wg=NUL, gu=NUL, dn=NUL, out=NUL, ws=NUL, nws=0) == hy3moe.OK


def _fwd_na(L, T=16, d=512, E=32, k=8, F=128, x=A, wg=A, gu=A, dn=A, out=A, bias=NUL, idx=NUL, w=NUL):
    return L.hy3moe_forward_noalloc(x, wg, gu, dn, out, T, d, E, k, F, 2.826, NUL, bias, idx, w)


def test_forward_noalloc_argument_checks(L):
    """Checked on the host before the scratch is looked up: bad arguments,
    and sizes beyond the static scratch (64 MiB) with a status of their own."""
    assert _fwd_na(L, T=-1) == hy3moe.ERR_SHAPE
    assert _fwd_na(L, k=17, E=64) == hy3moe.ERR_UNSUPPORTED
    assert _fwd_na(L, x=NUL) == hy3moe.ERR_NULL
    assert _fwd_na(L, out=NUL) == hy3moe.ERR_NULL
    assert _fwd_na(L, gu=MIS) == hy3moe.ERR_ALIGN
    assert _fwd_na(L, idx=MIS) == hy3moe.ERR_ALIGN
    assert _fwd_na(L, T=0, x=NUL) == hy3moe.OK
    assert hy3moe.workspace_size(603, 4096, 192, 8, 1536) <= hy3moe.NOALLOC_SCRATCH_BYTES
    assert hy3moe.workspace_size(604, 4096, 192, 8, 1536) > hy3moe.NOALLOC_SCRATCH_BYTES
    assert _fwd_na(L, T=604, d=4096, E=192, k=8, F=1536) == hy3moe.ERR_SCRATCH
    assert _fwd_na(L, T=8192, d=4096, E=192, k=8, F=1536) == hy3moe.ERR_SCRATCH
    assert b"static scratch" in L.hy3moe_status_string(hy3moe.ERR_SCRATCH)


def test_forward_fp8_argument_checks(L):
    def f(T=16, sgu=A, sdn=A, ws=A, nws=1 << 40, k=8):
        return L.hy3moe_forward_fp8(A, A, A, sgu, A, sdn, A, T, 512, 32, k, 128, 2.826, NUL, NUL,
                                    NUL, NUL, ws, nws)
    assert f(T=-3) == hy3moe.ERR_SHAPE
    assert f(sgu=NUL) == hy3moe.ERR_NULL
    assert f(sdn=MIS) == hy3moe.ERR_ALIGN
    assert f(nws=10) == hy3moe.ERR_WORKSPACE
    assert f(T=0, ws=NUL, nws=0) == hy3moe.OK


def test_route_and_permute_argument_checks(L):
    def r(T=16, d=512, E=32, k=8, x=A, idx=A, ws=A, nws=1 << 40):
        return L.hy3moe_route(x, A, NUL, T, d, E, k, 2.826, idx, A, ws, nws, NUL)
    assert r(k=40) == hy3moe.ERR_SHAPE
    assert r(x=NUL) == hy3moe.ERR_NULL
    assert r(idx=MIS) == hy3moe.ERR_ALIGN
    assert r(nws=0) == hy3moe.ERR_WORKSPACE
    assert r(d=96) == hy3moe.ERR_UNSUPPORTED
    assert r(T=0, x=NUL, ws=NUL, nws=0) == hy3moe.OK

    def p(T=16, E=32, k=8, idx=A, row=A, ws=A, nws=1 << 40):
        return L.hy3moe_permute(idx, T, E, k, A, A, row, A, ws, nws, NUL)
    assert p(k=0) == hy3moe.ERR_SHAPE
    assert p(idx=NUL) == hy3moe.ERR_NULL
    assert p(row=MIS) == hy3moe.ERR_ALIGN
    assert p(nws=4) == hy3moe.ERR_WORKSPACE
    assert p(T=0, idx=NUL, ws=NUL, nws=0) == hy3moe.OK


def test_quantize_rows_argument_checks(L):
    q = L.hy3moe_quantize_rows_e4m3
    assert q(A, -1, 64, A, A, NUL) == hy3moe.ERR_SHAPE
    assert q(A, 4, 100, A, A, NUL) == hy3moe.ERR_UNSUPPORTED
    assert q(NUL, 4, 64, A, A, NUL) == hy3moe.ERR_NULL
    assert q(A, 4, 64, MIS, A, NUL) == hy3moe.ERR_ALIGN
    assert q(NUL, 0, 64, NUL, NUL, NUL) == hy3moe.OK


def _bws(L, T, d=4096, E=192, k=8, F=1536):
    n = ctypes.c_size_t(0)
    st = L.hy3moe_block_workspace_size(T, d, E, k, F, ctypes.byref(n))
    return st, n.value


def test_block_workspace_size(L):
    prev = -1
    for T in (1, 64, 8192, 65536):
        st, n = _bws(L, T)
        assert st == 0 and n > prev
        prev = n
        # the shared expert's T rows of y and the route_norm copy of x on top
        assert n >= _ws(L, T)[1] + T * 4096 * 2 + T * 4096 * 2
    assert _bws(L, 8, E=1024)[0] == hy3moe.ERR_UNSUPPORTED     # E + 1 experts in the dispatch
    assert _bws(L, 8, E=1023)[0] == hy3moe.OK
    assert L.hy3moe_block_workspace_size(8, 4096, 192, 8, 1536, None) == hy3moe.ERR_NULL


def _blk(L, T=16, d=512, E=32, k=8, F=128, x=A, nw=A, eps=1e-6, wg=A, sb=NUL, gu=A, dn=A, sgu=A,
         sdn=A, out=A, ws=A, nws=1 << 40):
    return L.hy3moe_block_forward(x, nw, eps, wg, sb, gu, dn, sgu, sdn, out, T, d, E, k, F, 2.826,
                                  NUL, NUL, NUL, ws, nws)


def test_block_forward_argument_checks(L):
    assert _blk(L, T=-1) == hy3moe.ERR_SHAPE
    assert _blk(L, eps=-1.0) == hy3moe.ERR_SHAPE
    assert _blk(L, eps=float("nan")) == hy3moe.ERR_SHAPE
    assert _blk(L, E=1024, k=8) == hy3moe.ERR_UNSUPPORTED
    assert _blk(L, x=NUL) == hy3moe.ERR_NULL
    assert _blk(L, sgu=NUL) == hy3moe.ERR_NULL                  # shared expert: both or neither
    assert _blk(L, sdn=NUL) == hy3moe.ERR_NULL
    assert _blk(L, sb=MIS) == hy3moe.ERR_ALIGN
    assert _blk(L, nw=MIS) == hy3moe.ERR_ALIGN
    assert _blk(L, sgu=MIS) == hy3moe.ERR_ALIGN
    st, need = _bws(L, 16, 512, 32, 8, 128)
    assert _blk(L, nws=need - 1) == hy3moe.ERR_WORKSPACE
    assert _blk(L, T=0, x=NUL, nw=NUL, wg=NUL, gu=NUL, dn=NUL, sgu=NUL, sdn=NUL, out=NUL, ws=NUL,
                nws=0) == hy3moe.OK


def test_block_forward_bf16_argument_checks(L):
    def b(T=16, d=512, E=32, k=8, F=128, res=A, out=A, x=A, sgu=A, ws=A, nws=1 << 40):
        return L.hy3moe_block_forward_bf16(x, A, 1e-6, A, NUL, A, A, sgu, A, res, out, T, d, E, k, F,
                                           2.826, NUL, NUL, NUL, ws, nws)
    assert b(T=-1) == hy3moe.ERR_SHAPE
    assert b(out=NUL) == hy3moe.ERR_NULL
    assert b(x=NUL) == hy3moe.ERR_NULL
    assert b(sgu=NUL) == hy3moe.ERR_NULL
    assert b(out=MIS) == hy3moe.ERR_ALIGN
    assert b(res=MIS) == hy3moe.ERR_ALIGN
    st, need = _bws(L, 16, 512, 32, 8, 128)
    assert b(nws=need - 1) == hy3moe.ERR_WORKSPACE
    assert b(T=0, res=NUL, out=NUL, x=NUL, sgu=NUL, ws=NUL, nws=0) == hy3moe.OK


def test_forward_fp8_block128_argument_checks(L):
    def f(T=16, d=512, E=32, k=8, F=256, x=A, sg=A, out=A, ws=A, nws=64):
        return L.hy3moe_forward_fp8_block128(x, A, A, sg, A, A, out, T, d, E, k, F, 2.826, NUL, NUL,
                                             NUL, NUL, ws, nws)
    assert f(T=-1) == hy3moe.ERR_SHAPE
    assert f(F=384) == hy3moe.ERR_UNSUPPORTED            # whole 256-element batches only
    assert f(d=640) == hy3moe.ERR_UNSUPPORTED
    assert f(d=16640) == hy3moe.ERR_UNSUPPORTED          # more than 128 k-blocks per row
    assert f(sg=NUL) == hy3moe.ERR_NULL
    assert f(sg=MIS) == hy3moe.ERR_ALIGN
    assert f(nws=64) == hy3moe.ERR_WORKSPACE
    assert f(T=0, x=NUL, sg=NUL, out=NUL, ws=NUL, nws=0) == hy3moe.OK


def test_route_ex_argument_checks(L):
    def r(T=16, d=512, E=32, k=8, x=A, nw=NUL, eps=1e-6, sb=NUL, ws=A, nws=1 << 40):
        return L.hy3moe_route_ex(x, nw, eps, A, NUL, sb, T, d, E, k, 2.826, A, A, ws, nws, NUL)
    assert r(k=40) == hy3moe.ERR_SHAPE
    assert r(eps=-0.5) == hy3moe.ERR_SHAPE
    assert r(x=NUL) == hy3moe.ERR_NULL
    assert r(sb=MIS) == hy3moe.ERR_ALIGN
    assert r(nw=MIS) == hy3moe.ERR_ALIGN
    assert r(nws=64) == hy3moe.ERR_WORKSPACE
    assert r(nw=A, nws=64) == hy3moe.ERR_WORKSPACE
    assert r(T=0, x=NUL, ws=NUL, nws=0) == hy3moe.OK


def test_header_compiles_as_c_and_links(tmp_path, L):
    """A plain C99 caller: include/hy3moe.h compiles as C with warnings as
    errors, every declared function links against libhy3moe.so, and host-only
    calls (sizes, argument rejection) work without a GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    names = sorted(hy3moe.EXPORTS)
    table = ",\n    ".join(f"(fn){n}" for n in names)
    src = tmp_path / "use_abi.c"
    src.write_text(f"""#include <stdio.h>
#include "hy3moe.h"
typedef void (*fn)(void);
static fn every_entry[] = {{
    {table}
}};
int main(void) {{
    size_t bytes = 0;
    int ok = hy3moe_workspace_size(64, 4096, 192, 8, 1536, HY3MOE_WEIGHTS_BF16, &bytes);
    int bad = hy3moe_workspace_size(-1, 4096, 192, 8, 1536, HY3MOE_WEIGHTS_BF16, &bytes);
    printf("%d %d %d %s\\n", (int)(sizeof every_entry / sizeof every_entry[0]), ok, bad,
           hy3moe_status_string(bad));
    return (ok == HY3MOE_OK && bad != HY3MOE_OK) ? 0 : 1;
}}
""")
    exe = tmp_path / "use_abi"
    # a sanitized build of the library (tests/test_abi_sanitized.py) needs the
    # preloaded sanitizer runtime on the link line as well
    san_rt = [p for p in os.environ.get("LD_PRELOAD", "").split() if "libclang_rt.asan" in p]
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), hy3moe.LIB_PATH, *san_rt, f"-Wl,-rpath,{os.path.dirname(hy3moe.LIB_PATH)}",
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    n, ok, bad, msg = res.stdout.split(maxsplit=3)
    assert int(n) == len(names) and int(ok) == 0 and int(bad) < 0 and msg.strip()
