"""The C-ABI library: it loads, exports what include/pk.h declares, and the
binding's struct layouts match the header. No compute calls (no GPU here)."""

import ctypes
import os
import re
import subprocess

import pytest

from iterative_stencil_pde_amd import pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pk_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pk.LIB_PATH):
        pytest.skip("engine library not built")
    return pk.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["pk_create", "pk_submit", "pk_wait", "pk_readback",
                     "pk_run_launch_per_iter", "pk_destroy", "pk_strerror"]:
        assert required in names
    assert sorted(pk.EXPORTED) == names


PAGES = ("Persistent Kernels", "Grid-Wide Barriers", "persistent-thread page", "@persistent")


def comments_before_declarations():
    """Map each declared function to the comment block right above its declaration."""
    text = open(HEADER).read()
    out = {}
    for m in re.finditer(r"/\*((?:(?!\*/).)*)\*/\s*(?:(?:const\s+)?[a-z_]+\**\s+)+\**(pk_[a-z_]+)\s*\(",
                         text, flags=re.S):
        out[m.group(2)] = m.group(1)
    return out


def test_every_declared_call_cites_a_page():
    """Each entry point's comment names the page (and section) that defines the
    operation it performs."""
    blocks = comments_before_declarations()
    for name in declared_functions():
        assert name in blocks, f"{name}: no comment block above its declaration"
        if "callers that cannot allocate" in blocks[name]:
            continue  # names the callers it serves instead of a page (no page defines it)
        assert any(p in blocks[name] for p in PAGES), f"{name}: its comment cites no page"


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", pk.LIB_PATH], text=True)
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_struct_layouts_match_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "pk.h"
#define P(T, F) printf(#T "." #F " %zu\\n", offsetof(T, F))
int main(void) {
  printf("pk_opts %zu\\npk_task %zu\\npk_result %zu\\npk_info %zu\\n",
         sizeof(pk_opts), sizeof(pk_task), sizeof(pk_result), sizeof(pk_info));
  P(pk_opts, h); P(pk_opts, flags); P(pk_opts, stream); P(pk_opts, idle_timeout_s); P(pk_opts, exchange);
  P(pk_opts, reserved);
  P(pk_result, residual); P(pk_result, errors); P(pk_result, status);
  P(pk_info, exchange); P(pk_info, lds_bytes); P(pk_info, tasks_carried); P(pk_info, kernel_ms); P(pk_info, kernel_launches);
  P(pk_info, tasks_fused);
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-I", os.path.join(ROOT, "include"),
                           str(prog), "-o", str(exe)])
    got = dict(ln.rsplit(" ", 1) for ln in subprocess.check_output([str(exe)], text=True).splitlines())
    assert int(got["pk_opts"]) == ctypes.sizeof(pk.pk_opts)
    assert int(got["pk_task"]) == ctypes.sizeof(pk.pk_task)
    assert int(got["pk_result"]) == ctypes.sizeof(pk.pk_result)
    assert int(got["pk_info"]) == ctypes.sizeof(pk.pk_info)
    for key, val in got.items():
        if "." in key:
            s, f = key.split(".")
            assert getattr(getattr(pk, s), f).offset == int(val), key


def test_status_strings_and_defaults(lib):
    assert pk.pk_strerror(pk.PK_OK) == "ok"
    assert "invalid" in pk.pk_strerror(pk.PK_EINVAL)
    assert "unknown" in pk.pk_strerror(12345)
    o = pk.pk_opts_default()
    assert o.dtype == pk.PK_F32 and o.mode == pk.PK_PERSISTENT and o.layout == pk.PK_LAYOUT_AUTO
    assert o.h == 0.0 and o.max_blocks == 0 and o.stream is None


def test_create_rejects_bad_arguments_before_touching_a_device(lib):
    import numpy as np
    h = ctypes.c_void_p()
    bc = np.zeros((2, 8), np.float32)
    o = pk.pk_opts_default()
    # ny < 3, NULL bc, NULL out: refused by argument checks alone
    assert lib.pk_create(8, 2, bc.ctypes.data, None, ctypes.byref(o), ctypes.byref(h)) == pk.PK_EINVAL
    assert lib.pk_create(8, 8, None, None, ctypes.byref(o), ctypes.byref(h)) == pk.PK_EINVAL
    assert lib.pk_create(8, 8, bc.ctypes.data, None, ctypes.byref(o), None) == pk.PK_EINVAL
    bad = pk.pk_opts_default(dtype=7)
    assert lib.pk_create(8, 8, bc.ctypes.data, None, ctypes.byref(bad), ctypes.byref(h)) == pk.PK_EINVAL
    bad = pk.pk_opts_default(threads=100)
    assert lib.pk_create(8, 8, bc.ctypes.data, None, ctypes.byref(bad), ctypes.byref(h)) == pk.PK_EINVAL
    bad = pk.pk_opts_default(exchange=4)
    assert lib.pk_create(8, 8, bc.ctypes.data, None, ctypes.byref(bad), ctypes.byref(h)) == pk.PK_EINVAL
    for k in (-1, 9, 10, 11, 13, 16):  # pass depths the kernel does not carry
        bad = pk.pk_opts_default(pass_sweeps=k)
        assert lib.pk_create(8, 8, bc.ctypes.data, None, ctypes.byref(bad), ctypes.byref(h)) == pk.PK_EINVAL
    for x in (pk.PK_EXCHANGE_NEIGHBOR, pk.PK_EXCHANGE_TAGGED):  # the negative control keeps barriers
        bad = pk.pk_opts_default(exchange=x, flags=pk.PK_DBG_BROKEN_BARRIER)
        assert lib.pk_create(8, 8, bc.ctypes.data, None, ctypes.byref(bad), ctypes.byref(h)) == pk.PK_EINVAL
    for lay in (pk.PK_LAYOUT_STREAM, pk.PK_LAYOUT_RESIDENT):  # tagged words: register tile only
        bad = pk.pk_opts_default(exchange=pk.PK_EXCHANGE_TAGGED, layout=lay)
        assert lib.pk_create(8, 8, bc.ctypes.data, None, ctypes.byref(bad), ctypes.byref(h)) == pk.PK_EINVAL
    bad = pk.pk_opts_default()
    bad.reserved[3] = 1
    assert lib.pk_create(8, 8, bc.ctypes.data, None, ctypes.byref(bad), ctypes.byref(h)) == pk.PK_EINVAL
    # h = 0 needs a square grid
    assert lib.pk_create(8, 9, bc.ctypes.data, None, ctypes.byref(o), ctypes.byref(h)) == pk.PK_EINVAL
    assert h.value is None
    # NULL engine handles
    assert lib.pk_destroy(None) == pk.PK_OK
    assert lib.pk_submit(None, pk.pk_task(pk.PK_SWEEP, 1), None) == pk.PK_EINVAL
    assert lib.pk_wait(None, 1, 1.0, None) == pk.PK_EINVAL
    assert lib.pk_readback(None, None, 0) == pk.PK_EINVAL
    assert lib.pk_get_info(None, None) == pk.PK_EINVAL
