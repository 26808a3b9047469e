"""CPU-side checks of the C ABI library: it loads, exports every symbol the
header declares, and its pure host functions behave. No GPU compute."""
import ctypes
import os
import re
import subprocess

import pytest

from moe_expert_ffn_persistent_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def _lib_or_skip():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmoe_ffn.so not built")
    return _lib.load()


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    _lib_or_skip()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in _declared_functions():
        assert name in exported, name
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared_functions():
        assert getattr(lib, name) is not None


def test_abi_version_and_status_strings():
    _lib_or_skip()
    assert _lib.abi_version() == 5
    for st in (0, -1, -2, -3, -4, -5):
        assert _lib.status_string(st) and "unknown" not in _lib.status_string(st)
    assert "unknown" in _lib.status_string(-99)


def test_layout_scratch_bytes_host_only():
    _lib_or_skip()
    s = _lib.MoeShape(8, 512, 256, 8, 0, 32, 7168, 2048, 0)
    chunks = -(-8 * 512 * 8 // 256)
    assert _lib.layout_scratch_bytes(s) == chunks * 32 * 4
    bad = _lib.MoeShape(8, 512, 256, 8, 250, 32, 7168, 2048, 0)   # local range past E
    assert _lib.layout_scratch_bytes(bad) == 0
    bad2 = _lib.MoeShape(8, 512, 256, 8, 0, 32, 7000, 2048, 0)    # H not a multiple of 128
    assert _lib.layout_scratch_bytes(bad2) == 0
