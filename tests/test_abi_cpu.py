"""The C-ABI library loads and exports every symbol include/lacache.h declares.

No GPU: only calls that return before touching the device are made.
"""

import ctypes
import os
import re

import pytest

from exact_attention_state_amd import lacache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lacache.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LACACHE_API\s+[\w\s\*]+?\b(lacache_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lacache.LIB_PATH):
        from exact_attention_state_amd import build
        build.build()
    return lacache.load_library()


def test_header_declares_the_abi():
    names = _declared()
    assert set(names) == set(lacache.EXPORTED), names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(5):
        assert lib.lacache_status_string(s)
    assert lib.lacache_status_string(99) == b"unknown status"


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, lacache.ERR_UNSUPPORTED),
    ("d_model", 300, lacache.ERR_UNSUPPORTED),
    ("n_kv_heads", 3, lacache.ERR_INVALID_ARG),
    ("max_seq_len", 0, lacache.ERR_INVALID_ARG),
    ("rope_theta", -1.0, lacache.ERR_INVALID_ARG),
    ("dtype", 7, lacache.ERR_INVALID_ARG),
])
def test_create_rejects_bad_configs_before_touching_the_device(lib, field, value, status):
    cfg = lacache.Config(4096, 32, 32, 128, 126464, 1024, 5e5, 1e-5, 0.0, lacache.BF16)
    setattr(cfg, field, value)
    h = ctypes.c_void_p(1)
    assert lib.lacache_create(ctypes.byref(cfg), ctypes.byref(h)) == status
    assert not h.value


def test_null_handles_are_rejected(lib):
    n = ctypes.c_size_t()
    assert lib.lacache_workspace_size(None, 1, None, 1, ctypes.byref(n)) == lacache.ERR_INVALID_ARG
    assert lib.lacache_block_step(None, None, None, None, 0, None, None, None, None, 0, None) == lacache.ERR_INVALID_ARG
    assert lib.lacache_destroy(None) == lacache.OK
