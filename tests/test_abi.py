"""The C ABI on the CPU: the library loads, exports every function that
include/prnn.h declares, and rejects NULL handles before touching a GPU."""
import ctypes
import os
import re

import pytest

from persistent_rnn_fwd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prnn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prnn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("prnn_create", "prnn_destroy", "prnn_forward_dense", "prnn_forward_sparse"):
        assert required in names
    assert set(names) == set(binding.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    lib = binding.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_every_public_enum_spans_all_ints():
    """Any int can cross the C ABI as an enum argument; an enum whose members
    span only a few bits would make reading such a value undefined, so each
    public enum carries a member at 0x7FFFFFFF."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    enums = re.findall(r"typedef enum \{(.*?)\}\s*(\w+);", text, flags=re.S)
    assert len(enums) >= 7
    for body, name in enums:
        assert re.search(r"_MAX_ENUM\s*=\s*0x7FFFFFFF", body), name


def test_null_handle_of_later_setters():
    lib = binding.load_library()
    bp = binding.BAD_PARAM
    assert lib.prnn_set_launch(None, binding.LAUNCH_PLAIN) == bp
    assert lib.prnn_set_launch(None, 0x7FFFFFFF) == bp
    assert lib.prnn_set_stack_mode(None, binding.STACK_AUTO) == bp


def test_status_strings():
    lib = binding.load_library()
    for code, name in binding.STATUS_NAMES.items():
        assert lib.prnn_status_string(code).decode() == name
    assert lib.prnn_status_string(99).decode() == "PRNN_STATUS_UNKNOWN"


def test_null_handle_is_bad_param():
    lib = binding.load_library()
    bp = binding.BAD_PARAM
    assert lib.prnn_create(None) == bp
    assert lib.prnn_destroy(None) == binding.SUCCESS
    assert lib.prnn_forward_dense(None, 4, 1, 1, 0, 16, 16, None, 16, None) == bp
    assert lib.prnn_forward_sparse(None, 4, 1, 1, 1, 16, 1, 16, 16, None, 16, None) == bp
    assert lib.prnn_sync_floor(None, 4, 1, 1, 16, None) == bp
    assert lib.prnn_synchronize(None, None) == bp
    assert lib.prnn_set_grid(None, 0) == bp
    assert lib.prnn_set_team_waves(None, 0) == bp
    assert lib.prnn_set_watchdog_us(None, 1) == bp
    assert lib.prnn_get_last_plan(None, None) == bp
    assert lib.prnn_debug_skip_publish(None, 0, 0) == bp
    assert lib.prnn_debug_jitter(None, 0, 0) == bp


def test_binding_refuses_cpu_tensors():
    import torch
    X = torch.zeros(2, 1, 4)
    W = torch.zeros(4, 4)
    h = object.__new__(binding.Handle)   # no GPU here: exercise argument checks only
    h._lib = binding.load_library()
    h._h = None
    with pytest.raises(ValueError):
        h.forward_dense(W, X)
