"""The C ABI without a GPU: the built library loads, exports every function
include/flashmap.h declares, and its host-side checks (sizes, NULL pointers,
temperatures, configurations) fail with the documented status before anything
would be enqueued.  No call here reaches a kernel."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashmap.h")

fm = pytest.importorskip("step_flow_map_amd")
if not os.path.exists(fm.binding.LIB_PATH):
    pytest.skip("libflashmap.so is not built", allow_module_level=True)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert {"fm_create", "fm_draft", "fm_verify", "fm_draft_sample", "fm_verify_sample"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", fm.binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = fm.lib()
    for n in names:
        assert getattr(L, n) is not None


def _cfg(**kw):
    base = dict(V=1024, d=256, L=2, n_heads=4, H=512, C_max=64, dtype="f32")
    base.update(kw)
    return fm.make_config(**base)


def test_workspace_size_and_config_checks():
    n = fm.fm_workspace_bytes(_cfg())
    assert n > 0
    # more context or more branches need more workspace
    assert fm.fm_workspace_bytes(_cfg(C_max=4096)) > n
    assert fm.fm_workspace_bytes(_cfg(max_branches=4)) > n
    for bad in (dict(d=200), dict(n_heads=3), dict(V=10), dict(K=8), dict(max_branches=5),
                dict(n_ctx_layers=4), dict(max_steps=0), dict(d=8192, n_heads=64)):
        assert fm.fm_workspace_bytes(_cfg(**bad)) == 0, bad
        assert fm.fm_last_error() != ""


def test_null_and_range_checks_return_einval():
    L = fm.lib()
    null = ctypes.c_void_p(None)
    # greedy verify: NULL pointers, bad sizes
    assert L.fm_verify(null, fm.FM_BF16, 1, 16, 100, null, null, null, null, null) == fm.FM_EINVAL
    dummy = ctypes.c_void_p(256)   # never dereferenced: the size check fails first
    assert L.fm_verify(dummy, fm.FM_BF16, 0, 16, 100, dummy, dummy, dummy, dummy, null) == fm.FM_EINVAL
    assert L.fm_verify(dummy, fm.FM_BF16, 1, 65, 100, dummy, dummy, dummy, dummy, null) == fm.FM_EINVAL
    assert L.fm_verify(dummy, 7, 1, 16, 100, dummy, dummy, dummy, dummy, null) == fm.FM_EINVAL
    assert "dtype" in fm.fm_last_error()
    # handle-based calls with a NULL handle
    assert L.fm_draft(null, dummy, 1, null, 0, dummy, null, null, null) == fm.FM_EINVAL
    assert L.fm_verify_sample(null, dummy, fm.FM_BF16, 1, dummy, dummy, dummy, 1.0, 0, dummy, dummy,
                              null) == fm.FM_EINVAL
    assert L.fm_verify_greedy(null, dummy, fm.FM_BF16, 1, dummy, dummy, dummy, dummy, null) == fm.FM_EINVAL
    seeds = (ctypes.c_uint64 * 2)(1, 2)
    counts = (ctypes.c_int * 2)(0, 0)
    assert L.fm_draft_batch_sample(null, dummy, 2, null, counts, 1.0, seeds, dummy, dummy, dummy,
                                   null) == fm.FM_EINVAL
    assert L.fm_verify_sample_batch(null, dummy, fm.FM_BF16, 2, dummy, dummy, dummy, 1.0, seeds, dummy, dummy,
                                    null) == fm.FM_EINVAL
    assert L.fm_context_length(null) == -1
    assert L.fm_context_truncate(null, 0, null) == fm.FM_EINVAL
    assert L.fm_context_truncate_req(null, 0, 0, null) == fm.FM_EINVAL
    assert L.fm_context_sync(null, null) == fm.FM_EINVAL


def test_sampling_temperature_checks():
    L = fm.lib()
    null = ctypes.c_void_p(None)
    dummy = ctypes.c_void_p(256)
    for tau in (0.0, -1.0, float("inf"), float("nan")):
        assert L.fm_draft_sample(dummy, dummy, 1, null, 0, tau, 1, dummy, dummy, dummy, null) == fm.FM_EINVAL
        assert "temperature" in fm.fm_last_error()
    # sampling needs the logits and log-normaliser outputs
    assert L.fm_draft_sample(dummy, dummy, 1, null, 0, 1.0, 1, dummy, null, dummy, null) == fm.FM_EINVAL
    assert L.fm_draft_sample(dummy, dummy, 1, null, 0, 1.0, 1, dummy, dummy, null, null) == fm.FM_EINVAL


def test_create_rejects_bad_arguments_before_touching_a_device():
    L = fm.lib()
    h = ctypes.c_void_p()
    cfg = _cfg()
    # NULL workspace, misaligned workspace, too small a workspace
    assert L.fm_create(ctypes.byref(cfg), ctypes.c_void_p(None), 1 << 30, 0, ctypes.byref(h)) == fm.FM_EINVAL
    assert L.fm_create(ctypes.byref(cfg), ctypes.c_void_p(4096 + 8), 1 << 30, 0, ctypes.byref(h)) == fm.FM_EINVAL
    assert L.fm_create(ctypes.byref(cfg), ctypes.c_void_p(4096), 16, 0, ctypes.byref(h)) == fm.FM_ECAPACITY
    bad = _cfg(d=200)
    assert L.fm_create(ctypes.byref(bad), ctypes.c_void_p(4096), 1 << 30, 0, ctypes.byref(h)) == fm.FM_EINVAL
