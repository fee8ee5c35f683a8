"""Host-side checks of the C-ABI library (no GPU needed).

The library loads, exports every function include/ragged_prefill.h declares,
and its host logic (validation, planning, status codes, empty-batch early
return) behaves as the header states.  No kernel is launched.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import varlen_prefill_amd as vp
from varlen_prefill_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert declared == set(_lib.EXPORTS), declared ^ set(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = declared - exported
    assert not missing, missing
    for name in declared:
        assert hasattr(lib, name)


def test_version_and_status_strings():
    lib = _lib.load()
    assert lib.rp_abi_version() == 7
    for st in (0, -1, -2, -3, -4):
        assert lib.rp_status_string(st)
    assert lib.rp_status_string(12345) == b"unknown status"


def test_not_available_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert vp.available() is False


def _plan(qi, ki, hq=8, hkv=2, d=128, causal=True, **kw):
    return vp.Plan(qi, ki, hq, hkv, d, causal, host_only=True, **kw)


@pytest.mark.parametrize("kwargs,status", [
    (dict(hq=8, hkv=3), _lib.RP_EINVAL),              # Hq % Hkv != 0
    (dict(d=64), _lib.RP_EUNSUPPORTED),               # head_dim
    (dict(hq=0, hkv=1), _lib.RP_EINVAL),              # no heads
    (dict(hq=256, hkv=1), _lib.RP_EUNSUPPORTED),      # group above 128
    (dict(kv_chunk=100), _lib.RP_EINVAL),             # chunk not a multiple of 64
    (dict(split_mode=7), _lib.RP_EINVAL),
    (dict(split_mode=-1), _lib.RP_EINVAL),
])
def test_plan_validation(kwargs, status):
    with pytest.raises(vp.RaggedPrefillError) as ei:
        _plan([0, 5], [0, 5], **kwargs)
    assert ei.value.status == status
    assert _lib.load().rp_last_error()


def test_plan_rejects_bad_offsets():
    for qi, ki in (([0, 5, 3], [0, 5, 9]), ([0, 5, 9], [0, 5, 4]), ([-2, 5], [0, 5])):
        with pytest.raises(vp.RaggedPrefillError) as ei:
            _plan(qi, ki)
        assert ei.value.status == _lib.RP_EINVAL


def test_empty_batches_plan_to_nothing():
    p = _plan([0], [0])
    assert p.info["num_items"] == 0 and p.workspace_bytes == 0
    p = _plan([4, 4, 4], [0, 10, 20])
    assert p.info["num_items"] == 0 and p.info["total_q"] == 0


def test_one_shot_empty_batch_returns_ok_without_device():
    lib = _lib.load()
    st = lib.ragged_prefill_bf16(None, None, None, None, None, None, None, 0, 8, 2, 128, 1,
                                 ctypes.c_float(0.1), None)
    assert st == _lib.RP_OK
    st = lib.ragged_prefill_bf16(None, None, None, None, None, None, None, -1, 8, 2, 128, 1,
                                 ctypes.c_float(0.1), None)
    assert st == _lib.RP_EINVAL


def test_run_rejects_host_only_plan():
    lib = _lib.load()
    p = _plan([0, 5], [0, 5])
    st = lib.rp_run(p.handle, None, None, None, None, None, ctypes.c_float(0.1), None, 0, None)
    assert st == _lib.RP_EINVAL
    assert b"host-only" in lib.rp_last_error()
    st = lib.rp_run(None, None, None, None, None, None, ctypes.c_float(0.1), None, 0, None)
    assert st == _lib.RP_EINVAL


def test_merge_entry_points_validate_before_any_launch():
    lib = _lib.load()
    P = ctypes.c_void_p
    buf = (ctypes.c_char * 4096)()
    p = ctypes.cast(buf, P)
    # head_dim must be a power of two in [8, 512]
    for d in (0, 4, 96, 1024):
        assert lib.rp_merge_state(p, p, p, p, p, p, 4, 2, d, None) == -1
        assert lib.rp_merge_states(p, p, p, p, 4, 2, 2, d, None) == -1
    assert lib.rp_merge_states(p, p, p, p, 4, 0, 2, 128, None) == -1      # num_states >= 1
    assert lib.rp_merge_state(p, p, p, p, p, p, -1, 2, 128, None) == -1   # rows >= 0
    assert lib.rp_merge_state(None, None, None, None, None, None, 0, 2, 128, None) == 0  # no rows
    assert lib.rp_merge_state(None, p, p, p, p, p, 3, 2, 128, None) == -1
    assert lib.rp_merge_state_in_place(p, None, p, p, 3, 2, 128, None) == -1


def test_shared_prefix_plan_host_logic():
    qo, kv, p_len = [30, 130, 0, 7], [30, 200, 9, 7], 700
    qi = np.concatenate([[5], 5 + np.cumsum(qo)]).astype(np.int32)
    ki = np.concatenate([[0], np.cumsum(kv)]).astype(np.int32)
    sp = vp.SharedPrefixPlan(qi, ki, p_len, 32, 8, 128, causal=True, host_only=True)
    unique = vp.Plan(qi, ki, 32, 8, 128, causal=True, host_only=True)
    shared = vp.Plan([0, sum(qo)], [0, p_len], 32, 8, 128, causal=False, host_only=True)
    i_sp, i_u, i_s = sp.info, unique.info, shared.info
    assert i_sp["num_items"] == i_u["num_items"] + i_s["num_items"]
    assert i_sp["flops"] == i_u["flops"] + i_s["flops"]
    assert i_sp["total_kv"] == sum(kv) + p_len
    # algorithmic bytes add the shared K and V once
    assert i_sp["bytes"] == i_u["bytes"] + 2 * 2 * p_len * 8 * 128
    # workspace: level workspace, shared O (bf16) and LSE, own-level LSE over rows [0, q_end)
    rows = sum(qo)
    al = lambda x: (x + 255) // 256 * 256
    need = (al(max(i_u["workspace_bytes"], i_s["workspace_bytes"])) + al(rows * 32 * 128 * 2)
            + al(rows * 32 * 4) + al(int(qi[-1]) * 32 * 4))
    assert sp.workspace_bytes == need
    for x in (sp, unique, shared):
        x.close()
    # causal needs qo_len <= kv_len in every request once the prefix is non-empty
    with pytest.raises(vp.RaggedPrefillError, match="qo_len <= kv_len"):
        vp.SharedPrefixPlan([0, 10], [0, 5], 1, 4, 2, 128, causal=True, host_only=True)
    vp.SharedPrefixPlan([0, 10], [0, 5], 0, 4, 2, 128, causal=True, host_only=True).close()
    vp.SharedPrefixPlan([0, 10], [0, 5], 1, 4, 2, 128, causal=False, host_only=True).close()
    with pytest.raises(vp.RaggedPrefillError):
        vp.SharedPrefixPlan([0, 10], [0, 5], -1, 4, 2, 128, causal=False, host_only=True)


def test_noalloc_rejects_plans_beyond_its_array():
    """rp_run_noalloc refuses, before any device call, a plan whose split-KV
    workspace exceeds its fixed 32 MiB array."""
    import ctypes
    # 64 decode-like requests over 16K keys in 2048-key chunks: 8 partial
    # states per (request, kv head), 64 KiB each
    p = _plan([i for i in range(65)], [16384 * i for i in range(65)], hq=32, hkv=8)
    assert p.workspace_bytes > (32 << 20)
    st = _lib.load().rp_run_noalloc(p.handle, None, None, None, None, None, ctypes.c_float(1.0), None)
    assert st == _lib.RP_EUNSUPPORTED
    assert b"32" in _lib.load().rp_last_error()
