"""The C-ABI library loads and exports every symbol include/dap.h declares;
host-side argument checks answer without touching a GPU."""
import ctypes
import os
import re

import pytest

import decoder_attention_paged_amd as dap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "dap.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(dap_\w+)\s*\(", text, re.M)))


def test_header_and_exports_agree():
    names = _declared()
    assert len(names) >= 12
    lib = dap.load_library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dap.h but not exported"
    assert sorted(dap.EXPORTS) == names


def _model(**kw):
    m = dap._Model()
    m.n_q_heads, m.n_kv_heads, m.head_dim, m.page_size = 32, 8, 128, 64
    m.window, m.max_position, m.rope_theta = 0, 4096, 1e4
    for k, v in kw.items():
        setattr(m, k, v)
    return m


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=80), dap.UNSUPPORTED),
    (dict(page_size=16), dap.UNSUPPORTED),
    (dict(n_kv_heads=5), dap.INVALID_ARG),
    (dict(n_q_heads=64, n_kv_heads=2), dap.UNSUPPORTED),
    (dict(max_position=0), dap.INVALID_ARG),
    (dict(window=-1), dap.INVALID_ARG),
    (dict(rope_theta=0.0), dap.INVALID_ARG),
    (dict(llama3=1, llama3_factor=8.0, llama3_low_freq_factor=4.0, llama3_high_freq_factor=1.0,
          llama3_original_max_position=8192.0), dap.INVALID_ARG),
    (dict(qk_norm=1, qk_norm_eps=0.0), dap.INVALID_ARG),
])
def test_create_rejects_bad_models_before_any_device_call(kw, status):
    lib = dap.load_library()
    h = ctypes.c_void_p()
    rc = lib.dap_create(ctypes.byref(_model(**kw)), ctypes.byref(h))
    assert rc == status
    assert h.value is None
    assert lib.dap_last_error()


def test_null_handle_is_rejected():
    lib = dap.load_library()
    assert lib.dap_set_validate(None, 1) == dap.INVALID_ARG
    assert lib.dap_decode_workspace_bytes(None, 4) == 0
    assert lib.dap_attn_decode_paged(None, None, 0, 1, None, None, None, 1, 1, None, None, 1, None, 0,
                                     None, 0, None) == dap.INVALID_ARG
