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


@pytest.mark.parametrize("head_dim", [64, 96, 128])
def test_tile_layout_is_a_permutation_of_16_byte_chunks(head_dim):
    """dap_tile_layout (host only) maps each logical element to a distinct
    tile offset; every 8-element chunk of a K row (dims 8c..8c+7) and of a V
    dim (keys 8c..8c+7) is contiguous; the binding's pool helpers round-trip."""
    import torch
    D = head_dim
    ko, vo = dap.tile_offsets(D)
    for off in (ko, vo):
        assert sorted(off.reshape(-1).tolist()) == list(range(64 * D))
    for c in range(D // 8):
        run = ko[:, 8 * c:8 * c + 8]
        assert torch.equal(run - run[:, :1], torch.arange(8).expand(64, 8))
    for c in range(8):
        run = vo[8 * c:8 * c + 8, :].t()
        assert torch.equal(run - run[:, :1], torch.arange(8).expand(D, 8))
    # one kilobyte = one decode load: K chunk 0..63 are keys unit_key(0, i) at dims 0..31
    keys = [8 * (i >> 2) + (i & 3) for i in range(16)]
    first = sorted(int(ko[k, 8 * g]) for g in range(4) for k in keys)
    assert first == list(range(0, 512, 8))
    kp, vp = dap.pools(3, 2, D, device="cpu")
    kl = torch.randint(0, 16000, (2, 2, 64, D), dtype=torch.int16)
    vl = torch.randint(0, 16000, (2, 2, 64, D), dtype=torch.int16)
    dap.store_pages(kp, vp, [2, 0], kl, vl)
    k2, v2 = dap.pool_logical(kp, vp, [2, 0])
    assert torch.equal(k2.view(torch.int16), kl) and torch.equal(v2.view(torch.int16), vl)
    kg, vg = dap.gather_slots(kp, vp, torch.tensor([2 * 64 + 7, 63]))
    assert torch.equal(kg.view(torch.int16), torch.stack([kl[0, :, 7], kl[1, :, 63]]))
    assert torch.equal(vg.view(torch.int16), torch.stack([vl[0, :, 7], vl[1, :, 63]]))
