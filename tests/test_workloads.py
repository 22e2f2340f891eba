"""The seeded synthetic inputs: deterministic, CPU/GPU-independent counters,
shapes and model constants as the pages state them."""
import json
import os

import numpy as np
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_generator_is_deterministic_and_sliceable():
    key = W.stream_key("t", "x")
    a = W.normal_matrix(key, 16, 300)
    b = W.normal_matrix(key, 16, 300)
    assert torch.equal(a, b)
    tail = W.normal_matrix(key, 6, 300, row0=10)        # regenerate a slice alone
    assert torch.equal(a[10:], tail)
    other = W.normal_matrix(W.stream_key("t", "y"), 16, 300)
    assert not torch.equal(a, other)


def test_generator_values_look_standard_normal():
    x = W.normal_matrix(W.stream_key("stats"), 512, 1024).view(torch.bfloat16).double()
    assert abs(float(x.mean())) < 0.01
    assert abs(float(x.std()) - 1.0) < 0.01
    g = W.uniform_bf16(W.stream_key("g"), torch.arange(100000), 0.5, 1.5).view(torch.bfloat16).double()
    assert float(g.min()) >= 0.5 and float(g.max()) <= 1.5


def test_page_values_depend_only_on_page_id():
    key = W.stream_key("pages")
    a = W.page_values(key, [3, 9, 3], 2, 64)
    assert torch.equal(a[0], a[2]) and not torch.equal(a[0], a[1])
    assert torch.equal(W.page_values(key, [9], 2, 64)[0], a[1])


def test_model_constants_match_the_pages():
    with open(os.path.join(GOLDEN, "models.json")) as fh:
        g = json.load(fh)
    for name in ("phi3", "mistral", "qwen3", "llama31"):
        m = W.ALL[name]().model
        want = g[name]
        assert m.n_q_heads == want["n_q_heads"] and m.n_kv_heads == want["n_kv_heads"]
        assert m.head_dim == want["head_dim"] and m.rope_theta == want["rope_theta"]
        assert m.window == want["window"]
        assert m.qk_norm_eps == want.get("qk_norm_eps")
        assert (list(m.llama3) if m.llama3 else None) == want.get("llama3")


def _check_tables(wl, shared_ok=False):
    t = wl.table
    used = t[t >= 0]
    assert used.min() >= 0 and used.max() < wl.n_pages
    if not shared_ok:
        assert len(np.unique(used)) == used.size


def test_workload_shapes():
    tiny = W.tiny()
    assert tiny.n_pre == 128 and tiny.model.qkv_width == 512
    phi = W.phi3()
    assert phi.n_pre == 4096 and phi.n_pages == 256 and phi.model.qkv_width == 9216
    _check_tables(phi)
    steps = W.phi3_decode_schedule()
    assert len(steps) == 2489 and sum(len(r) for r, _ in steps) == 7908
    mis = W.mistral()
    assert mis.n_dec == 64 and mis.dec_positions.min() >= 1023 and mis.dec_positions.max() <= 32767
    _check_tables(mis)
    lla = W.llama31()
    assert lla.n_pre == 8192 and lla.pre_positions[0] == 57344 and lla.pre_positions[-1] == 65535
    _check_tables(lla)
    q = W.qwen3()
    assert q.n_pre == 2048 and q.n_dec == 128 and q.model.qkv_width == 6144
    assert q.dec_positions.min() >= 512 and q.dec_positions.max() <= 40959
    _check_tables(q, shared_ok=True)
    assert all((q.table[r, :2] == q.table[4, :2]).all() for r in range(4, 8))
    own = np.concatenate([q.table[r][q.table[r] >= 0] for r in list(range(4)) + list(range(8, 136))]
                         + [q.table[r, 2:6] for r in range(4, 8)] + [q.table[4, :2]])
    assert len(np.unique(own)) == own.size == q.n_pages
