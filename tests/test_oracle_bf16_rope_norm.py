"""Pins for the oracle's bf16 codec, frequency table, rope and QK-norm.

Each check compares the oracle with something other than itself: a library
routine (torch's bfloat16 cast, torch's rms_norm, transformers' llama3 table
and rotate-half rope), a closed form, a brute-force search, or a property the
mathematics fixes."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bf16, norm, rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 codec

def test_bf16_decode_exhaustive_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16.to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_float32_inputs_match_torch_rne():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(20000) * 1e38).astype(np.float32),    # near overflow
        # exact ties: low 16 bits == 0x8000, with even and odd kept mantissas
        ((rng.integers(0, 1 << 15, 20000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38, 3.4e38], np.float32),
    ])
    x = x[np.isfinite(x) | np.isinf(x)]
    ours = bf16.from_f64(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _brute_force_bf16(x: float) -> int:
    """Nearest bf16 by searching the two neighbouring patterns; ties to even."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    b = int(np.float32(x).view(np.uint32)) >> 16     # truncation, same sign
    best = None
    for cand in (b - 1, b, b + 1, b + 2):
        if cand < 0 or (cand & 0x7F80) == 0x7F80 and (cand & 0x7F):
            continue
        v = float(bf16.to_f64(np.array([cand & 0xFFFF]))[0])
        d = abs(v - x)
        key = (d, cand & 1)
        if best is None or key < best[0]:
            best = (key, cand & 0xFFFF)
    return best[1]


def test_bf16_encode_float64_brute_force():
    rng = np.random.default_rng(2)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    # float64 values just off a bf16 tie, where rounding through float32 first
    # would round twice and land on the wrong side
    for m in range(1, 200):
        base = 1.0 + (2 * m + 1) * 2.0 ** -8          # exact tie between two bf16 values
        xs += [base + 2.0 ** -40, base - 2.0 ** -40, -(base + 2.0 ** -40)]
    xs = np.array(xs)
    ours = bf16.from_f64(xs)
    ref = np.array([_brute_force_bf16(float(v)) for v in xs], dtype=np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------ frequency table

def test_inv_freq_closed_form():
    f = rope.inv_freq(1e4, 4)
    assert f[0] == 1.0 and abs(f[1] - 0.01) < 1e-17
    f = rope.inv_freq(1e4, 128)
    assert abs(f[32] - 0.01) < 1e-16              # theta^(-1/2)
    assert abs(f[16] - 10.0 ** -1) < 1e-16        # theta^(-1/4)
    f = rope.inv_freq(1e6, 96)
    assert abs(f[24] - 1e-3) < 1e-18             # theta^(-1/2) at i = D/4
    assert np.all(np.diff(f) < 0)


def _llama3_golden():
    with open(os.path.join(GOLDEN, "llama3_bands.json")) as fh:
        return json.load(fh)


def test_llama3_bands_match_the_pages():
    g = _llama3_golden()
    l3 = (g["factor"], g["low_freq_factor"], g["high_freq_factor"], g["original_max_position"])
    base = rope.inv_freq(g["theta"], g["head_dim"])
    scaled = rope.inv_freq(g["theta"], g["head_dim"], l3)
    assert scaled.shape[0] == g["n_frequencies"]
    changed = np.nonzero(~np.isclose(scaled, base, rtol=0, atol=0) & ~np.isclose(scaled, base / 8, rtol=1e-15, atol=0))[0]
    assert list(changed) == g["blended_indices"]
    wl = 2 * math.pi / base
    short = wl < g["short_wavelength_edge"]
    long_ = wl > g["long_wavelength_edge"]
    assert np.array_equal(scaled[short], base[short])                 # unchanged exactly
    assert np.array_equal(scaled[long_], base[long_] / 8.0)           # divided by exactly 8
    mid = ~short & ~long_
    assert np.all((scaled[mid] > base[mid] / 8) & (scaled[mid] < base[mid]))  # strictly between
    longest = 2 * math.pi / scaled.min()
    assert abs(longest / g["largest_period_tokens"] - 1) < g["largest_period_rel_tol"]


def test_llama3_blend_is_continuous_at_both_edges():
    # A wide head gives densely spaced wavelengths through the blend band, so
    # the scaling ratio can be watched as the wavelength approaches each edge:
    # it must meet the unchanged band (ratio 1) at 2048 and the divided band
    # (ratio 1/8) at 8192, and fall monotonically in between.
    D = 1 << 16
    base = rope.inv_freq(5e5, D)
    scaled = rope.inv_freq(5e5, D, (8.0, 1.0, 4.0, 8192.0))
    wl = 2 * math.pi / base
    ratio = scaled / base
    near_short = (wl > 2048) & (wl < 2048 * 1.001)
    near_long = (wl < 8192) & (wl > 8192 * 0.999)
    assert near_short.any() and near_long.any()
    assert np.all(np.abs(ratio[near_short] - 1.0) < 2e-3)
    assert np.all(np.abs(ratio[near_long] - 0.125) < 2e-3)
    band = (wl >= 2048) & (wl <= 8192)
    assert np.all(np.diff(ratio[band]) <= 0)


def test_llama3_table_matches_transformers_black_box():
    tr = pytest.importorskip("transformers")
    from transformers import LlamaConfig
    from transformers import modeling_rope_utils as ru
    g = _llama3_golden()
    cfg = LlamaConfig(hidden_size=4096, num_attention_heads=32, num_key_value_heads=8,
                      head_dim=128, rope_theta=g["theta"], max_position_embeddings=131072,
                      rope_scaling={"rope_type": "llama3", "factor": g["factor"],
                                    "low_freq_factor": g["low_freq_factor"],
                                    "high_freq_factor": g["high_freq_factor"],
                                    "original_max_position_embeddings": int(g["original_max_position"])})
    ref, _ = ru._compute_llama3_parameters(cfg, "cpu")
    ref = ref.double().numpy()
    ours = rope.inv_freq(g["theta"], 128, (g["factor"], g["low_freq_factor"],
                                          g["high_freq_factor"], g["original_max_position"]))
    # transformers builds its table in float32
    assert np.max(np.abs(ours - ref) / ref) < 2e-6


# ---------------------------------------------------------------------- rope

def test_rope_worked_example_closed_form():
    with open(os.path.join(GOLDEN, "rope_worked.json")) as fh:
        g = json.load(fh)
    f = rope.inv_freq(g["theta"], g["head_dim"])
    assert np.allclose(f, g["inv_freq"], rtol=0, atol=1e-17)
    x = np.array(g["x"])
    for p in g["positions"]:
        y = rope.rotate(x[None, None, :], [p], f)[0, 0]
        a, b = float(p), p / 100.0
        expect = [x[0] * math.cos(a) - x[2] * math.sin(a),
                  x[1] * math.cos(b) - x[3] * math.sin(b),
                  x[2] * math.cos(a) + x[0] * math.sin(a),
                  x[3] * math.cos(b) + x[1] * math.sin(b)]
        assert np.allclose(y, expect, rtol=0, atol=1e-12)


def test_rope_identity_norm_composition_relative():
    rng = np.random.default_rng(3)
    D = 128
    f = rope.inv_freq(5e5, D, (8.0, 1.0, 4.0, 8192.0))
    x = rng.standard_normal((5, 3, D))
    # position 0 is the identity
    assert np.array_equal(rope.rotate(x, [0] * 5, f), x)
    # each (i, i + D/2) pair keeps its norm
    p = rng.integers(0, 65536, 5)
    y = rope.rotate(x, p, f)
    n_x = x[..., : D // 2] ** 2 + x[..., D // 2:] ** 2
    n_y = y[..., : D // 2] ** 2 + y[..., D // 2:] ** 2
    assert np.allclose(n_x, n_y, rtol=1e-12)
    # R_a then R_b equals R_{a+b}
    a = rng.integers(0, 30000, 5)
    b = rng.integers(0, 30000, 5)
    assert np.allclose(rope.rotate(rope.rotate(x, a, f), b, f), rope.rotate(x, a + b, f), atol=1e-9)
    # <R_p q, R_p' k> depends only on p - p'
    q, k = x[:1], x[1:2]
    d1 = np.sum(rope.rotate(q, [1000], f) * rope.rotate(k, [700], f))
    d2 = np.sum(rope.rotate(q, [50300], f) * rope.rotate(k, [50000], f))
    assert abs(d1 - d2) < 1e-9


def test_rope_matches_transformers_rotate_half():
    pytest.importorskip("transformers")
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    rng = np.random.default_rng(4)
    D = 96
    f = rope.inv_freq(1e4, D)
    pos = np.array([0, 1, 17, 2046, 4095])
    q = rng.standard_normal((len(pos), 4, D))
    k = rng.standard_normal((len(pos), 2, D))
    ang = pos[:, None].astype(np.float64) * f[None, :]
    emb = np.concatenate([ang, ang], axis=-1)
    cos = torch.from_numpy(np.cos(emb))[None]           # [1, T, D]
    sin = torch.from_numpy(np.sin(emb))[None]
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]     # [1, H, T, D]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    rq, rk = apply_rotary_pos_emb(tq, tk, cos, sin)
    assert np.allclose(rope.rotate(q, pos, f), rq[0].permute(1, 0, 2).numpy(), atol=1e-12)
    assert np.allclose(rope.rotate(k, pos, f), rk[0].permute(1, 0, 2).numpy(), atol=1e-12)


# ------------------------------------------------------------------- QK-norm

def test_qk_norm_matches_torch_rms_norm_per_head():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 8, 128)) * rng.uniform(0.1, 10, (7, 8, 1))
    g = rng.uniform(0.5, 1.5, 128)
    ours = norm.rms_norm_heads(x, g, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), 1e-6).numpy()
    assert np.allclose(ours, ref, rtol=1e-13, atol=1e-13)


def test_qk_norm_is_per_head_not_flattened():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 8, 128))
    g = np.ones(128)
    y = norm.rms_norm_heads(x, g, 1e-6)
    x2 = x.copy()
    x2[:, 3] *= 10.0                      # scale one head's slice
    y2 = norm.rms_norm_heads(x2, g, 1e-6)
    others = [h for h in range(8) if h != 3]
    assert np.array_equal(y[:, others], y2[:, others])     # other heads untouched
    assert np.allclose(y[:, 3], y2[:, 3], atol=1e-6)       # scale-invariant up to eps
    # unit gains: mean(y^2) = ms / (ms + eps)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-6), rtol=1e-12)
    # a flattened norm would differ
    flat = x.reshape(3, -1)
    yf = (flat / np.sqrt(np.mean(flat * flat, axis=-1, keepdims=True) + 1e-6)).reshape(x.shape)
    assert not np.allclose(yf, y, atol=1e-3)


def test_near_tie_flags_exactly_the_rounding_midpoints():
    # midpoints between adjacent bf16 values, built from their bit patterns
    rng = np.random.default_rng(7)
    bits = rng.integers(0x0001, 0x7F7F, 20000).astype(np.int64)
    bits |= rng.integers(0, 2, bits.size) << 15            # both signs
    lo = bf16.to_f64(bits)
    hi = bf16.to_f64(bits + 1)                             # next magnitude, same sign
    mid = 0.5 * (lo + hi)
    assert bf16.near_tie(mid, 0.0).all()
    # a quarter of the gap away from a midpoint is far from it
    assert not bf16.near_tie(mid + 0.25 * (hi - lo), 0.0).any()
    assert not bf16.near_tie(lo, 0.0).any()                # bf16 values themselves
    # the spacing halves below a power of two: 1 - 2^-9 is a midpoint, 1 + 2^-9 is not
    assert bf16.near_tie(np.array([1 - 2.0 ** -9, 1 + 2.0 ** -8, 2.0 ** -130 + 2.0 ** -134]), 0.0).all()
    assert not bf16.near_tie(np.array([1 + 2.0 ** -9, 1 - 2.0 ** -10]), 0.0).any()
    # the tolerance widens the band symmetrically
    x = np.array([1 + 2.0 ** -8 + 5e-13, 1 + 2.0 ** -8 - 5e-13, 1 + 2.0 ** -8 + 2e-12])
    assert list(bf16.near_tie(x, 1e-12)) == [True, True, False]
    assert not bf16.near_tie(np.array([np.nan, np.inf, 0.0]), 1e-12).any()
