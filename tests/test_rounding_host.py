"""The kernels' float64 -> bf16 rounding (used for q_out and the K pages),
compiled for the host and checked bit for bit against the oracle's direct
round-to-nearest-even on values chosen to hit every case: random bit
patterns over the whole float64 range, values a fraction of a bf16 step
either side of the bf16 grid at every exponent (subnormals included), exact
ties, overflow to infinity and the specials. The oracle's codec is pinned
against torch and a brute-force search in test_oracle_bf16_rope_norm.py."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import bf16

HERE = os.path.dirname(os.path.abspath(__file__))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _inputs():
    rng = np.random.default_rng(11)
    parts = [rng.integers(0, 2 ** 63, 400000, dtype=np.int64).view(np.float64),
             -rng.integers(0, 2 ** 63, 100000, dtype=np.int64).view(np.float64)]
    # bf16 grid points at exponents -140..127 and offsets of quarter steps plus tiny nudges
    e = rng.integers(-140, 128, 300000)
    m = rng.integers(128, 256, 300000)
    step = np.ldexp(1.0, np.maximum(e, -126) - 7)
    base = np.where(e >= -126, np.ldexp(m / 128.0, e), rng.integers(0, 128, 300000) * 2.0 ** -133)
    k = rng.integers(-3, 4, 300000) / 4.0
    nudge = rng.integers(-2, 3, 300000) * np.ldexp(step, -40)
    sign = np.where(rng.integers(0, 2, 300000) == 1, -1.0, 1.0)
    parts.append(sign * (base + k * step + nudge))
    # exact ties at every exponent, normal and subnormal
    ee, mm = np.meshgrid(np.arange(-126, 128), np.arange(128), indexing="ij")
    ties = np.ldexp(1.0 + mm / 128.0 + 1.0 / 256.0, ee).ravel()
    sub_ties = (np.arange(128) + 0.5) * 2.0 ** -133
    parts += [ties, -ties, sub_ties, -sub_ties]
    parts.append(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan,
                           (2.0 - 2.0 ** -7) * 2.0 ** 127,           # largest finite bf16
                           (2.0 - 2.0 ** -8) * 2.0 ** 127,           # its tie with infinity
                           np.nextafter((2.0 - 2.0 ** -8) * 2.0 ** 127, 0.0),
                           3.4028234663852886e38, 2.0 ** 128, 1e300,
                           2.0 ** -126, 2.0 ** -133, 2.0 ** -134, np.nextafter(2.0 ** -134, 1.0),
                           2.0 ** -149, 2.0 ** -150, 5e-324, -5e-324]))
    return np.concatenate(parts)


def test_kernel_rounding_matches_oracle(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available to build the host driver")
    exe = tmp_path / "round"
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "--offload-arch=gfx950", "-w",
                        os.path.join(HERE, "host", "round_f64_to_bf16.hip"), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    x = _inputs()
    (tmp_path / "in.bin").write_bytes(x.tobytes())
    r = subprocess.run([str(exe), str(tmp_path / "in.bin"), str(tmp_path / "out.bin")], capture_output=True)
    assert r.returncode == 0
    got = np.frombuffer((tmp_path / "out.bin").read_bytes(), dtype=np.uint16)
    ref = bf16.from_f64(x)
    nan = np.isnan(x)
    assert got.shape == ref.shape
    # a NaN stays a quiet NaN (its sign bit may differ from the oracle's)
    assert np.all((got[nan] & 0x7FFF) == 0x7FC0)
    bad = np.nonzero(got[~nan] != ref[~nan])[0]
    assert bad.size == 0, f"{bad.size} of {x.size} differ, e.g. {x[~nan][bad[:5]]!r}"
