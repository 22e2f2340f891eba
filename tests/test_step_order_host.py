"""The fused step kernel's block order (step_order.h), compiled for the host:
over many sizes every prefill id and every decode id is launched exactly
once, each kind's ids come in increasing order, an id sits at a position
with the same remainder mod 8 (its XCD), and every decode group comes before
every prefill group."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_step_order_is_a_bijection_that_keeps_xcd_placement(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    exe = tmp_path / "order"
    subprocess.run([cc, "-std=c++17", "-O1", "-x", "hip", "--offload-arch=gfx950",
                    os.path.join(HERE, "host", "step_order_host.hip"), "-o", str(exe)], check=True,
                   capture_output=True)
    cases = [(p, d) for p in (0, 1, 7, 8, 9, 64, 576, 1000) for d in (0, 1, 8, 100, 8192, 8200)]
    cases = [c for c in cases if c[0] + c[1] > 0]
    inp = "".join(f"{p} {d}\n" for p, d in cases)
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.splitlines()
    assert len(out) == len(cases)
    for (n_pre, n_dec), line in zip(cases, out):
        fields = line.split()
        n = int(fields[0])
        roles = fields[1:]
        pg, dg = -(-n_pre // 8), -(-n_dec // 8)
        assert n == 8 * (pg + dg) == len(roles)
        pre = [(x, int(r[1:])) for x, r in enumerate(roles) if r[0] == "p"]
        dec = [(x, int(r[1:])) for x, r in enumerate(roles) if r[0] == "d"]
        assert [i for _, i in pre] == list(range(8 * pg)), (n_pre, n_dec)
        assert [i for _, i in dec] == list(range(8 * dg)), (n_pre, n_dec)
        assert all(x % 8 == i % 8 for x, i in pre + dec)
        assert "".join(r[0] for r in roles[::8]) == "d" * dg + "p" * pg
