"""The decode's split plan (decode_plan.h), compiled for the host with g++,
over extreme (window, max_position, rows) triples: every plan must fit the
kernel's LDS arrays (at most 256 pages per chunk and 256 chunks per row),
and its chunks must cover the most pages any row can attend, counted by
brute force over every position."""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
MAX_POSITION = 1 << 22


def _most_pages(window, max_position):
    p = np.arange(max_position, dtype=np.int64)
    lo = np.maximum(0, p - window + 1) if window > 0 else np.zeros_like(p)
    return int(((p >> 6) - (lo >> 6) + 1).max())


def test_decode_plan_fits_the_kernel_at_extremes(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "plan"
    subprocess.run([gxx, "-std=c++17", "-O1", os.path.join(HERE, "host", "decode_plan_host.cpp"), "-o", str(exe)],
                   check=True)
    windows = [0, 1, 63, 64, 65, 2047, 4096, 65535, MAX_POSITION - 65, MAX_POSITION - 1, MAX_POSITION,
               MAX_POSITION + 1000]
    positions = [1, 63, 64, 65, 4096, 40960, 65536, 1 << 20, MAX_POSITION - 1, MAX_POSITION]
    rows = [1, 64, 65535]
    cases = [(n, 32, 8, 128, w, mp) for w in windows for mp in positions for n in rows]
    cases += [(n, 16, 1, 64, w, MAX_POSITION) for w in (0, MAX_POSITION - 1, MAX_POSITION) for n in rows]
    cases = [c for c in cases if c[4] <= 2 ** 31 - 1]
    inp = "".join(" ".join(map(str, c)) + "\n" for c in cases)
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    most = {}
    for c, line in zip(cases, out):
        pps, splits, ws = (int(x) for x in line.split())
        n, hq, hkv, d, w, mp = c
        assert 4 <= pps <= 256 and 1 <= splits <= 256, (c, pps, splits)
        key = (w, mp)
        if key not in most:
            most[key] = _most_pages(w, mp)
        assert pps * splits >= most[key] and (splits - 1) * pps < most[key], (c, pps, splits, most[key])
        assert ws == n * hq * splits * (d + 2) * 4
