import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_sessionstart(session):
    """The tests load the in-tree libdap.so as built; when none is built yet
    (a fresh checkout), build it once before anything loads it."""
    lib = os.path.join(ROOT, "decoder_attention_paged_amd", "libdap.so")
    if not os.path.exists(lib):
        from decoder_attention_paged_amd.build import build
        build(verbose=False)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")
    config.addinivalue_line("markers", "slow: larger CPU oracle cases")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """Bit-exactness report: elements the oracle flagged as near a bf16
    rounding midpoint, and how many of them the GPU rounded the other way."""
    parity = sys.modules.get("parity")
    rep = getattr(parity, "TIE_REPORT", None)
    if not rep:
        return
    n = sum(r[1] for r in rep)
    flagged = sum(r[2] for r in rep)
    diff = sum(r[3] for r in rep)
    terminalreporter.write_line(f"bit-exact checks: {len(rep)} calls, {n} rounded elements, {flagged} flagged "
                                f"near-ties, {diff} differing (all of them flagged)")
