"""dap_attn_decode_paged_noalloc: the decode with its partials in the
library's static device scratch instead of a caller workspace.

Two calls in a row through the C ABI, the second with fewer rows (so it
runs over what the first left in the scratch), each compared bit for bit
with dap_attn_decode_paged on the same inputs (the same kernels and the
same chunking run under both) and against the fp64 oracle; a call whose
partials would not fit is refused with DAP_WORKSPACE_TOO_SMALL and leaves
its output untouched."""
import zlib

import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import attention, bf16

from parity import OraclePool, check_close, device_pools, handle_for, to_np_bits, torch_i32

pytestmark = pytest.mark.gpu


def _case(model, n_rows, ppr, tag):
    rng = np.random.default_rng(zlib.crc32(tag.encode()))
    perm = rng.permutation(n_rows * ppr).astype(np.int32)
    return W.Workload(tag, model, n_rows * ppr, perm.reshape(n_rows, ppr)), rng


def test_noalloc_decode_matches_the_workspace_decode_twice():
    model = W.ModelShape("noalloc", 32, 8, 128, 1e6, max_position=8192)
    wl, rng = _case(model, 48, 128, "noalloc")
    kp, vp = device_pools(wl)
    h = handle_for(model)
    table = torch_i32(wl.table)
    op = OraclePool(wl, "cuda")
    width = model.n_q_heads * model.head_dim
    # first call: 48 rows over 1-128 pages (several chunks each); second: 5 rows
    for n, tag in ((48, "first"), (5, "second")):
        rows = rng.permutation(48)[:n].astype(np.int32)
        positions = rng.integers(0, 8192, n).astype(np.int32)
        positions[0] = 8191
        q = W.normal_matrix(wl.key("q", tag), n, width, "cuda")
        out = torch.empty(n, width, dtype=torch.int16, device="cuda")
        h.attn_decode_paged_noalloc(q, torch_i32(positions), table, kp, vp, out=out, rows=torch_i32(rows))
        ref_ws = h.attn_decode_paged(q, torch_i32(positions), table, kp, vp, rows=torch_i32(rows))
        torch.cuda.synchronize()
        assert torch.equal(out, ref_ws.view(torch.int16)), f"{tag} call differs from the workspace decode"
        ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(n, 32, 128), positions, rows, wl.table,
                              op.read_page, 0)
        check_close(to_np_bits(out), ref, f"no-alloc decode, {tag} call ({n} rows)")


def test_noalloc_decode_refuses_partials_beyond_its_scratch():
    # 8 rows at max_position 2^22: 256 chunks per row x 32 heads x 130 floats x 8 rows > 32 MiB
    model = W.ModelShape("noalloc-big", 32, 8, 128, 1e6, max_position=1 << 22)
    wl, _ = _case(model, 1, 4, "noalloc-big")
    kp, vp = device_pools(wl)
    h = handle_for(model)
    assert h.decode_workspace_bytes(8) > 32 << 20 and h.decode_workspace_bytes(7) <= 32 << 20
    q = W.normal_matrix(wl.key("q"), 8, 32 * 128, "cuda")
    out = torch.full((8, 32 * 128), 0x5A5A, dtype=torch.int16, device="cuda")
    pos = torch_i32(np.arange(8, dtype=np.int32))
    rows = torch_i32(np.zeros(8, np.int32))
    with pytest.raises(dap.DapError) as e:
        h.attn_decode_paged_noalloc(q, pos, torch_i32(wl.table), kp, vp, out=out, rows=rows)
    assert e.value.status == dap.WORKSPACE_TOO_SMALL and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 0x5A5A).all()), "a refused call wrote its output"
    # 7 rows fit and run
    out7 = h.attn_decode_paged_noalloc(q[:7], pos[:7], torch_i32(wl.table), kp, vp, out=out[:7], rows=rows[:7])
    ref7 = h.attn_decode_paged(q[:7], pos[:7], torch_i32(wl.table), kp, vp, rows=rows[:7])
    torch.cuda.synchronize()
    assert torch.equal(out7, ref7.view(torch.int16))
