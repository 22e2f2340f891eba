"""Python binding of libdap.so, the paged decoder-attention core for MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. torch tensors supply device memory and the current HIP stream. The
functions mirror the C ABI in include/dap.h; bf16 tensors may be
torch.bfloat16 or int16 (bit patterns), index tensors are int32, and all of
them live on the GPU the handle was created on.

There is no fallback: importing works anywhere, but creating a handle needs
the built library and a GPU, and fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdap.so")

OK, INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP_ERROR, BAD_INDEX = 0, -1, -2, -3, -4, -5

EXPORTS = ("dap_create", "dap_destroy", "dap_last_error", "dap_set_validate", "dap_inv_freq",
           "dap_rope_qknorm_write_pages", "dap_prefill_workspace_bytes", "dap_attn_prefill_packed",
           "dap_decode_workspace_bytes", "dap_attn_decode_paged", "dap_attn_decode_paged_noalloc",
           "dap_step_workspace_bytes",
           "dap_step_paged", "dap_set_profiling", "dap_profile_read", "dap_cache_workspace_bytes",
           "dap_decode", "dap_decode_rows", "dap_prefill", "dap_prefill_slots", "dap_inpass_workspace_bytes",
           "dap_packed", "dap_forward", "dap_tile_layout")

KERNELS = ("write", "prefill_tiles", "prefill", "decode", "decode_merge", "prep", "step")


class DapError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dap status {status}: {message}")
        self.status = status


class _Model(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("window", ctypes.c_int32), ("max_position", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("llama3", ctypes.c_int32),
                ("llama3_factor", ctypes.c_double), ("llama3_low_freq_factor", ctypes.c_double),
                ("llama3_high_freq_factor", ctypes.c_double),
                ("llama3_original_max_position", ctypes.c_double),
                ("qk_norm", ctypes.c_int32), ("qk_norm_eps", ctypes.c_double)]


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


def load_library(path: str = LIB_PATH):
    """Load libdap.so and declare its signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with "
                                "`python -m decoder_attention_paged_amd.build`")
    lib = ctypes.CDLL(path)
    lib.dap_create.argtypes = [ctypes.POINTER(_Model), ctypes.POINTER(_P)]
    lib.dap_create.restype = ctypes.c_int
    lib.dap_destroy.argtypes = [_P]
    lib.dap_destroy.restype = None
    lib.dap_last_error.argtypes = []
    lib.dap_last_error.restype = ctypes.c_char_p
    lib.dap_set_validate.argtypes = [_P, ctypes.c_int]
    lib.dap_inv_freq.argtypes = [_P, ctypes.POINTER(ctypes.c_double), _I32]
    lib.dap_rope_qknorm_write_pages.argtypes = [
        _P, _P, _P, _P, _I64, _I32, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _I64, _P, _P, _I32, _P]
    lib.dap_prefill_workspace_bytes.argtypes = [_P, _I32, _I32]
    lib.dap_prefill_workspace_bytes.restype = _SZ
    lib.dap_attn_prefill_packed.argtypes = [
        _P, _P, _I64, _I32, _P, _P, _I32, _P, _I32, _I32, _P, _P, _I32, _P, _I64, _P, _SZ, _P]
    lib.dap_decode_workspace_bytes.argtypes = [_P, _I32]
    lib.dap_decode_workspace_bytes.restype = _SZ
    lib.dap_attn_decode_paged.argtypes = [
        _P, _P, _I64, _I32, _P, _P, _P, _I32, _I32, _P, _P, _I32, _P, _I64, _P, _SZ, _P]
    lib.dap_attn_decode_paged_noalloc.argtypes = [
        _P, _P, _I64, _I32, _P, _P, _P, _I32, _I32, _P, _P, _I32, _P, _I64, _P]
    lib.dap_step_workspace_bytes.argtypes = [_P, _I32, _I32, _I32]
    lib.dap_step_workspace_bytes.restype = _SZ
    lib.dap_step_paged.argtypes = [
        _P, _P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _I64,
        _P, _P, _I32, _P, _I64, _P, _SZ, _P]
    lib.dap_cache_workspace_bytes.argtypes = [_P, _I32, _I32, _I32, _I32]
    lib.dap_cache_workspace_bytes.restype = _SZ
    lib.dap_decode.argtypes = [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _I64, _P, _SZ, _P]
    lib.dap_decode_rows.argtypes = [_P, _P, _P, _P, _I64, _I32, _P, _I32, _P, _P, _P, _P, _P, _I64, _P, _SZ, _P]
    lib.dap_prefill.argtypes = [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _I64, _P, _SZ,
                                _P]
    lib.dap_prefill_slots.argtypes = [_P, _P, _P, _P, _I64, _I32, _I32, _P, _I32, _I32, _P, _P, _P, _P, _P, _I64,
                                      _P, _SZ, _P]
    lib.dap_inpass_workspace_bytes.argtypes = [_P, _I32, _I32]
    lib.dap_inpass_workspace_bytes.restype = _SZ
    lib.dap_packed.argtypes = [_P, _P, _P, _P, _I64, _I32, _P, _P, _I32, _P, _P, _P, _I64, _P, _SZ, _P]
    lib.dap_forward.argtypes = [_P, _P, _P, _P, _I64, _I32, _I32, _P, _P, _P, _I64, _P, _SZ, _P]
    lib.dap_tile_layout.argtypes = [_I32, _P, _P]
    lib.dap_set_profiling.argtypes = [_P, ctypes.c_int]
    lib.dap_profile_read.argtypes = [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                     ctypes.c_int]
    _lib = lib
    return lib


def _check(status: int):
    if status != OK:
        raise DapError(status, _lib.dap_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# Extents the C side cannot see: it receives pointers and the sizes derived
# here, so a short or misplaced tensor is refused before any kernel reads it.
def _need(cond: bool, msg: str):
    if not cond:
        raise DapError(INVALID_ARG, msg)


def _on_gpu(name: str, t: torch.Tensor):
    _need(t.is_cuda, f"{name} must be a GPU tensor")


def _mat(name: str, t: Optional[torch.Tensor], n: int, width: int):
    """A 2-D GPU tensor with at least n rows of at least width columns."""
    if t is None:
        return
    _on_gpu(name, t)
    _need(t.dim() == 2 and t.shape[0] >= n and t.shape[1] >= width,
          f"{name}: expected at least [{n}, {width}], got {list(t.shape)}")


def _vec(name: str, t: Optional[torch.Tensor], n: int):
    """A 1-D GPU tensor with at least n entries."""
    if t is None:
        return
    _on_gpu(name, t)
    _need(t.dim() == 1 and t.shape[0] >= n, f"{name}: expected at least {n} entries, got {list(t.shape)}")


def _pools(m: "Model", k_pool: torch.Tensor, v_pool: torch.Tensor, min_pages: int = 1):
    """Contiguous [n_pages, Hkv, 64 * D] pools of the same size."""
    per_page = m.n_kv_heads * m.page_size * m.head_dim
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        _on_gpu(name, t)
        _need(t.dim() >= 1 and t.is_contiguous() and t.shape[0] >= min_pages and t.numel() == t.shape[0] * per_page,
              f"{name}: expected a contiguous [n_pages >= {min_pages}, {m.n_kv_heads}, {m.page_size * m.head_dim}] "
              f"pool, got {list(t.shape)}")
    _need(k_pool.shape[0] == v_pool.shape[0], "k_pool and v_pool must hold the same number of pages")


def _table(t: Optional[torch.Tensor]):
    if t is not None:
        _on_gpu("table", t)
        _need(t.dim() == 2, f"table: expected [rows, table_ld], got {list(t.shape)}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _bf16(t: Optional[torch.Tensor]):
    if t is not None and t.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError("bf16 tensors must be torch.bfloat16 or int16 bit patterns")
    return t


def _i32(t: Optional[torch.Tensor]):
    if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
        raise TypeError("index tensors must be contiguous int32")
    return t


@dataclass
class Model:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_theta: float
    window: int = 0
    max_position: int = 4096
    llama3: Optional[tuple] = None          # (factor, low_freq_factor, high_freq_factor, original)
    qk_norm_eps: Optional[float] = None     # None: no QK-norm
    page_size: int = 64


class Handle:
    """A dap_handle: model constants plus the device frequency table."""

    def __init__(self, model: Model, validate: bool = False):
        lib = load_library()
        m = _Model()
        m.n_q_heads, m.n_kv_heads, m.head_dim = model.n_q_heads, model.n_kv_heads, model.head_dim
        m.page_size, m.window, m.max_position = model.page_size, model.window, model.max_position
        m.rope_theta = float(model.rope_theta)
        if model.llama3 is not None:
            m.llama3 = 1
            (m.llama3_factor, m.llama3_low_freq_factor, m.llama3_high_freq_factor,
             m.llama3_original_max_position) = (float(x) for x in model.llama3)
        if model.qk_norm_eps is not None:
            m.qk_norm, m.qk_norm_eps = 1, float(model.qk_norm_eps)
        h = ctypes.c_void_p()
        _check(lib.dap_create(ctypes.byref(m), ctypes.byref(h)))
        self._h = h
        self.model = model
        if validate:
            self.set_validate(True)

    def close(self):
        if getattr(self, "_h", None):
            _lib.dap_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_validate(self, on: bool):
        _check(_lib.dap_set_validate(self._h, int(bool(on))))

    def set_profiling(self, on: bool):
        """Bracket every kernel launch with timing events (measurement only)."""
        _check(_lib.dap_set_profiling(self._h, int(bool(on))))

    def profile_read(self, reset: bool = True) -> dict:
        """{kernel: (total_ms, launches)} since the last reset; waits for pending events."""
        ms = (ctypes.c_double * len(KERNELS))()
        n = (ctypes.c_int64 * len(KERNELS))()
        _check(_lib.dap_profile_read(self._h, ms, n, int(bool(reset))))
        return {k: (ms[i], int(n[i])) for i, k in enumerate(KERNELS)}

    def inv_freq(self) -> torch.Tensor:
        n = self.model.head_dim // 2
        buf = (ctypes.c_double * n)()
        _check(_lib.dap_inv_freq(self._h, buf, n))
        return torch.tensor(list(buf), dtype=torch.float64)

    # ------------------------------------------------------------ workspaces
    def prefill_workspace_bytes(self, n_tokens: int, n_segments: int) -> int:
        return int(_lib.dap_prefill_workspace_bytes(self._h, n_tokens, n_segments))

    def decode_workspace_bytes(self, n_rows: int) -> int:
        return int(_lib.dap_decode_workspace_bytes(self._h, n_rows))

    def step_workspace_bytes(self, n_prompt: int, n_segments: int, n_step: int) -> int:
        return int(_lib.dap_step_workspace_bytes(self._h, n_prompt, n_segments, n_step))

    @staticmethod
    def _workspace(ws, nbytes, like):
        """A caller-kept workspace is reused as is (its contents do not
        matter); otherwise one is allocated for this call."""
        if ws is None:
            ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=like.device)
        _on_gpu("workspace", ws)
        return ws

    def workspace(self, nbytes: int, device="cuda") -> torch.Tensor:
        """A zero-filled workspace to keep across calls."""
        return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)

    # ------------------------------------------------------------ entries
    def rope_qknorm_write_pages(self, q, k, v, positions, k_pool, v_pool, *, rows=None, slots=None,
                                table=None, q_out=None, q_gain=None, k_gain=None, stream=None):
        """q, k, v: [T, width] views sharing one row stride (e.g. column slices
        of the fused qkv). Returns q_out [T, Hq*D]."""
        m = self.model
        T = positions.shape[0]
        if q_out is None:
            q_out = torch.empty(T, m.n_q_heads * m.head_dim, dtype=q.dtype, device=q.device)
        self._check_tokens(T, q, k, v, positions, (rows, slots), q_gain, k_gain, q_out, k_pool, v_pool, table)
        ld = _ld(q)
        if _ld(k) != ld or _ld(v) != ld:
            raise ValueError("q, k and v must share one row stride")
        tld, trows = (table.shape[1], table.shape[0]) if table is not None else (0, 0)
        _check(_lib.dap_rope_qknorm_write_pages(
            self._h, _ptr(_bf16(q)), _ptr(_bf16(k)), _ptr(_bf16(v)), ld, T, _ptr(_i32(positions)),
            _ptr(_i32(rows)), _ptr(_i32(slots)), _ptr(_i32(table)), tld, trows,
            _ptr(_bf16(q_gain)), _ptr(_bf16(k_gain)), _ptr(_bf16(q_out)), _ld(q_out),
            _ptr(_bf16(k_pool)), _ptr(_bf16(v_pool)), k_pool.shape[0], _stream(stream)))
        return q_out

    def attn_prefill_packed(self, q, positions, segments, table, k_pool, v_pool, *, n_segments=None,
                            out=None, workspace=None, stream=None):
        """q: [T, Hq*D] roped queries; segments[t] = table row of token t."""
        m = self.model
        T = positions.shape[0]
        if n_segments is None:
            n_segments = T
        if out is None:
            out = torch.empty(T, m.n_q_heads * m.head_dim, dtype=q.dtype, device=q.device)
        self._check_attn(T, q, positions, segments, out, k_pool, v_pool, table)
        nb = self.prefill_workspace_bytes(T, n_segments)
        ws = self._workspace(workspace, nb, q)
        _check(_lib.dap_attn_prefill_packed(
            self._h, _ptr(_bf16(q)), _ld(q), T, _ptr(_i32(positions)), _ptr(_i32(segments)), n_segments,
            _ptr(_i32(table)), table.shape[1], table.shape[0], _ptr(_bf16(k_pool)), _ptr(_bf16(v_pool)),
            k_pool.shape[0], _ptr(_bf16(out)), _ld(out), _ptr(ws), ws.numel(), _stream(stream)))
        return out

    def attn_decode_paged(self, q, positions, table, k_pool, v_pool, *, rows=None, out=None,
                          workspace=None, stream=None):
        """q: [R, Hq*D] roped queries, one per row; row b uses table row rows[b] (or b)."""
        m = self.model
        R = positions.shape[0]
        if out is None:
            out = torch.empty(R, m.n_q_heads * m.head_dim, dtype=q.dtype, device=q.device)
        self._check_attn(R, q, positions, rows, out, k_pool, v_pool, table)
        nb = self.decode_workspace_bytes(R)
        ws = self._workspace(workspace, nb, q)
        _check(_lib.dap_attn_decode_paged(
            self._h, _ptr(_bf16(q)), _ld(q), R, _ptr(_i32(positions)), _ptr(_i32(rows)),
            _ptr(_i32(table)), table.shape[1], table.shape[0], _ptr(_bf16(k_pool)), _ptr(_bf16(v_pool)),
            k_pool.shape[0], _ptr(_bf16(out)), _ld(out), _ptr(ws), ws.numel(), _stream(stream)))
        return out

    def attn_decode_paged_noalloc(self, q, positions, table, k_pool, v_pool, *, out, rows=None, stream=None):
        """attn_decode_paged with no workspace: the library's static device
        scratch holds the partials. ``out`` is required (nothing is allocated)."""
        R = positions.shape[0]
        self._check_attn(R, q, positions, rows, out, k_pool, v_pool, table)
        _check(_lib.dap_attn_decode_paged_noalloc(
            self._h, _ptr(_bf16(q)), _ld(q), R, _ptr(_i32(positions)), _ptr(_i32(rows)),
            _ptr(_i32(table)), table.shape[1], table.shape[0], _ptr(_bf16(k_pool)), _ptr(_bf16(v_pool)),
            k_pool.shape[0], _ptr(_bf16(out)), _ld(out), _stream(stream)))
        return out

    def step_paged(self, q, k, v, positions, rows, table, k_pool, v_pool, *, n_prompt, n_segments,
                   slots=None, q_gain=None, k_gain=None, q_out=None, out=None, workspace=None, stream=None):
        """All tokens written, then prompts (tokens < n_prompt) prefill and the
        rest decode. Returns (q_out, out)."""
        m = self.model
        T = positions.shape[0]
        n_step = T - n_prompt
        if q_out is None:
            q_out = torch.empty(T, m.n_q_heads * m.head_dim, dtype=q.dtype, device=q.device)
        if out is None:
            out = torch.empty(T, m.n_q_heads * m.head_dim, dtype=q.dtype, device=q.device)
        self._check_tokens(T, q, k, v, positions, (rows, slots), q_gain, k_gain, q_out, k_pool, v_pool, table)
        _mat("out", out, T, m.n_q_heads * m.head_dim)
        nb = self.step_workspace_bytes(n_prompt, n_segments, n_step)
        ws = self._workspace(workspace, nb, q)
        ld = _ld(q)
        if _ld(k) != ld or _ld(v) != ld:
            raise ValueError("q, k and v must share one row stride")
        _check(_lib.dap_step_paged(
            self._h, _ptr(_bf16(q)), _ptr(_bf16(k)), _ptr(_bf16(v)), ld, n_prompt, n_segments, n_step,
            _ptr(_i32(positions)), _ptr(_i32(rows)), _ptr(_i32(slots)), _ptr(_i32(table)),
            table.shape[1], table.shape[0], _ptr(_bf16(q_gain)), _ptr(_bf16(k_gain)),
            _ptr(_bf16(q_out)), _ld(q_out), _ptr(_bf16(k_pool)), _ptr(_bf16(v_pool)), k_pool.shape[0],
            _ptr(_bf16(out)), _ld(out), _ptr(ws), ws.numel(), _stream(stream)))
        return q_out, out

    # ------------------------------------------------------------ contiguous-cache entries
    def cache_workspace_bytes(self, n_tokens: int, n_groups: int, cache_rows: int, max_seq: int) -> int:
        return int(_lib.dap_cache_workspace_bytes(self._h, n_tokens, n_groups, cache_rows, max_seq))

    def _check_tokens(self, T, q, k, v, positions, index_arrays, q_gain, k_gain, q_out, k_pool=None, v_pool=None,
                      table=None, min_pages=1):
        m = self.model
        _vec("positions", positions, T)
        _mat("q", q, T, m.n_q_heads * m.head_dim)
        _mat("k", k, T, m.n_kv_heads * m.head_dim)
        _mat("v", v, T, m.n_kv_heads * m.head_dim)
        for t in index_arrays:
            _vec("rows/slots/segments", t, T)
        _vec("q_gain", q_gain, m.head_dim)
        _vec("k_gain", k_gain, m.head_dim)
        _mat("q_out/out", q_out, T, m.n_q_heads * m.head_dim)
        if k_pool is not None:
            _pools(m, k_pool, v_pool, min_pages)
        _table(table)

    def _check_attn(self, T, q, positions, index, out, k_pool, v_pool, table):
        m = self.model
        _vec("positions", positions, T)
        _mat("q", q, T, m.n_q_heads * m.head_dim)
        _vec("rows/segments", index, T)
        _mat("out", out, T, m.n_q_heads * m.head_dim)
        _pools(m, k_pool, v_pool)
        _table(table)

    def _cache_pages(self, cache_rows, max_seq):
        return -(-cache_rows * max_seq // self.model.page_size)

    def _qkv(self, q, k, v):
        ld = _ld(q)
        if _ld(k) != ld or _ld(v) != ld:
            raise ValueError("q, k and v must share one row stride")
        return _ptr(_bf16(q)), _ptr(_bf16(k)), _ptr(_bf16(v)), ld

    def _out(self, out, n, like):
        m = self.model
        return torch.empty(n, m.n_q_heads * m.head_dim, dtype=like.dtype, device=like.device) if out is None else out

    def decode(self, q, k, v, pos: int, k_pool, v_pool, *, max_seq, q_gain=None, k_gain=None, out=None,
               workspace=None, stream=None):
        """One token per cache row, all at position pos. The cache: pools of
        cache_rows * max_seq / 64 pages, row r owning pages r*max_seq/64 onward."""
        R = q.shape[0]
        out = self._out(out, R, q)
        self._check_tokens(R, q, k, v, None, (), q_gain, k_gain, out, k_pool, v_pool,
                           min_pages=self._cache_pages(R, max_seq))
        ws = self._workspace(workspace, self.cache_workspace_bytes(R, 1, R, max_seq), q)
        _check(_lib.dap_decode(self._h, *self._qkv(q, k, v), R, pos, max_seq, _ptr(_bf16(q_gain)),
                               _ptr(_bf16(k_gain)), _ptr(_bf16(k_pool)), _ptr(_bf16(v_pool)), _ptr(_bf16(out)),
                               _ld(out), _ptr(ws), ws.numel(), _stream(stream)))
        return out

    def decode_rows(self, q, k, v, positions, k_pool, v_pool, *, max_seq, q_gain=None, k_gain=None, out=None,
                    workspace=None, stream=None):
        """One token per cache row, row b at positions[b]."""
        R = q.shape[0]
        out = self._out(out, R, q)
        self._check_tokens(R, q, k, v, positions, (), q_gain, k_gain, out, k_pool, v_pool,
                           min_pages=self._cache_pages(R, max_seq))
        ws = self._workspace(workspace, self.cache_workspace_bytes(R, 1, R, max_seq), q)
        _check(_lib.dap_decode_rows(self._h, *self._qkv(q, k, v), R, _ptr(_i32(positions)), max_seq,
                                    _ptr(_bf16(q_gain)), _ptr(_bf16(k_gain)), _ptr(_bf16(k_pool)),
                                    _ptr(_bf16(v_pool)), _ptr(_bf16(out)), _ld(out), _ptr(ws), ws.numel(),
                                    _stream(stream)))
        return out

    def prefill(self, q, k, v, pos: int, k_pool, v_pool, *, cache_rows, max_seq, q_gain=None, k_gain=None,
                out=None, workspace=None, stream=None):
        """cache_rows * seq tokens: token b*seq+i is row b at position pos+i."""
        T = q.shape[0]
        seq = T // cache_rows
        out = self._out(out, T, q)
        self._check_tokens(T, q, k, v, None, (), q_gain, k_gain, out, k_pool, v_pool,
                           min_pages=self._cache_pages(cache_rows, max_seq))
        ws = self._workspace(workspace, self.cache_workspace_bytes(T, cache_rows, cache_rows, max_seq), q)
        _check(_lib.dap_prefill(self._h, *self._qkv(q, k, v), cache_rows, seq, pos, max_seq, _ptr(_bf16(q_gain)),
                                _ptr(_bf16(k_gain)), _ptr(_bf16(k_pool)), _ptr(_bf16(v_pool)), _ptr(_bf16(out)),
                                _ld(out), _ptr(ws), ws.numel(), _stream(stream)))
        return out

    def prefill_slots(self, q, k, v, slots, k_pool, v_pool, *, cache_rows, max_seq, q_gain=None, k_gain=None,
                      out=None, workspace=None, stream=None):
        """len(slots) prompts of seq tokens: token m*seq+i is row slots[m] at position i."""
        T = q.shape[0]
        M = slots.shape[0]
        out = self._out(out, T, q)
        self._check_tokens(T, q, k, v, None, (), q_gain, k_gain, out, k_pool, v_pool,
                           min_pages=self._cache_pages(cache_rows, max_seq))
        _vec("slots", slots, M)
        ws = self._workspace(workspace, self.cache_workspace_bytes(T, M, cache_rows, max_seq), q)
        _check(_lib.dap_prefill_slots(self._h, *self._qkv(q, k, v), M, T // M, _ptr(_i32(slots)), cache_rows,
                                      max_seq, _ptr(_bf16(q_gain)), _ptr(_bf16(k_gain)), _ptr(_bf16(k_pool)),
                                      _ptr(_bf16(v_pool)), _ptr(_bf16(out)), _ld(out), _ptr(ws), ws.numel(),
                                      _stream(stream)))
        return out

    # ------------------------------------------------------------ in-pass entries (no cache)
    def inpass_workspace_bytes(self, n_tokens: int, n_segments: int) -> int:
        return int(_lib.dap_inpass_workspace_bytes(self._h, n_tokens, n_segments))

    def packed(self, q, k, v, positions, segments, *, n_segments, q_gain=None, k_gain=None, out=None,
               workspace=None, stream=None):
        """Attention among the call's tokens: same segment, earlier or equal position."""
        T = positions.shape[0]
        out = self._out(out, T, q)
        self._check_tokens(T, q, k, v, positions, (segments,), q_gain, k_gain, out)
        ws = self._workspace(workspace, self.inpass_workspace_bytes(T, n_segments), q)
        _check(_lib.dap_packed(self._h, *self._qkv(q, k, v), T, _ptr(_i32(positions)), _ptr(_i32(segments)),
                               n_segments, _ptr(_bf16(q_gain)), _ptr(_bf16(k_gain)), _ptr(_bf16(out)), _ld(out),
                               _ptr(ws), ws.numel(), _stream(stream)))
        return out

    def forward(self, q, k, v, n_seqs: int, *, q_gain=None, k_gain=None, out=None, workspace=None, stream=None):
        """n_seqs sequences of T/n_seqs tokens from position 0, no cache."""
        T = q.shape[0]
        out = self._out(out, T, q)
        self._check_tokens(T, q, k, v, None, (), q_gain, k_gain, out)
        ws = self._workspace(workspace, self.inpass_workspace_bytes(T, n_seqs), q)
        _check(_lib.dap_forward(self._h, *self._qkv(q, k, v), n_seqs, T // n_seqs, _ptr(_bf16(q_gain)),
                                _ptr(_bf16(k_gain)), _ptr(_bf16(out)), _ld(out), _ptr(ws), ws.numel(),
                                _stream(stream)))
        return out


_TILE_CACHE = {}


def tile_offsets(head_dim: int, device="cpu"):
    """Element offsets of logical K (key, d) and V (key, d) inside one page
    tile, as two [64, D] int64 tensors, from the library (dap_tile_layout)."""
    key = (head_dim, str(device))
    if key not in _TILE_CACHE:
        lib = load_library()
        k = (ctypes.c_int32 * (64 * head_dim))()
        v = (ctypes.c_int32 * (64 * head_dim))()
        _check(lib.dap_tile_layout(head_dim, k, v))
        kt = torch.tensor(list(k), dtype=torch.int64).view(64, head_dim)
        vt = torch.tensor(list(v), dtype=torch.int64).view(64, head_dim)
        _TILE_CACHE[key] = (kt.to(device), vt.to(device))
    return _TILE_CACHE[key]


def pools(n_pages: int, n_kv_heads: int, head_dim: int, device="cuda", dtype=torch.bfloat16):
    """Uninitialised K and V pools: [n_pages, Hkv, 64 * D] each, one tile per
    (page, kv head) in the library's tile layout. Slots no query attends may
    hold anything (include/dap.h, stale slots). Use store_pages /
    pool_logical / gather_slots to move logical [.., 64, D] contents in and
    out."""
    k = torch.empty(n_pages, n_kv_heads, 64 * head_dim, dtype=dtype, device=device)
    v = torch.empty(n_pages, n_kv_heads, 64 * head_dim, dtype=dtype, device=device)
    return k, v


def store_pages(k_pool, v_pool, page_ids, k_logical, v_logical):
    """Place logical page contents [n, Hkv, 64, D] (key-major K and V) into
    the pools' tile layout."""
    n, hkv, _, D = k_logical.shape
    koff, voff = tile_offsets(D, k_pool.device)
    idx = torch.as_tensor(page_ids, dtype=torch.long, device=k_pool.device)
    kt = torch.empty(n, hkv, 64 * D, dtype=k_pool.dtype, device=k_pool.device)
    vt = torch.empty_like(kt)
    kt[:, :, koff.reshape(-1)] = k_logical.view(k_pool.dtype).reshape(n, hkv, 64 * D)
    vt[:, :, voff.reshape(-1)] = v_logical.view(v_pool.dtype).reshape(n, hkv, 64 * D)
    k_pool[idx] = kt
    v_pool[idx] = vt


def pool_logical(k_pool, v_pool, page_ids=None):
    """Logical contents [n, Hkv, 64, D] of K and V pages (all pages if None)."""
    D = k_pool.shape[-1] // 64
    koff, voff = tile_offsets(D, k_pool.device)
    kp = k_pool if page_ids is None else k_pool[torch.as_tensor(page_ids, dtype=torch.long, device=k_pool.device)]
    vp = v_pool if page_ids is None else v_pool[torch.as_tensor(page_ids, dtype=torch.long, device=v_pool.device)]
    n, hkv = kp.shape[0], kp.shape[1]
    return (kp[:, :, koff.reshape(-1)].reshape(n, hkv, 64, D), vp[:, :, voff.reshape(-1)].reshape(n, hkv, 64, D))


def gather_slots(k_pool, v_pool, slots):
    """Logical K and V at pool slots: two [T, Hkv, D] tensors."""
    D = k_pool.shape[-1] // 64
    koff, voff = tile_offsets(D, k_pool.device)
    s = torch.as_tensor(slots, dtype=torch.long, device=k_pool.device)
    pg, i = s // 64, s % 64
    hkv = k_pool.shape[1]
    kidx = koff[i].unsqueeze(1).expand(len(s), hkv, D)
    vidx = voff[i].unsqueeze(1).expand(len(s), hkv, D)
    return torch.gather(k_pool[pg], 2, kidx), torch.gather(v_pool[pg], 2, vidx)
