"""Python binding of libkvc.so, the gfx950 paged-KV ragged attention library.

Argument marshalling only: every function below checks tensor dtypes, devices
and contiguity, derives the sizes the C ABI wants from the tensor shapes, and
calls the entry point of the same name in ``libkvc.so``.  All device work runs
in the library's HIP kernels; there is no fallback path.  If the library has
not been built, importing this package raises ``ImportError``.

Tensor layouts follow ``include/kvc.h``:
  q, out [total_q, Hq, A] bf16;  k_new, v_new [total_q, Hkv, A] bf16;
  k_cache, v_cache [num_blocks, Hkv, block_size, A] bf16;
  block_table [S, max_blocks] int32;  cu_seqlens_q [S+1] int32;
  context_lens [S] int32 (tokens cached before the call).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python batching_kv_append_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_lib_status_string = _sig("kvc_status_string", ctypes.c_char_p, [ctypes.c_int])
_lib_last_error = _sig("kvc_last_error", ctypes.c_char_p, [])
_sig("kvc_allocator_create", ctypes.c_int, [_I32, _I32, ctypes.POINTER(_P)])
_sig("kvc_allocator_destroy", None, [_P])
_sig("kvc_alloc_blocks", ctypes.c_int, [_P, _I32, _P])
_sig("kvc_share_blocks", ctypes.c_int, [_P, _P, _I32])
_sig("kvc_free_blocks", ctypes.c_int, [_P, _P, _I32])
_sig("kvc_num_free_blocks", _I32, [_P])
_sig("kvc_num_blocks", _I32, [_P])
_sig("kvc_block_refcount", _I32, [_P, _I32])
_sig("kvc_extend_table", ctypes.c_int, [_P, _P, _I32, ctypes.POINTER(_I32), _I64])
_sig("kvc_extend_tables", ctypes.c_int, [_P, _P, _I32, _P, _P, _I32])
_sig("kvc_cache_bytes", _I64, [_I64, _I32, _I32, _I32, _I32])
_sig("kvc_allocator_block_size", _I32, [_P])
_sig("kvc_cow_block", ctypes.c_int, [_P, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)])
_sig("kvc_scheduler_create", ctypes.c_int, [_P, _I32, _I32, _I32, ctypes.POINTER(_P)])
_sig("kvc_scheduler_destroy", None, [_P])
_sig("kvc_scheduler_add", ctypes.c_int, [_P, _I64, _I32, _I32])
_sig("kvc_scheduler_step", ctypes.c_int,
     [_P, _P, _P, _P, _P, ctypes.POINTER(_I32), ctypes.POINTER(_I32), ctypes.POINTER(_I32),
      ctypes.POINTER(_I32)])
_sig("kvc_scheduler_complete", ctypes.c_int, [_P, _P, ctypes.POINTER(_I32)])
_sig("kvc_scheduler_num_waiting", _I32, [_P])
_sig("kvc_scheduler_num_running", _I32, [_P])
_sig("kvc_fork_table", ctypes.c_int,
     [_P, _P, _I64, _P, _I32, ctypes.POINTER(_I32), _P, _P, ctypes.POINTER(_I32)])
_sig("kvc_copy_blocks", ctypes.c_int, [_P, _P, _I64, _P, _P, _I32, _I32, _I32, _I32, _P])
_sig("kvc_append_kv", ctypes.c_int,
     [_P, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _P])
_sig("kvc_gather_kv", ctypes.c_int,
     [_P, _P, _I64, _P, _I32, _P, _P, _I64, _P, _P, _I32, _I32, _I32, _I32, _P])
_sig("kvc_workspace_size", _SZ, [_I32] * 8)
_sig("kvc_paged_attention_varlen", ctypes.c_int,
     [_P, _P, _P, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
      _I32, _I32, ctypes.c_float, _P, _SZ, _P])
_sig("kvc_paged_attention_varlen_noalloc", ctypes.c_int,
     [_P, _P, _P, _P, _P, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
      _I32, _I32, ctypes.c_float, _P])
_sig("kvc_workspace_flags", ctypes.c_int, [_P, _P, ctypes.POINTER(_I32)])
_sig("kvc_padded_workspace_size", _SZ, [_I32] * 6)
_sig("kvc_padded_decode_attention", ctypes.c_int,
     [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _SZ, _P])
_sig("kvc_profile_begin", ctypes.c_int, [_I32])
_sig("kvc_profile_end", ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I32)])

KVC_OK = 0
KVC_ERR_INVALID_ARG = -1
KVC_ERR_OOM = -2
KVC_ERR_UNSUPPORTED = -3
KVC_ERR_WORKSPACE = -4
KVC_ERR_HIP = -5
NOALLOC_SCRATCH_BYTES = 128 << 20  # KVC_NOALLOC_SCRATCH_BYTES of include/kvc.h

EXPORTED = [
    "kvc_status_string", "kvc_last_error", "kvc_allocator_create", "kvc_allocator_destroy",
    "kvc_alloc_blocks", "kvc_share_blocks", "kvc_free_blocks", "kvc_num_free_blocks",
    "kvc_num_blocks", "kvc_block_refcount", "kvc_extend_table", "kvc_extend_tables", "kvc_cache_bytes",
    "kvc_cow_block", "kvc_fork_table", "kvc_copy_blocks", "kvc_allocator_block_size",
    "kvc_scheduler_create", "kvc_scheduler_destroy", "kvc_scheduler_add", "kvc_scheduler_step",
    "kvc_scheduler_complete", "kvc_scheduler_num_waiting", "kvc_scheduler_num_running",
    "kvc_append_kv", "kvc_gather_kv", "kvc_workspace_size", "kvc_paged_attention_varlen",
    "kvc_paged_attention_varlen_noalloc", "kvc_workspace_flags",
    "kvc_padded_workspace_size", "kvc_padded_decode_attention", "kvc_profile_begin", "kvc_profile_end",
]

PROF_PHASES = ["plan", "append", "prefill", "decode", "merge"]


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = (_lib_last_error() or b"").decode(errors="replace")
        super().__init__(f"{where}: {kvc_status_string(status)} ({status}): {detail}")


def _check(status: int, where: str):
    if status != KVC_OK:
        raise KvcError(status, where)


def kvc_status_string(status: int) -> str:
    return _lib_status_string(status).decode()


def kvc_last_error() -> str:
    return (_lib_last_error() or b"").decode(errors="replace")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, ndim, name, cuda=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous():
        raise TypeError(f"{name}: expected a contiguous {dtype} tensor with {ndim} dims, got "
                        f"{t.dtype} {tuple(t.shape)}")
    if cuda and not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    return t


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


# --------------------------------------------------------------------------
# allocator (host)
# --------------------------------------------------------------------------
class Allocator:
    """Host block allocator (kvc_allocator_*): free list + reference counts."""

    def __init__(self, num_blocks: int, block_size: int):
        h = _P()
        _check(_lib.kvc_allocator_create(num_blocks, block_size, ctypes.byref(h)),
               "kvc_allocator_create")
        self._h = h
        self.block_size = block_size

    def close(self):
        if self._h:
            _lib.kvc_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h


def _ids(ids):
    import numpy as np
    a = np.ascontiguousarray(ids, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def kvc_alloc_blocks(alloc: Allocator, n: int):
    import numpy as np
    out = np.empty(max(n, 0), dtype=np.int32)
    _check(_lib.kvc_alloc_blocks(alloc.handle, n, out.ctypes.data_as(ctypes.c_void_p)),
           "kvc_alloc_blocks")
    return out


def kvc_share_blocks(alloc: Allocator, ids):
    a, p = _ids(ids)
    _check(_lib.kvc_share_blocks(alloc.handle, p, a.size), "kvc_share_blocks")


def kvc_free_blocks(alloc: Allocator, ids):
    a, p = _ids(ids)
    _check(_lib.kvc_free_blocks(alloc.handle, p, a.size), "kvc_free_blocks")


def kvc_num_free_blocks(alloc: Allocator) -> int:
    return int(_lib.kvc_num_free_blocks(alloc.handle))


def kvc_num_blocks(alloc: Allocator) -> int:
    return int(_lib.kvc_num_blocks(alloc.handle))


def kvc_block_refcount(alloc: Allocator, block_id: int) -> int:
    return int(_lib.kvc_block_refcount(alloc.handle, block_id))


def kvc_extend_table(alloc: Allocator, row, held: int, new_len: int) -> int:
    """Grow a host table row (int32 numpy array, modified in place) to cover
    new_len tokens; returns the new number of held blocks."""
    import numpy as np
    if not (isinstance(row, np.ndarray) and row.dtype == np.int32 and row.flags["C_CONTIGUOUS"]):
        raise TypeError("row: expected a C-contiguous int32 numpy array")
    h = _I32(held)
    _check(_lib.kvc_extend_table(alloc.handle, row.ctypes.data_as(ctypes.c_void_p), row.size,
                                 ctypes.byref(h), new_len), "kvc_extend_table")
    return int(h.value)


def kvc_extend_tables(alloc: Allocator, table, held, new_lens) -> None:
    """Grow every row of a host table ([S, max_blocks] int32, modified in
    place) to cover new_lens[s] tokens; held ([S] int32) is updated.  All or
    nothing."""
    import numpy as np
    for name, a, dt, nd in (("table", table, np.int32, 2), ("held", held, np.int32, 1),
                            ("new_lens", new_lens, np.int64, 1)):
        if not (isinstance(a, np.ndarray) and a.dtype == dt and a.ndim == nd
                and a.flags["C_CONTIGUOUS"]):
            raise TypeError(f"{name}: expected a C-contiguous {np.dtype(dt).name} numpy array "
                            f"with {nd} dims")
    s = table.shape[0]
    if held.shape[0] != s or new_lens.shape[0] != s:
        raise ValueError("held and new_lens must have one entry per table row")
    _check(_lib.kvc_extend_tables(alloc.handle, table.ctypes.data_as(ctypes.c_void_p),
                                  table.shape[1], held.ctypes.data_as(ctypes.c_void_p),
                                  new_lens.ctypes.data_as(ctypes.c_void_p), s),
           "kvc_extend_tables")


def kvc_allocator_block_size(alloc: Allocator) -> int:
    return int(_lib.kvc_allocator_block_size(alloc.handle))


class StepPlan:
    """Host arrays of one planned step (numpy views sized to the step)."""

    def __init__(self, cu_seqlens_q, context_lens, block_table, request_ids, max_q_len,
                 max_context_len):
        self.cu_seqlens_q = cu_seqlens_q
        self.context_lens = context_lens
        self.block_table = block_table
        self.request_ids = request_ids
        self.max_q_len = max_q_len
        self.max_context_len = max_context_len

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])


class Scheduler:
    """Host continuous-batching scheduler over an Allocator (kvc_scheduler_*)."""

    def __init__(self, alloc: Allocator, token_budget: int, max_seqs: int, max_blocks_per_seq: int):
        import numpy as np
        h = _P()
        _check(_lib.kvc_scheduler_create(alloc.handle, token_budget, max_seqs, max_blocks_per_seq,
                                         ctypes.byref(h)), "kvc_scheduler_create")
        self._h, self._alloc = h, alloc  # keeps the allocator alive
        self.max_seqs, self.max_blocks = max_seqs, max_blocks_per_seq
        self._cu = np.zeros(max_seqs + 1, np.int32)
        self._ctx = np.zeros(max_seqs, np.int32)
        self._table = np.zeros((max_seqs, max_blocks_per_seq), np.int32)
        self._ids = np.zeros(max_seqs, np.int64)
        self._fin = np.zeros(max_seqs, np.int64)

    def close(self):
        if self._h:
            _lib.kvc_scheduler_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, request_id: int, prompt_len: int, max_new_tokens: int):
        _check(_lib.kvc_scheduler_add(self._h, request_id, prompt_len, max_new_tokens),
               "kvc_scheduler_add")

    def step(self) -> StepPlan:
        """Plan the next step; the returned arrays are views valid until the next step."""
        n, t, mq, mc = _I32(0), _I32(0), _I32(0), _I32(0)
        p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        _check(_lib.kvc_scheduler_step(self._h, p(self._cu), p(self._ctx), p(self._table),
                                       p(self._ids), ctypes.byref(n), ctypes.byref(t),
                                       ctypes.byref(mq), ctypes.byref(mc)), "kvc_scheduler_step")
        k = int(n.value)
        return StepPlan(self._cu[:k + 1], self._ctx[:k], self._table[:k], self._ids[:k],
                        int(mq.value), int(mc.value))

    def complete(self):
        """Mark the planned step as executed; returns the finished request ids."""
        n = _I32(0)
        _check(_lib.kvc_scheduler_complete(self._h, self._fin.ctypes.data_as(ctypes.c_void_p),
                                           ctypes.byref(n)), "kvc_scheduler_complete")
        return self._fin[:n.value].tolist()

    @property
    def num_waiting(self) -> int:
        return int(_lib.kvc_scheduler_num_waiting(self._h))

    @property
    def num_running(self) -> int:
        return int(_lib.kvc_scheduler_num_running(self._h))


def kvc_cow_block(alloc: Allocator, block_id: int):
    """Copy-on-write before writing into block_id: returns (id to write,
    copied); when copied is True the caller copies the old block's contents
    (kvc_copy_blocks) into the returned one first."""
    out, copied = _I32(0), _I32(0)
    _check(_lib.kvc_cow_block(alloc.handle, block_id, ctypes.byref(out), ctypes.byref(copied)),
           "kvc_cow_block")
    return int(out.value), bool(copied.value)


def kvc_fork_table(alloc: Allocator, parent_row, length: int, child_row):
    """Fork: child_row (int32 numpy array, written in place) takes the
    parent's first ceil(length / block_size) blocks, sharing the full ones and
    copying a partially filled last one on write.  Returns (held, copies) with
    copies a list of (src, dst) block pairs for kvc_copy_blocks."""
    import numpy as np
    for name, r in (("parent_row", parent_row), ("child_row", child_row)):
        if not (isinstance(r, np.ndarray) and r.dtype == np.int32 and r.flags["C_CONTIGUOUS"]):
            raise TypeError(f"{name}: expected a C-contiguous int32 numpy array")
    src, dst = np.zeros(1, np.int32), np.zeros(1, np.int32)
    held, n = _I32(0), _I32(0)
    _check(_lib.kvc_fork_table(alloc.handle, parent_row.ctypes.data_as(ctypes.c_void_p), length,
                               child_row.ctypes.data_as(ctypes.c_void_p), child_row.size,
                               ctypes.byref(held), src.ctypes.data_as(ctypes.c_void_p),
                               dst.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)),
           "kvc_fork_table")
    return int(held.value), [(int(src[0]), int(dst[0]))] if n.value else []


def kvc_cache_bytes(num_blocks, block_size, num_kv_heads, head_dim, elem_bytes=2) -> int:
    return int(_lib.kvc_cache_bytes(num_blocks, block_size, num_kv_heads, head_dim, elem_bytes))


# --------------------------------------------------------------------------
# device operations
# --------------------------------------------------------------------------
def _cache_dims(k_cache, v_cache):
    _need(k_cache, torch.bfloat16, 4, "k_cache")
    _need(v_cache, torch.bfloat16, 4, "v_cache")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    return k_cache.shape  # nb, hkv, bs, a


def kvc_append_kv(k_new, v_new, k_cache, v_cache, block_table, cu_seqlens_q, context_lens,
                  stream=None):
    nb, hkv, bs, a = _cache_dims(k_cache, v_cache)
    _need(k_new, torch.bfloat16, 3, "k_new")
    _need(v_new, torch.bfloat16, 3, "v_new")
    _need(block_table, torch.int32, 2, "block_table")
    _need(cu_seqlens_q, torch.int32, 1, "cu_seqlens_q")
    _need(context_lens, torch.int32, 1, "context_lens")
    if tuple(k_new.shape[1:]) != (hkv, a) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [total_q, Hkv, A] matching the cache")
    s = context_lens.shape[0]
    if cu_seqlens_q.shape[0] != s + 1 or block_table.shape[0] != s:
        raise ValueError("cu_seqlens_q must be [S+1] and block_table [S, max_blocks]")
    _check(_lib.kvc_append_kv(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), nb,
                              _ptr(block_table), block_table.shape[1], _ptr(cu_seqlens_q),
                              _ptr(context_lens), s, k_new.shape[0], hkv, a, bs,
                              _stream(stream)), "kvc_append_kv")


def kvc_gather_kv(k_cache, v_cache, block_table, seq_lens, cu_seq_lens, k_out, v_out,
                  stream=None):
    nb, hkv, bs, a = _cache_dims(k_cache, v_cache)
    _need(block_table, torch.int32, 2, "block_table")
    _need(seq_lens, torch.int32, 1, "seq_lens")
    _need(cu_seq_lens, torch.int64, 1, "cu_seq_lens")
    _need(k_out, torch.bfloat16, 3, "k_out")
    _need(v_out, torch.bfloat16, 3, "v_out")
    s = seq_lens.shape[0]
    if cu_seq_lens.shape[0] != s + 1 or block_table.shape[0] != s:
        raise ValueError("cu_seq_lens must be [S+1] and block_table [S, max_blocks]")
    if tuple(k_out.shape[1:]) != (hkv, a) or k_out.shape != v_out.shape:
        raise ValueError("k_out/v_out must be [total, Hkv, A]")
    _check(_lib.kvc_gather_kv(_ptr(k_cache), _ptr(v_cache), nb, _ptr(block_table),
                              block_table.shape[1], _ptr(seq_lens), _ptr(cu_seq_lens),
                              k_out.shape[0], _ptr(k_out), _ptr(v_out), s, hkv, a, bs,
                              _stream(stream)), "kvc_gather_kv")


def kvc_copy_blocks(k_cache, v_cache, src_ids, dst_ids, stream=None):
    """Block dst_ids[i] := block src_ids[i] in both pools (int32 GPU tensors)."""
    nb, hkv, bs, a = _cache_dims(k_cache, v_cache)
    _need(src_ids, torch.int32, 1, "src_ids")
    _need(dst_ids, torch.int32, 1, "dst_ids")
    if src_ids.shape != dst_ids.shape:
        raise ValueError("src_ids and dst_ids must have the same length")
    _check(_lib.kvc_copy_blocks(_ptr(k_cache), _ptr(v_cache), nb, _ptr(src_ids), _ptr(dst_ids),
                                src_ids.shape[0], hkv, a, bs, _stream(stream)),
           "kvc_copy_blocks")


def kvc_workspace_size(num_seqs, total_q, max_q_len, max_context_len, num_q_heads,
                       num_kv_heads, head_dim, block_size) -> int:
    return int(_lib.kvc_workspace_size(num_seqs, total_q, max_q_len, max_context_len,
                                       num_q_heads, num_kv_heads, head_dim, block_size))


def kvc_paged_attention_varlen(out, q, k_new, v_new, k_cache, v_cache, block_table,
                               cu_seqlens_q, context_lens, scale, *, max_q_len,
                               max_context_len, workspace, stream=None):
    """One ragged step: append k_new/v_new (unless both are None), then attend.

    ``max_q_len`` / ``max_context_len`` are host-side upper bounds of the
    per-sequence lengths; ``workspace`` is a uint8 GPU tensor of at least
    ``kvc_workspace_size(...)`` bytes (256-byte aligned)."""
    nb, hkv, bs, a = _cache_dims(k_cache, v_cache)
    _need(q, torch.bfloat16, 3, "q")
    _need(out, torch.bfloat16, 3, "out")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    if k_new is not None:
        _need(k_new, torch.bfloat16, 3, "k_new")
        _need(v_new, torch.bfloat16, 3, "v_new")
        if tuple(k_new.shape) != (q.shape[0], hkv, a) or k_new.shape != v_new.shape:
            raise ValueError("k_new/v_new must be [total_q, Hkv, A]")
    _need(block_table, torch.int32, 2, "block_table")
    _need(cu_seqlens_q, torch.int32, 1, "cu_seqlens_q")
    _need(context_lens, torch.int32, 1, "context_lens")
    _need(workspace, torch.uint8, 1, "workspace")
    tq, hq, a2 = q.shape
    if a2 != a or out.shape != q.shape:
        raise ValueError("q/out must be [total_q, Hq, A] with the cache's head_dim")
    s = context_lens.shape[0]
    if cu_seqlens_q.shape[0] != s + 1 or block_table.shape[0] != s:
        raise ValueError("cu_seqlens_q must be [S+1] and block_table [S, max_blocks]")
    _check(_lib.kvc_paged_attention_varlen(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), nb,
        _ptr(block_table), block_table.shape[1], _ptr(cu_seqlens_q), _ptr(context_lens), s, tq,
        int(max_q_len), int(max_context_len), hq, hkv, a, bs, float(scale), _ptr(workspace),
        workspace.numel(), _stream(stream)), "kvc_paged_attention_varlen")


def _step_args(out, q, k_new, v_new, k_cache, v_cache, block_table, cu_seqlens_q,
               context_lens):
    """Checks shared by the attention entry points; returns the sizes."""
    nb, hkv, bs, a = _cache_dims(k_cache, v_cache)
    _need(q, torch.bfloat16, 3, "q")
    _need(out, torch.bfloat16, 3, "out")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    if k_new is not None:
        _need(k_new, torch.bfloat16, 3, "k_new")
        _need(v_new, torch.bfloat16, 3, "v_new")
        if tuple(k_new.shape) != (q.shape[0], hkv, a) or k_new.shape != v_new.shape:
            raise ValueError("k_new/v_new must be [total_q, Hkv, A]")
    _need(block_table, torch.int32, 2, "block_table")
    _need(cu_seqlens_q, torch.int32, 1, "cu_seqlens_q")
    _need(context_lens, torch.int32, 1, "context_lens")
    tq, hq, a2 = q.shape
    if a2 != a or out.shape != q.shape:
        raise ValueError("q/out must be [total_q, Hq, A] with the cache's head_dim")
    s = context_lens.shape[0]
    if cu_seqlens_q.shape[0] != s + 1 or block_table.shape[0] != s:
        raise ValueError("cu_seqlens_q must be [S+1] and block_table [S, max_blocks]")
    return nb, hkv, bs, a, tq, hq, s


def kvc_paged_attention_varlen_noalloc(out, q, k_new, v_new, k_cache, v_cache, block_table,
                                       cu_seqlens_q, context_lens, scale, *, max_q_len,
                                       max_context_len, stream=None):
    """The step without a workspace: scratch is the library's static device
    array (NOALLOC_SCRATCH_BYTES per GPU, shared by every call on that GPU, so
    overlapping calls race); every kernel runs on ``stream``."""
    nb, hkv, bs, a, tq, hq, s = _step_args(out, q, k_new, v_new, k_cache, v_cache, block_table,
                                           cu_seqlens_q, context_lens)
    _check(_lib.kvc_paged_attention_varlen_noalloc(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), nb,
        _ptr(block_table), block_table.shape[1], _ptr(cu_seqlens_q), _ptr(context_lens), s, tq,
        int(max_q_len), int(max_context_len), hq, hkv, a, bs, float(scale), _stream(stream)),
        "kvc_paged_attention_varlen_noalloc")


def kvc_padded_workspace_size(batch, n_max, num_q_heads, num_kv_heads, head_dim,
                              block_size) -> int:
    return int(_lib.kvc_padded_workspace_size(batch, n_max, num_q_heads, num_kv_heads, head_dim,
                                              block_size))


def kvc_padded_decode_attention(out, q, k_new, v_new, k_cache, v_cache, pad_lens, scale, *,
                                n_max, workspace, stream=None):
    """One decode step of a left-padded batch over a contiguous cache that
    reserves n_max positions per sequence (k_cache/v_cache
    [batch * n_max / block_size, Hkv, block_size, A], sequence b's pages
    consecutive); pad_lens [batch] int32 on the GPU: sequence b's tokens sit
    at positions pad_lens[b] .. n_max - 1."""
    nb, hkv, bs, a = _cache_dims(k_cache, v_cache)
    _need(q, torch.bfloat16, 3, "q")
    _need(out, torch.bfloat16, 3, "out")
    _need(pad_lens, torch.int32, 1, "pad_lens")
    _need(workspace, torch.uint8, 1, "workspace")
    b, hq, a2 = q.shape
    if a2 != a or out.shape != q.shape or pad_lens.shape[0] != b:
        raise ValueError("q/out must be [batch, Hq, A] with the cache's head_dim; pad_lens [batch]")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    if k_new is not None:
        _need(k_new, torch.bfloat16, 3, "k_new")
        _need(v_new, torch.bfloat16, 3, "v_new")
        if tuple(k_new.shape) != (b, hkv, a) or k_new.shape != v_new.shape:
            raise ValueError("k_new/v_new must be [batch, Hkv, A]")
    if n_max % bs or nb != b * (n_max // bs):
        raise ValueError("the cache must hold batch * n_max / block_size pages")
    _check(_lib.kvc_padded_decode_attention(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(pad_lens), b, int(n_max), hq, hkv, a, bs, float(scale), _ptr(workspace),
        workspace.numel(), _stream(stream)), "kvc_padded_decode_attention")


def kvc_workspace_flags(workspace, stream=None) -> int:
    v = _I32(0)
    _check(_lib.kvc_workspace_flags(_ptr(workspace), _stream(stream), ctypes.byref(v)),
           "kvc_workspace_flags")
    return int(v.value)


def new_workspace(num_seqs, total_q, max_q_len, max_context_len, num_q_heads, num_kv_heads,
                  head_dim, block_size, device="cuda"):
    """Allocate (with torch) a workspace tensor of the size the step needs."""
    n = kvc_workspace_size(num_seqs, total_q, max_q_len, max_context_len, num_q_heads,
                           num_kv_heads, head_dim, block_size)
    if n == 0:
        raise KvcError(KVC_ERR_UNSUPPORTED, "kvc_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def kvc_profile_begin(max_calls: int):
    """Record HIP events around each kernel of the next max_calls steps."""
    _check(_lib.kvc_profile_begin(max_calls), "kvc_profile_begin")


def kvc_profile_end():
    """Wait for the recorded events; returns ({phase: total ms}, calls)."""
    ms = (ctypes.c_double * len(PROF_PHASES))()
    n = _I32(0)
    _check(_lib.kvc_profile_end(ms, ctypes.byref(n)), "kvc_profile_end")
    return {p: float(ms[i]) for i, p in enumerate(PROF_PHASES)}, int(n.value)
