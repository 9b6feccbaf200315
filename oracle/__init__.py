"""CPU oracle for the ragged paged-attention step — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (``batching_kv_append_amd``)
never imports it, and this package imports nothing from the product: the two
share no code.  The arithmetic lives in ``kvc_oracle.c`` (plain fp64 loops);
this module only marshals numpy arrays into it.

Array conventions (all host numpy, C-contiguous):
  bf16 tensors are ``uint16`` arrays of raw bf16 bit patterns;
  q [Tq, Hq, A], k_new/v_new [Tq, Hkv, A];
  pools [num_blocks, Hkv, block_size, A];
  block_table int32 [S, max_blocks]; cu_seqlens_q int32 [S+1];
  context_lens int32 [S] (tokens cached before the step).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _need(a, dtype, ndim, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or a.ndim != ndim \
            or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name}: expected C-contiguous {np.dtype(dtype).name} "
                        f"array with {ndim} dims")
    return a


class Oracle:
    """ctypes handle on one build of ``kvc_oracle.c``."""

    def __init__(self, lib_path: str | None = None):
        path = lib_path or _build.LIB
        if not os.path.exists(path):
            _build.build(path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.kvco_kv_bytes_per_token.restype = _I64
        lib.kvco_kv_bytes_per_token.argtypes = [_I32, _I32, _I32, _I32]
        lib.kvco_append.restype = ctypes.c_int
        lib.kvco_append.argtypes = [_P, _P, _I64, _P, _P, _P, _I32, _P, _P,
                                    _I32, _I32, _I32, _I32]
        lib.kvco_gather.restype = ctypes.c_int
        lib.kvco_gather.argtypes = [_P, _P, _I64, _P, _I32, _P, _P, _P, _P,
                                    _I32, _I32, _I32, _I32]
        lib.kvco_attention.restype = ctypes.c_int
        lib.kvco_attention.argtypes = [_P, _P, _P, _P, _P, _I64, _P, _I32, _P,
                                       _P, _I32, _I32, _I32, _I32, _I32,
                                       ctypes.c_double, ctypes.c_int]
        self.lib = lib

    # ------------------------------------------------------------------
    def kv_bytes_per_token(self, num_layers, num_kv_heads, head_dim, elem_bytes=2):
        return int(self.lib.kvco_kv_bytes_per_token(num_layers, num_kv_heads,
                                                    head_dim, elem_bytes))

    def append(self, k_pool, v_pool, k_new, v_new, block_table, cu_seqlens_q,
               context_lens):
        """Write k_new/v_new into the pools IN PLACE (bit copy)."""
        _need(k_pool, np.uint16, 4, "k_pool")
        _need(v_pool, np.uint16, 4, "v_pool")
        _need(k_new, np.uint16, 3, "k_new")
        _need(v_new, np.uint16, 3, "v_new")
        _need(block_table, np.int32, 2, "block_table")
        _need(cu_seqlens_q, np.int32, 1, "cu_seqlens_q")
        _need(context_lens, np.int32, 1, "context_lens")
        nb, hkv, bs, a = k_pool.shape
        s = context_lens.shape[0]
        rc = self.lib.kvco_append(_ptr(k_pool), _ptr(v_pool), nb, _ptr(k_new),
                                  _ptr(v_new), _ptr(block_table),
                                  block_table.shape[1], _ptr(cu_seqlens_q),
                                  _ptr(context_lens), s, hkv, a, bs)
        if rc != 0:
            raise ValueError("oracle append: position outside the block table "
                             "or block id out of range")

    def gather(self, k_pool, v_pool, block_table, seq_lens):
        """Contiguous [sum L, Hkv, A] K and V (bf16 bits) of every sequence."""
        _need(k_pool, np.uint16, 4, "k_pool")
        _need(v_pool, np.uint16, 4, "v_pool")
        _need(block_table, np.int32, 2, "block_table")
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        nb, hkv, bs, a = k_pool.shape
        cu = np.zeros(len(seq_lens) + 1, dtype=np.int64)
        np.cumsum(seq_lens, out=cu[1:])
        k_out = np.empty((int(cu[-1]), hkv, a), dtype=np.uint16)
        v_out = np.empty_like(k_out)
        rc = self.lib.kvco_gather(_ptr(k_pool), _ptr(v_pool), nb,
                                  _ptr(block_table), block_table.shape[1],
                                  _ptr(seq_lens), _ptr(cu), _ptr(k_out),
                                  _ptr(v_out), len(seq_lens), hkv, a, bs)
        if rc != 0:
            raise ValueError("oracle gather: position outside the block table "
                             "or block id out of range")
        return k_out, v_out

    def attention(self, q, k_pool, v_pool, block_table, cu_seqlens_q,
                  context_lens, scale, row_select=None, nthreads=0, out=None):
        """fp64 attention over the (already appended) pools.

        Returns (out [Tq, Hq, A] float64, threads used).  With ``row_select``
        ([Tq] bool), unselected rows of ``out`` are left as they were (NaN
        when ``out`` is not given)."""
        _need(q, np.uint16, 3, "q")
        _need(k_pool, np.uint16, 4, "k_pool")
        _need(v_pool, np.uint16, 4, "v_pool")
        _need(block_table, np.int32, 2, "block_table")
        _need(cu_seqlens_q, np.int32, 1, "cu_seqlens_q")
        _need(context_lens, np.int32, 1, "context_lens")
        tq, hq, a = q.shape
        nb, hkv, bs, a2 = k_pool.shape
        if a2 != a:
            raise ValueError("head_dim mismatch")
        if out is None:
            out = np.full((tq, hq, a), np.nan, dtype=np.float64)
        _need(out, np.float64, 3, "out")
        sel = None
        if row_select is not None:
            sel = np.ascontiguousarray(row_select, dtype=np.uint8)
            if sel.shape != (tq,):
                raise ValueError("row_select must have shape [Tq]")
        used = self.lib.kvco_attention(_ptr(out), _ptr(sel), _ptr(q),
                                       _ptr(k_pool), _ptr(v_pool), nb,
                                       _ptr(block_table), block_table.shape[1],
                                       _ptr(cu_seqlens_q), _ptr(context_lens),
                                       context_lens.shape[0], hq, hkv, a, bs,
                                       float(scale), int(nthreads))
        if used < 0:
            raise ValueError("oracle attention: bad shapes, table or block id")
        return out, used

    def step(self, q, k_new, v_new, k_pool, v_pool, block_table, cu_seqlens_q,
             context_lens, scale, row_select=None, nthreads=0):
        """Append into COPIES of the pools, then attend.

        Returns (out float64, k_pool_after, v_pool_after)."""
        kp = k_pool.copy()
        vp = v_pool.copy()
        self.append(kp, vp, k_new, v_new, block_table, cu_seqlens_q, context_lens)
        out, _ = self.attention(q, kp, vp, block_table, cu_seqlens_q,
                                context_lens, scale, row_select, nthreads)
        return out, kp, vp


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from the unmodified source."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
