"""Helpers for the GPU tests: move seeded workloads to the device, run steps
through the C-ABI binding, compare with the oracle.  Input construction only;
no attention arithmetic lives here."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

MAX_ABS = 2e-2   # per-element bound on |gpu - oracle|, bf16 inputs and output
MEAN_ABS = 2e-3  # bound on the mean of |gpu - oracle| over the compared rows


def dev_bits(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a bf16 tensor on the GPU (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


class DevStep:
    """Device copies of one Step's arrays."""

    def __init__(self, st: W.Step):
        self.st = st
        self.q = dev_bits(st.q)
        self.k_new = dev_bits(st.k_new)
        self.v_new = dev_bits(st.v_new)
        self.cu = dev_i32(st.cu_seqlens_q)
        self.ctx = dev_i32(st.context_lens)
        self.table = dev_i32(st.block_table)


def run_steps(kvc, wl: W.Workload, steps=None, k_cache=None, v_cache=None, ws=None,
              stream=None):
    """Run the steps in order on the GPU; returns (outputs as uint16 arrays,
    k_cache, v_cache)."""
    steps = steps if steps is not None else wl.steps
    if k_cache is None:
        k_cache = dev_bits(wl.k_pool)
        v_cache = dev_bits(wl.v_pool)
    outs = []
    for st in steps:
        d = DevStep(st)
        w = ws if ws is not None else kvc.new_workspace(
            st.num_seqs, st.total_q, st.max_q_len, st.max_context_len, wl.num_q_heads,
            wl.num_kv_heads, wl.head_dim, wl.block_size)
        out = torch.empty_like(d.q)
        kvc.kvc_paged_attention_varlen(out, d.q, d.k_new, d.v_new, k_cache, v_cache, d.table,
                                       d.cu, d.ctx, wl.scale, max_q_len=st.max_q_len,
                                       max_context_len=st.max_context_len, workspace=w,
                                       stream=stream)
        torch.cuda.synchronize()
        flags = kvc.kvc_workspace_flags(w)
        assert flags == 0, f"kernel flags {flags}"
        outs.append(host_bits(out))
    return outs, k_cache, v_cache


def compare(gpu_bits: np.ndarray, ref: np.ndarray, rows=None, what=""):
    """Element-wise comparison of a bf16 GPU output with the fp64 oracle."""
    g = W.bits_to_f32(gpu_bits).astype(np.float64)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert g.size > 0, f"{what}: nothing to compare"
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    assert np.isfinite(ref).all(), f"{what}: non-finite oracle output"
    d = np.abs(g - ref)
    mx, mean = float(d.max()), float(d.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, \
        f"{what}: max |diff| {mx:.3e} (<= {MAX_ABS}), mean {mean:.3e} (<= {MEAN_ABS})"
    return mx, mean


def oracle_run(orc, wl: W.Workload, steps=None, row_select=None):
    """Oracle outputs of the steps in order (append then attend each)."""
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    outs = []
    for i, st in enumerate(steps if steps is not None else wl.steps):
        orc.append(kp, vp, st.k_new, st.v_new, st.block_table, st.cu_seqlens_q, st.context_lens)
        sel = None if row_select is None else row_select[i]
        out, _ = orc.attention(st.q, kp, vp, st.block_table, st.cu_seqlens_q, st.context_lens,
                               wl.scale, sel)
        outs.append(out)
    return outs, kp, vp
