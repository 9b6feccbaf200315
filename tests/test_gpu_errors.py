"""Error behaviour on the GPU.  Argument errors return a status before
anything is enqueued.  Bad values inside the device arrays (block ids, table
rows too short for a length, lengths above the host bounds, inconsistent
cu_seqlens_q) are caught by the kernels' own bounds checks, never
dereferenced, and reported through the workspace flags; KVC_DEBUG=1 rejects
them on the host before any launch."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DevStep, compare, dev_bits, dev_i32, host_bits, oracle_run

pytestmark = pytest.mark.gpu

FLAG_TABLE_SHORT, FLAG_BAD_BLOCK, FLAG_CAPACITY, FLAG_CU_SEQLENS = 1, 2, 4, 8
# (context, new rows): a 5-row chunk, a first-token decode, a long decode and
# a 40-row chunk; block size 16, so sequence 2 spans 19 blocks
SPECS = [(7, 5), (0, 1), (300, 1), (33, 40)]


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def _wl(seed=31):
    return W.make_step_workload("err", SPECS, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                block_size=16, seed=seed, spare_blocks=4)


def _call(kvc, wl, st, max_c=None, table=None, cu=None, ctx=None):
    """One step on fresh device copies; returns (out, k_cache, flags)."""
    d = DevStep(st)
    kc, vc = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
    out = torch.zeros_like(d.q)
    max_c = st.max_context_len if max_c is None else max_c
    ws = kvc.new_workspace(st.num_seqs, st.total_q, st.max_q_len, max_c, wl.num_q_heads,
                           wl.num_kv_heads, wl.head_dim, wl.block_size)
    kvc.kvc_paged_attention_varlen(
        out, d.q, d.k_new, d.v_new, kc, vc, d.table if table is None else dev_i32(table),
        d.cu if cu is None else dev_i32(cu), d.ctx if ctx is None else dev_i32(ctx), wl.scale,
        max_q_len=st.max_q_len, max_context_len=max_c, workspace=ws)
    torch.cuda.synchronize()
    return out, kc, kvc.kvc_workspace_flags(ws)


def test_workspace_too_small_enqueues_nothing(kvc):
    wl = _wl()
    st = wl.steps[0]
    d = DevStep(st)
    kc, vc = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
    out = torch.zeros_like(d.q)
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_paged_attention_varlen(out, d.q, d.k_new, d.v_new, kc, vc, d.table, d.cu, d.ctx,
                                       wl.scale, max_q_len=st.max_q_len,
                                       max_context_len=st.max_context_len, workspace=ws)
    assert e.value.status == kvc.KVC_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out.float() == 0).all(), "output written by a rejected call"
    assert np.array_equal(host_bits(kc), wl.k_pool), "pool written by a rejected call"


def test_bad_arguments_enqueue_nothing(kvc):
    wl = _wl()
    st = wl.steps[0]
    d = DevStep(st)
    kc, vc = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
    out = torch.zeros_like(d.q)
    ws = kvc.new_workspace(st.num_seqs, st.total_q, st.max_q_len, st.max_context_len, 8, 2,
                           128, 16)
    kw = dict(max_q_len=st.max_q_len, max_context_len=st.max_context_len, workspace=ws)
    with pytest.raises(kvc.KvcError) as e:  # scale not finite
        kvc.kvc_paged_attention_varlen(out, d.q, d.k_new, d.v_new, kc, vc, d.table, d.cu, d.ctx,
                                       float("nan"), **kw)
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    with pytest.raises(kvc.KvcError) as e:  # max_q_len above total_q
        kvc.kvc_paged_attention_varlen(out, d.q, d.k_new, d.v_new, kc, vc, d.table, d.cu, d.ctx,
                                       wl.scale, max_q_len=st.total_q + 1,
                                       max_context_len=st.max_context_len, workspace=ws)
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    # head_dim 96 is not built
    k96 = torch.zeros(wl.num_blocks, 2, 16, 96, dtype=torch.bfloat16, device="cuda")
    q96 = torch.zeros(st.total_q, 8, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_paged_attention_varlen(torch.zeros_like(q96), q96, None, None, k96, k96.clone(),
                                       d.table, d.cu, d.ctx, wl.scale, **kw)
    assert e.value.status == kvc.KVC_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (out.float() == 0).all(), "output written by a rejected call"
    assert np.array_equal(host_bits(kc), wl.k_pool), "pool written by a rejected call"


def test_bad_cached_block_is_flagged_and_contained(kvc, orc):
    wl = _wl()
    st = wl.steps[0]
    bad = st.block_table.copy()
    bad[2, 3] = wl.num_blocks + 5      # cached block of the long decode row
    bad[3, 1] = -3                     # cached block of the 40-row chunk
    out, _, flags = _call(kvc, wl, st, table=bad)
    assert flags & FLAG_BAD_BLOCK, flags
    assert not flags & ~FLAG_BAD_BLOCK, flags
    (ref,), _, _ = oracle_run(orc, wl)
    cu = st.cu_seqlens_q
    compare(host_bits(out), ref, rows=np.r_[cu[0]:cu[2]], what="sequences with intact rows")


def test_bad_append_block_skips_those_rows(kvc, orc):
    wl = _wl()
    st = wl.steps[0]
    bad = st.block_table.copy()
    lost = int(bad[3, 3])              # positions 48..63 of the chunk (rows 15..30 of it)
    bad[3, 3] = wl.num_blocks + 100
    _, kc, flags = _call(kvc, wl, st, table=bad)
    assert flags & FLAG_BAD_BLOCK, flags
    _, kp, _ = oracle_run(orc, wl)
    kp[lost] = wl.k_pool[lost]         # that block is never written
    assert np.array_equal(host_bits(kc), kp)


def test_short_table_is_flagged(kvc):
    wl = _wl()
    st = wl.steps[0]
    ctx = st.context_lens.copy()
    ctx[3] = 700                        # needs 47 table entries; the row has fewer
    assert (700 + 40 + 15) // 16 > st.block_table.shape[1]
    _, kc, flags = _call(kvc, wl, st, max_c=700, ctx=ctx)
    assert flags & FLAG_TABLE_SHORT, flags


def test_lengths_above_host_bounds_are_flagged(kvc):
    wl = _wl()
    st = wl.steps[0]
    _, _, flags = _call(kvc, wl, st, max_c=100)  # the long decode row has context 300
    assert flags & FLAG_CAPACITY, flags


@pytest.mark.parametrize("case", ["end_past_total", "decreasing", "start_nonzero"])
def test_inconsistent_cu_seqlens_is_flagged(kvc, case):
    wl = _wl()
    st = wl.steps[0]
    cu = st.cu_seqlens_q.copy()
    if case == "end_past_total":
        cu[-1] += 3
    elif case == "decreasing":
        cu[2] = cu[1] - 1
    else:
        cu[0] = 1
    _, _, flags = _call(kvc, wl, st, cu=cu)
    assert flags & FLAG_CU_SEQLENS, flags


def test_debug_mode_rejects_bad_table_on_host(kvc, monkeypatch):
    wl = _wl()
    st = wl.steps[0]
    bad = st.block_table.copy()
    bad[2, 3] = wl.num_blocks + 5
    monkeypatch.setenv("KVC_DEBUG", "1")
    with pytest.raises(kvc.KvcError) as e:
        _call(kvc, wl, st, table=bad)
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    assert "block id" in str(e.value)
    _, _, flags = _call(kvc, wl, st)   # the intact table passes the same checks
    assert flags == 0
