"""Pools larger than 4 GiB: the blocks a step uses sit 5 GiB into each pool,
so every block address needs 64-bit arithmetic.  A mixed GQA step (decode
rows and prompt chunks) equals the oracle's, which sees the same blocks in a
compact pool (the same ids less the offset); the appended rows land in the
high blocks bit for bit, a gather through the high ids returns them, a copy
between high blocks is exact, and the block just below stays untouched."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev_bits, dev_i32, host_bits, oracle_run

pytestmark = pytest.mark.gpu

HQ, HKV, A, BS = 32, 8, 128, 16
BLOCK_BYTES = HKV * BS * A * 2    # one block, all kv heads, one pool: 32 KiB
BASE = (5 << 30) // BLOCK_BYTES   # id of the first block the step uses


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def test_blocks_past_4gib(kvc, orc):
    specs = [(1000, 1), (37, 1), (300, 64), (0, 90), (4095, 1), (2000, 129), (255, 1)]
    wl = W.make_step_workload("large_pool", specs, num_q_heads=HQ, num_kv_heads=HKV, head_dim=A,
                              block_size=BS, seed=31)
    st = wl.steps[0]
    nb = wl.k_pool.shape[0]
    total = BASE + nb
    assert (BASE * BLOCK_BYTES) >> 32 >= 1
    kc = torch.empty((total, HKV, BS, A), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    kc[BASE:] = dev_bits(wl.k_pool)
    vc[BASE:] = dev_bits(wl.v_pool)
    kc[BASE - 1].fill_(7.0)
    vc[BASE - 1].fill_(-7.0)
    table = st.block_table.copy()
    table[table >= 0] += BASE

    q = dev_bits(st.q)
    out = torch.empty_like(q)
    ws = kvc.new_workspace(st.num_seqs, st.total_q, st.max_q_len, st.max_context_len, HQ, HKV,
                           A, BS)
    kvc.kvc_paged_attention_varlen(out, q, dev_bits(st.k_new), dev_bits(st.v_new), kc, vc,
                                   dev_i32(table), dev_i32(st.cu_seqlens_q),
                                   dev_i32(st.context_lens), wl.scale, max_q_len=st.max_q_len,
                                   max_context_len=st.max_context_len, workspace=ws)
    torch.cuda.synchronize()
    assert kvc.kvc_workspace_flags(ws) == 0

    (ref,), kp, vp = oracle_run(orc, wl)
    compare(host_bits(out), ref, what="blocks past 4 GiB")
    assert np.array_equal(host_bits(kc[BASE:]), kp) and np.array_equal(host_bits(vc[BASE:]), vp)
    below = BASE - 1
    assert torch.all(kc[below] == 7.0).item() and torch.all(vc[below] == -7.0).item()

    # gather through the high ids: each sequence's rows, in position order
    lens = (st.context_lens + np.diff(st.cu_seqlens_q)).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ko = torch.empty((int(cu[-1]), HKV, A), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    kvc.kvc_gather_kv(kc, vc, dev_i32(table), dev_i32(lens),
                      torch.from_numpy(cu).cuda(), ko, vo)
    torch.cuda.synchronize()
    ek = np.concatenate([kp[st.block_table[i, np.arange(n) // BS], :, np.arange(n) % BS, :]
                         for i, n in enumerate(lens)])
    ev = np.concatenate([vp[st.block_table[i, np.arange(n) // BS], :, np.arange(n) % BS, :]
                         for i, n in enumerate(lens)])
    assert np.array_equal(host_bits(ko), ek) and np.array_equal(host_bits(vo), ev)

    # copy-on-write copy into the block below (also past 4 GiB) is a bit copy
    src, dst = int(table[0, 0]), below
    kvc.kvc_copy_blocks(kc, vc, dev_i32([src]), dev_i32([dst]))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(kc[dst]), host_bits(kc[src]))
    assert np.array_equal(host_bits(vc[dst]), host_bits(vc[src]))
