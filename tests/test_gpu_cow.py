"""Copy-on-write on the GPU: kvc_copy_blocks is a bit copy of whole blocks,
and a fork of a sequence whose prefix ends inside a block (the last block
copied, the full ones shared by reference) gives both sequences exactly the
attention the oracle computes over their own tables, while the shared
blocks stay bit-identical."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev_bits, dev_i32, host_bits

pytestmark = pytest.mark.gpu

HQ, HKV, A, BS, NB, MB = 8, 2, 128, 16, 32, 8
SCALE = 1.0 / math.sqrt(A)


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def _pool(seed):
    n = NB * HKV * BS * A
    return (W._normal_bf16(n, seed, "k_cache").reshape(NB, HKV, BS, A),
            W._normal_bf16(n, seed, "v_cache").reshape(NB, HKV, BS, A))


def test_copy_blocks_bit_exact(kvc):
    kp, vp = _pool(11)
    kc, vc = dev_bits(kp), dev_bits(vp)
    src, dst = [3, 7, 11, 5], [20, 0, 33, 6]  # the pair (11, 33) is out of range: skipped
    kvc.kvc_copy_blocks(kc, vc, dev_i32(src), dev_i32(dst))
    torch.cuda.synchronize()
    ek, ev = kp.copy(), vp.copy()
    for s, d in zip(src, dst):
        if s < NB and d < NB:
            ek[d], ev[d] = kp[s], vp[s]
    assert np.array_equal(host_bits(kc), ek)
    assert np.array_equal(host_bits(vc), ev)


def _step(seed, lens, ctx, rows):
    """One call's host arrays: q/k_new/v_new drawn for sum(lens) new rows."""
    tq = int(sum(lens))
    q = W._normal_bf16(tq * HQ * A, seed, "q").reshape(tq, HQ, A)
    kn = W._normal_bf16(tq * HKV * A, seed, "k_new").reshape(tq, HKV, A)
    vn = W._normal_bf16(tq * HKV * A, seed, "v_new").reshape(tq, HKV, A)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return W.Step(q=q, k_new=kn, v_new=vn, cu_seqlens_q=cu,
                  context_lens=np.asarray(ctx, np.int32), block_table=np.stack(rows).astype(np.int32))


def _gpu_call(kvc, st, kc, vc):
    out = torch.empty(st.total_q, HQ, A, dtype=torch.bfloat16, device="cuda")
    ws = kvc.new_workspace(st.num_seqs, st.total_q, st.max_q_len, st.max_context_len, HQ, HKV, A, BS)
    kvc.kvc_paged_attention_varlen(out, dev_bits(st.q), dev_bits(st.k_new), dev_bits(st.v_new),
                                   kc, vc, dev_i32(st.block_table), dev_i32(st.cu_seqlens_q),
                                   dev_i32(st.context_lens), SCALE, max_q_len=st.max_q_len,
                                   max_context_len=st.max_context_len, workspace=ws)
    torch.cuda.synchronize()
    assert kvc.kvc_workspace_flags(ws) == 0
    return host_bits(out)


def _oracle_call(orc, st, kp, vp):
    orc.append(kp, vp, st.k_new, st.v_new, st.block_table, st.cu_seqlens_q, st.context_lens)
    out, _ = orc.attention(st.q, kp, vp, st.block_table, st.cu_seqlens_q, st.context_lens, SCALE)
    return out


@pytest.mark.parametrize("prefix", [37, 32])
def test_fork_with_partial_block(kvc, orc, prefix):
    alloc = kvc.Allocator(NB, BS)
    parent = np.full(MB, -1, np.int32)
    held_p = kvc.kvc_extend_table(alloc, parent, 0, prefix)
    kp, vp = _pool(5)
    kc, vc = dev_bits(kp), dev_bits(vp)

    # 1. the parent writes its prefix (one chunk at context 0)
    st1 = _step(21, [prefix], [0], [parent])
    compare(_gpu_call(kvc, st1, kc, vc), _oracle_call(orc, st1, kp, vp), what="prefix")

    # 2. fork: full blocks shared, a partially filled last block copied
    child = np.full(MB, -1, np.int32)
    held_c, copies = kvc.kvc_fork_table(alloc, parent, prefix, child)
    assert len(copies) == (1 if prefix % BS else 0)
    if copies:
        src = [s for s, _ in copies]
        dst = [d for _, d in copies]
        kvc.kvc_copy_blocks(kc, vc, dev_i32(src), dev_i32(dst))
        kp[dst], vp[dst] = kp[src], vp[src]
    shared = parent[:prefix // BS].copy()
    before_k = host_bits(kc)[shared]

    # 3. both append different rows in one call: chunks of 20 and 11 rows
    held_p = kvc.kvc_extend_table(alloc, parent, held_p, prefix + 20)
    held_c = kvc.kvc_extend_table(alloc, child, held_c, prefix + 11)
    st2 = _step(22, [20, 11], [prefix, prefix], [parent, child])
    compare(_gpu_call(kvc, st2, kc, vc), _oracle_call(orc, st2, kp, vp), what="chunks after fork")

    # 4. one decode row each
    held_p = kvc.kvc_extend_table(alloc, parent, held_p, prefix + 21)
    held_c = kvc.kvc_extend_table(alloc, child, held_c, prefix + 12)
    st3 = _step(23, [1, 1], [prefix + 20, prefix + 11], [parent, child])
    compare(_gpu_call(kvc, st3, kc, vc), _oracle_call(orc, st3, kp, vp), what="decode after fork")

    # the pools agree bit for bit, and the shared full blocks never changed
    assert np.array_equal(host_bits(kc), kp) and np.array_equal(host_bits(vc), vp)
    assert np.array_equal(host_bits(kc)[shared], before_k)
    kvc.kvc_free_blocks(alloc, parent[:held_p])
    kvc.kvc_free_blocks(alloc, child[:held_c])
    assert kvc.kvc_num_free_blocks(alloc) == NB
