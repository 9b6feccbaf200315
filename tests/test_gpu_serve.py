"""Scheduler-driven multi-step run on the GPU: the host scheduler plans every
step (decode rows, prompt chunks, admissions, blocks just in time, blocks
freed and reused), the library runs it, and every step's output and the final
pools equal the oracle's on the same plans."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev_bits, dev_i32, host_bits

pytestmark = pytest.mark.gpu

HQ, HKV, A, BS, NB, MB = 8, 2, 128, 16, 48, 12
SCALE = 1.0 / math.sqrt(A)


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def test_scheduled_steps_match_oracle(kvc, orc):
    rng = np.random.default_rng(17)
    alloc = kvc.Allocator(NB, BS)
    sched = kvc.Scheduler(alloc, token_budget=64, max_seqs=6, max_blocks_per_seq=MB)
    for i in range(14):  # prompts 1..90 tokens, 1..12 new tokens
        sched.add(i, int(rng.integers(1, 91)), int(rng.integers(1, 13)))
    n = NB * HKV * BS * A
    kp = W._normal_bf16(n, 3, "k_cache").reshape(NB, HKV, BS, A)
    vp = W._normal_bf16(n, 3, "v_cache").reshape(NB, HKV, BS, A)
    kc, vc = dev_bits(kp), dev_bits(vp)
    steps = finished = 0
    reused = set()
    seen_blocks = set()
    while True:
        p = sched.step()
        if p.num_seqs == 0:
            break
        tq = p.total_q
        q = W._normal_bf16(tq * HQ * A, 100 + steps, "q").reshape(tq, HQ, A)
        kn = W._normal_bf16(tq * HKV * A, 100 + steps, "k_new").reshape(tq, HKV, A)
        vn = W._normal_bf16(tq * HKV * A, 100 + steps, "v_new").reshape(tq, HKV, A)
        table = p.block_table.copy()
        cu, ctx = p.cu_seqlens_q.copy(), p.context_lens.copy()
        # GPU
        out = torch.empty(tq, HQ, A, dtype=torch.bfloat16, device="cuda")
        ws = kvc.new_workspace(p.num_seqs, tq, p.max_q_len, p.max_context_len, HQ, HKV, A, BS)
        kvc.kvc_paged_attention_varlen(out, dev_bits(q), dev_bits(kn), dev_bits(vn), kc, vc,
                                       dev_i32(table), dev_i32(cu), dev_i32(ctx), SCALE,
                                       max_q_len=p.max_q_len, max_context_len=p.max_context_len,
                                       workspace=ws)
        torch.cuda.synchronize()
        assert kvc.kvc_workspace_flags(ws) == 0
        # oracle on the same plan
        orc.append(kp, vp, kn, vn, table, cu, ctx)
        ref, _ = orc.attention(q, kp, vp, table, cu, ctx, SCALE)
        compare(host_bits(out), ref, what=f"step {steps}")
        for k in range(p.num_seqs):
            for b in table[k][table[k] >= 0].tolist():
                if b in seen_blocks and ctx[k] == 0:
                    reused.add(b)
                seen_blocks.add(b)
        finished += len(sched.complete())
        steps += 1
        assert steps < 500
    assert finished == 14
    assert kvc.kvc_num_free_blocks(alloc) == NB
    assert reused, "the trace should reuse freed blocks"
    assert np.array_equal(host_bits(kc), kp) and np.array_equal(host_bits(vc), vp)
