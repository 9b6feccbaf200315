"""kv_append and block gather on the GPU: bit-exact against the oracle over the
whole pool (untouched slots included)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DevStep, dev_bits, dev_i32, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


SMALL = [
    ("ragged_a128_bs16", [(5, 3), (0, 4), (9, 1), (16, 2), (0, 0), (31, 17)], 2, 128, 16),
    ("ragged_a16_bs4", [(5, 3), (0, 4), (9, 1), (16, 2), (0, 0), (31, 17)], 3, 16, 4),
    ("ragged_a128_bs4", [(1, 70), (64, 1), (3, 3)], 8, 128, 4),
    ("ragged_a16_bs16", [(0, 33), (15, 2), (16, 1)], 1, 16, 16),
    ("ragged_a64_bs4", [(5, 3), (0, 4), (9, 1), (16, 2), (0, 0), (31, 17)], 2, 64, 4),
    ("ragged_a256_bs16", [(0, 33), (15, 2), (16, 1), (40, 0), (3, 20)], 3, 256, 16),
]


def _append_case(kvc, orc, wl):
    st = wl.steps[0]
    d = DevStep(st)
    kc, vc = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
    kvc.kvc_append_kv(d.k_new, d.v_new, kc, vc, d.table, d.cu, d.ctx)
    torch.cuda.synchronize()
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    orc.append(kp, vp, st.k_new, st.v_new, st.block_table, st.cu_seqlens_q, st.context_lens)
    assert np.array_equal(host_bits(kc), kp), "K pool differs from the oracle's"
    assert np.array_equal(host_bits(vc), vp), "V pool differs from the oracle's"
    return kc, vc, kp, vp


def _gather_case(kvc, orc, kc, vc, kp, vp, table, lens):
    lens = np.asarray(lens, dtype=np.int32)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=cu[1:])
    hkv, a = kc.shape[1], kc.shape[3]
    ko = torch.empty((int(cu[-1]), hkv, a), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    kvc.kvc_gather_kv(kc, vc, dev_i32(table), dev_i32(lens),
                      torch.from_numpy(cu).cuda(), ko, vo)
    torch.cuda.synchronize()
    kg, vg = orc.gather(kp, vp, table, lens)
    assert np.array_equal(host_bits(ko), kg), "gathered K differs"
    assert np.array_equal(host_bits(vo), vg), "gathered V differs"


@pytest.mark.parametrize("name,specs,hkv,a,bs", SMALL, ids=[c[0] for c in SMALL])
def test_append_gather_small(kvc, orc, name, specs, hkv, a, bs):
    wl = W.make_step_workload(name, specs, num_q_heads=hkv, num_kv_heads=hkv, head_dim=a,
                              block_size=bs, seed=41)
    kc, vc, kp, vp = _append_case(kvc, orc, wl)
    st = wl.steps[0]
    _gather_case(kvc, orc, kc, vc, kp, vp, st.block_table, st.context_lens + st.q_lens)


def test_append_gather_mixed_step_full(kvc, orc):
    """The mixed continuous-batching step at full size (4.4 GB pool)."""
    wl = W.mixed()
    kc, vc, kp, vp = _append_case(kvc, orc, wl)
    st = wl.steps[0]
    # gather a sample of sequences: the 4 chunks and 60 decode rows
    pick = np.r_[0:4, 4:516:8]
    _gather_case(kvc, orc, kc, vc, kp, vp, np.ascontiguousarray(st.block_table[pick]),
                 (st.context_lens + st.q_lens)[pick])


def test_append_without_rows_is_noop(kvc):
    wl = W.make_step_workload("empty", [(4, 0), (0, 0)], num_q_heads=1, num_kv_heads=1,
                              head_dim=16, block_size=4, seed=3)
    st = wl.steps[0]
    kc, vc = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
    e = torch.empty((0, 1, 16), dtype=torch.bfloat16, device="cuda")
    kvc.kvc_append_kv(e, e, kc, vc, dev_i32(st.block_table), dev_i32(st.cu_seqlens_q),
                      dev_i32(st.context_lens))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(kc), wl.k_pool)
