"""Seeded synthetic inputs: deterministic, shaped like the pages' workloads,
with the poison layout the GPU tests rely on (CPU only)."""
import numpy as np

import workloads as W


def test_deterministic():
    a, b = W.decode_gqa(), W.decode_gqa()
    assert np.array_equal(a.k_pool, b.k_pool) and np.array_equal(a.steps[0].q, b.steps[0].q)
    assert np.array_equal(a.steps[0].block_table, b.steps[0].block_table)
    c = W.decode_gqa(seed=99)
    assert not np.array_equal(a.steps[0].context_lens, c.steps[0].context_lens)


def test_shapes():
    m = W.mixed()
    st = m.steps[0]
    assert st.total_q == 2560 and st.num_seqs == 516
    assert list(st.q_lens[:4]) == [512] * 4 and (st.q_lens[4:] == 1).all()
    assert list(st.context_lens[:4]) == [0, 512, 1024, 3584]
    assert st.context_lens[4:].min() >= 128 and st.context_lens[4:].max() <= 4096
    assert st.q.shape == (2560, 32, 128) and st.k_new.shape == (2560, 8, 128)
    g = W.decode_gqa().steps[0]
    assert g.context_lens.min() >= 16 and g.context_lens.max() <= 8192
    assert 700 < np.median(g.context_lens) < 1400
    t = W.toy()
    assert [s.total_q for s in t.steps] == [4, 3] + [1] * 8
    assert [int(s.context_lens[0]) for s in t.steps] == [0, 4] + list(range(7, 15))
    lp = W.long_prefill()
    assert len(lp.steps) == 16 and lp.steps[-1].context_lens[0] == 30720
    sp = W.shared_prefix()
    tab = sp.steps[1].block_table
    assert (tab[:, :128] == tab[0, :128]).all()
    assert len(np.unique(tab)) == 128 + 16 * 16


def test_poison_layout():
    wl = W.make_step_workload("p", [(5, 3), (16, 1)], num_q_heads=1, num_kv_heads=1,
                              head_dim=16, block_size=4, seed=2, spare_blocks=3)
    st = wl.steps[0]
    f = W.bits_to_f32(wl.k_pool)
    ref = set(np.unique(st.block_table[0, :2]).tolist()) | set(st.block_table[1, :5].tolist())
    for b in range(wl.num_blocks):
        if b not in ref:
            assert np.isnan(f[b]).all()
    # sequence 0: 5 cached -> block 0 all random, block 1 slot 0 random, slots 1..3 poison
    b1 = st.block_table[0, 1]
    assert (f[b1, 0, 1:] == 8192.0).all() and (f[b1, 0, 0] != 8192.0).all()
