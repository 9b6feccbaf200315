"""Invariants the pages fix, checked bit for bit on the GPU path itself:
physical placement does not matter (block-table indirection), a sequence's
rows do not depend on the other sequences of the batch (ragged batching with a
block-diagonal mask), repeated runs agree, closed forms hold exactly."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, oracle_run, run_steps

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


SPECS = [(7, 5), (0, 1), (300, 1), (3, 70), (0, 3), (1021, 1), (513, 200), (60, 0), (4000, 1)]


def _wl(seed=9, hq=8, hkv=2, a=128, bs=16, specs=SPECS):
    return W.make_step_workload("inv", specs, num_q_heads=hq, num_kv_heads=hkv, head_dim=a,
                                block_size=bs, seed=seed, spare_blocks=7)


def _relabel(wl, seed):
    pi = np.random.default_rng(seed).permutation(wl.num_blocks).astype(np.int32)
    k2, v2 = np.empty_like(wl.k_pool), np.empty_like(wl.v_pool)
    k2[pi] = wl.k_pool
    v2[pi] = wl.v_pool
    st = wl.steps[0]
    st2 = W.Step(q=st.q, k_new=st.k_new, v_new=st.v_new, cu_seqlens_q=st.cu_seqlens_q,
                 context_lens=st.context_lens, block_table=pi[st.block_table])
    return W.Workload(wl.name, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                      wl.scale, k2, v2, [st2]), pi


@pytest.mark.parametrize("geom", [(8, 2, 128, 16), (4, 4, 128, 4), (2, 1, 16, 4)])
def test_physical_placement_is_invisible(kvc, geom):
    hq, hkv, a, bs = geom
    wl = _wl(hq=hq, hkv=hkv, a=a, bs=bs)
    (g1,), kc1, _ = run_steps(kvc, wl)
    wl2, pi = _relabel(wl, 3)
    (g2,), kc2, _ = run_steps(kvc, wl2)
    if not np.array_equal(g1, g2):
        st = wl.steps[0]
        seq = np.repeat(np.arange(st.num_seqs), st.q_lens)
        bad = np.argwhere(g1 != g2)
        rows = sorted(set(int(r) for r in bad[:, 0]))
        detail = [(r, int(seq[r]), int(st.context_lens[seq[r]]), int(st.q_lens[seq[r]]))
                  for r in rows[:8]]
        raise AssertionError(f"output depends on physical block ids: {len(bad)} elements in "
                             f"{len(rows)} rows; (row, seq, ctx, q_len): {detail}")
    k1 = kc1.view(torch.int16).cpu().numpy()
    k2 = kc2.view(torch.int16).cpu().numpy()
    assert np.array_equal(k2[pi], k1), "appended pool is not the relabelled pool"


def test_batch_composition_is_invisible(kvc):
    wl = _wl()
    (g,), _, _ = run_steps(kvc, wl)
    st = wl.steps[0]
    # each sequence alone, and the batch in reverse order
    for s in range(st.num_seqs):
        lo, hi = int(st.cu_seqlens_q[s]), int(st.cu_seqlens_q[s + 1])
        if hi == lo:
            continue
        one = W.Step(q=st.q[lo:hi].copy(), k_new=st.k_new[lo:hi].copy(),
                     v_new=st.v_new[lo:hi].copy(), cu_seqlens_q=np.array([0, hi - lo], np.int32),
                     context_lens=st.context_lens[s:s + 1].copy(),
                     block_table=st.block_table[s:s + 1].copy())
        (g1,), _, _ = run_steps(kvc, wl, [one])
        assert np.array_equal(g1, g[lo:hi]), f"sequence {s} changes when run alone"
    order = list(range(st.num_seqs))[::-1]
    ql = st.q_lens[order]
    cu = np.zeros(len(order) + 1, np.int32)
    np.cumsum(ql, out=cu[1:])
    rows = np.concatenate([np.arange(st.cu_seqlens_q[s], st.cu_seqlens_q[s + 1]) for s in order])
    rev = W.Step(q=st.q[rows].copy(), k_new=st.k_new[rows].copy(), v_new=st.v_new[rows].copy(),
                 cu_seqlens_q=cu, context_lens=st.context_lens[order].copy(),
                 block_table=st.block_table[order].copy())
    (gr,), _, _ = run_steps(kvc, wl, [rev])
    assert np.array_equal(gr, g[rows]), "output depends on the order of the batch"


def test_repeatable(kvc):
    wl = _wl(seed=12)
    (g1,), _, _ = run_steps(kvc, wl)
    (g2,), _, _ = run_steps(kvc, wl)
    assert np.array_equal(g1, g2)


def test_first_row_is_v0_exactly(kvc):
    """A fresh sequence's first row sees one key with weight exactly 1: the
    output is v_0 bit for bit, on the prefill path (q_len > 1) and on the
    decode path (q_len = 1)."""
    wl = W.make_step_workload("v0", [(0, 9), (0, 1), (0, 130)], num_q_heads=8, num_kv_heads=2,
                              head_dim=128, block_size=16, seed=21)
    (g,), _, _ = run_steps(kvc, wl)
    st = wl.steps[0]
    for s in range(3):
        r = int(st.cu_seqlens_q[s])
        for h in range(8):
            assert np.array_equal(g[r, h], st.v_new[r, h // 4]), f"seq {s} head {h}"


def test_constant_values_reproduced(kvc):
    """With every value vector equal to kappa the output is kappa, up to the
    bf16 rounding of the output and of the softmax weights the prefill path
    feeds to the matrix cores (two bf16 ulps)."""
    wl = _wl(seed=14)
    kappa = W.bf16_bits(np.linspace(-3, 3, 128).astype(np.float32))
    wl.v_pool = np.broadcast_to(kappa, wl.v_pool.shape).copy()
    st = wl.steps[0]
    st.v_new = np.broadcast_to(kappa, st.v_new.shape).copy()
    (g,), _, _ = run_steps(kvc, wl)
    gv = W.bits_to_f32(g)
    kv = W.bits_to_f32(kappa)
    ulp = np.abs(kv) * 2.0 ** -6 + 1e-30
    assert (np.abs(gv - kv) <= ulp).all()


def test_no_poison_leaks(kvc):
    """Unreferenced blocks hold NaN, unused slots of referenced blocks 8192:
    neither reaches an output."""
    wl = _wl(seed=15)
    (g,), _, _ = run_steps(kvc, wl)
    gv = W.bits_to_f32(g)
    assert np.isfinite(gv).all()
    assert np.abs(gv).max() < 100.0


DEC_N = [1, 2, 15, 16, 63, 64, 65, 300, 1023, 1024, 1500, 4097]


def test_decode_equals_last_prefill_row(kvc, orc):
    """Row n of a prefill over tokens 0..n (the chunk that ends at token n)
    and the decode row of token n over n cached tokens are the same function
    (news.myit.tw article, "KV cache": with the cache, the new token's
    attention is the last row of the full computation).  On the GPU they run
    through different kernels (prefill: 32x32x16 products over 64-key tiles;
    decode: 16x16x32 products over split-K partitions), and both round the
    softmax weights to bf16 for the P.V product and sum the same rounded
    weights in the denominator.  Bound: the two results may sit on either side
    of a bf16 rounding of the output (one ulp of the value) and differ before
    rounding by the weight rounding (relative 2^-9 per weight, which with few
    keys moves the output by up to about |v_i - v_j| / 4 * 2^-8); hence
    |decode - prefill| <= 2^-7 |oracle| + 4e-3 per element and a mean under
    3e-4, both well inside the 2e-2 / 2e-3 oracle tolerance."""
    hq, hkv, a, bs = 8, 2, 128, 16
    wd = W.make_step_workload("dec", [(n, 1) for n in DEC_N], num_q_heads=hq, num_kv_heads=hkv,
                              head_dim=a, block_size=bs, seed=41)
    (gd,), kc, vc = run_steps(kvc, wd)
    (rd,), _, _ = oracle_run(orc, wd)
    compare(gd, rd, what="decode rows")
    st = wd.steps[0]
    # the chunk: the last m tokens of each sequence (its K/V already in the pool)
    ms = [min(64, n + 1) for n in DEC_N]
    extra_q = W._normal_bf16(sum(ms) * hq * a, 42, "q").reshape(sum(ms), hq, a)
    q, kn, vn, last = [], [], [], []
    o = 0
    for s, (n, m) in enumerate(zip(DEC_N, ms)):
        for p in range(n + 1 - m, n + 1):
            if p == n:
                kn.append(st.k_new[s])
                vn.append(st.v_new[s])
            else:
                blk = st.block_table[s, p // bs]
                kn.append(wd.k_pool[blk, :, p % bs, :])
                vn.append(wd.v_pool[blk, :, p % bs, :])
        q.append(extra_q[o:o + m - 1])
        q.append(st.q[s:s + 1])
        o += m
        last.append(o - 1)
    cu = np.concatenate([[0], np.cumsum(ms)]).astype(np.int32)
    pre = W.Step(q=np.concatenate(q), k_new=np.stack(kn), v_new=np.stack(vn), cu_seqlens_q=cu,
                 context_lens=np.array([n + 1 - m for n, m in zip(DEC_N, ms)], np.int32),
                 block_table=st.block_table)
    # the chunk rewrites the same K/V into the pool the decode call left
    (gp,), _, _ = run_steps(kvc, wd, [pre], k_cache=kc, v_cache=vc)
    gl = gp[last]
    dv = W.bits_to_f32(gd).astype(np.float64)
    pv = W.bits_to_f32(gl).astype(np.float64)
    diff = np.abs(dv - pv)
    bound = 2.0 ** -7 * np.abs(rd) + 4e-3
    print(f"decode vs last prefill row: max {diff.max():.3e} mean {diff.mean():.3e} "
          f"identical elements {np.mean(gd == gl):.3f}", flush=True)
    assert (diff <= bound).all(), f"max excess {(diff - bound).max():.3e}"
    assert diff.mean() <= 3e-4, diff.mean()
