"""Attention parity: the HIP path against the fp64 oracle, element by element.

Bar: max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3 over the
compared rows, bf16 inputs and bf16 output.  The small cases span several
tiles, partitions and ragged tails; the six workloads run at full size
(every row for the decode, mixed and shared-prefix steps; for the 32K-token
prompt every row of its first two chunks and the first and last row of every
32-position tile of the others; appended pools bit for bit)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, host_bits, oracle_run, run_steps

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def _case(kvc, orc, name, specs, hq, hkv, a, bs, seed=7, scale=None):
    wl = W.make_step_workload(name, specs, num_q_heads=hq, num_kv_heads=hkv, head_dim=a,
                              block_size=bs, seed=seed, scale=scale)
    (g,), _, _ = run_steps(kvc, wl)
    (r,), _, _ = oracle_run(orc, wl)
    return compare(g, r, what=name)


# decode edges: blocks (4, 16), 32-token steps, short items that leave some
# of the four waves without keys (one active wave up to L = 32, three at
# L = 257), the 1024-token wave share and the 4096-token work item (a
# sequence of L = c + 1 tokens has ceil(L / 4096) items)
DEC_LENS = [0, 1, 5, 15, 16, 17, 255, 256, 257, 511, 512, 600, 1500, 1023, 1024, 1025, 4095,
            4096, 4097, 8200]
PRE_SPECS = [(0, 2), (0, 63), (0, 64), (0, 65), (5, 130), (300, 200), (17, 1)]
# chunks of equal length: the host sizes rule decode rows out
PRE_ONLY = [(0, 77), (5, 77), (63, 77), (64, 77), (300, 77), (1000, 77), (1500, 77)]
MIXED_SPECS = [(10, 0), (0, 1), (17, 5), (64, 1), (0, 0), (129, 77), (3000, 1), (0, 300),
               (700, 2), (255, 1), (1024, 129)]
SMALL = [
    ("decode_mha", [(c, 1) for c in DEC_LENS], 4, 4, 128, 16),
    ("decode_gqa2_bs4", [(c, 1) for c in DEC_LENS], 4, 2, 128, 4),
    ("decode_gqa4", [(c, 1) for c in DEC_LENS], 8, 2, 128, 16),
    ("decode_gqa8", [(c, 1) for c in DEC_LENS], 16, 2, 128, 16),
    ("decode_gqa16", [(c, 1) for c in DEC_LENS], 16, 1, 128, 16),
    # MQA / large group ratios: one wave carries 32 q heads as two MFMA column groups
    ("decode_mqa32", [(c, 1) for c in DEC_LENS], 32, 1, 128, 16),
    ("decode_g32_bs4", [(c, 1) for c in DEC_LENS], 64, 2, 128, 4),
    ("decode_g64", [(c, 1) for c in DEC_LENS[:9]], 64, 1, 128, 16),
    ("mixed_mqa32", MIXED_SPECS, 32, 1, 128, 16),
    ("prefill_mha", PRE_SPECS, 2, 2, 128, 16),
    ("prefill_gqa2", PRE_SPECS, 4, 2, 128, 16),
    ("prefill_gqa4_bs4", PRE_SPECS, 8, 2, 128, 4),
    ("prefill_gqa8", PRE_SPECS, 8, 1, 128, 16),
    ("mixed_gqa4", MIXED_SPECS, 8, 2, 128, 16),
    # chunks only (no decode row): the 8-wave prefill workgroups, P.V a tile
    # late on half the waves, V tiles in four buffers (tile counts 2..25)
    ("chunks_only_mha", PRE_ONLY, 2, 2, 128, 16),
    ("chunks_only_gqa2_bs4", PRE_ONLY, 4, 2, 128, 4),
    ("chunks_only_gqa4", PRE_ONLY, 8, 2, 128, 16),
    ("chunks_only_g32", PRE_ONLY, 32, 1, 128, 16),
    ("chunks_only_a64_gqa4_bs4", PRE_ONLY, 8, 2, 64, 4),
    ("chunks_only_a16_gqa2", PRE_ONLY, 4, 2, 16, 16),
    ("chunks_only_a256_gqa4", PRE_ONLY, 8, 2, 256, 16),
    ("chunks_only_one_seq", [(2000, 131)], 8, 2, 128, 16),
    ("mixed_mha_bs4", MIXED_SPECS, 2, 2, 128, 4),
    ("a16_mixed", [(0, 7), (4, 3), (7, 1), (30, 1), (100, 40), (0, 1), (257, 1)], 1, 1, 16, 4),
    ("a16_gqa2_bs16", [(0, 7), (4, 3), (7, 1), (30, 1), (100, 40), (600, 1)], 4, 2, 16, 16),
    ("a16_gqa4_bs4", [(0, 70), (33, 1), (2, 2)], 4, 1, 16, 4),
    # The host rules decode rows out when total_q > (num_seqs - 1) * max_q_len + 1.
    # At the bound one decode row is still possible and must be served; one row
    # past it the step holds chunks only.
    ("bound_one_decode", [(50, 4), (300, 1)], 8, 2, 128, 16),
    ("bound_chunks_only", [(50, 4), (300, 2)], 8, 2, 128, 16),
    ("bound_empty_seq", [(50, 4), (300, 0), (10, 3), (2000, 1)], 8, 2, 128, 16),
    ("a16_bound_one_decode", [(9, 3), (40, 1)], 2, 1, 16, 4),
    # head dims 16, 64 and 256, block sizes 4 and 16, G = 1, 4 and 32 (at 16 a
    # K row fills half of one 32-dim step and a 32-row K load spans two blocks)
    ("a16_decode_g1_bs16", [(c, 1) for c in DEC_LENS], 4, 4, 16, 16),
    ("a16_decode_g4_bs4", [(c, 1) for c in DEC_LENS], 8, 2, 16, 4),
    ("a16_decode_g32", [(c, 1) for c in DEC_LENS], 32, 1, 16, 16),
    ("a16_decode_g32_bs4", [(c, 1) for c in DEC_LENS], 64, 2, 16, 4),
    ("a16_mixed_g32_bs16", MIXED_SPECS, 32, 1, 16, 16),
    ("a64_decode_g1_bs16", [(c, 1) for c in DEC_LENS], 4, 4, 64, 16),
    ("a64_decode_g4_bs4", [(c, 1) for c in DEC_LENS], 8, 2, 64, 4),
    ("a64_decode_g32", [(c, 1) for c in DEC_LENS[:9]], 32, 1, 64, 16),
    ("a64_prefill_g1_bs4", PRE_SPECS, 2, 2, 64, 4),
    ("a64_prefill_g4_bs16", PRE_SPECS, 8, 2, 64, 16),
    ("a64_mixed_g32_bs16", MIXED_SPECS, 32, 1, 64, 16),
    ("a256_decode_g1_bs16", [(c, 1) for c in DEC_LENS], 2, 2, 256, 16),
    ("a256_decode_g4_bs4", [(c, 1) for c in DEC_LENS], 8, 2, 256, 4),
    ("a256_decode_g32", [(c, 1) for c in DEC_LENS[:9]], 32, 1, 256, 16),
    ("a256_prefill_g1_bs16", PRE_SPECS, 2, 2, 256, 16),
    ("a256_prefill_g4_bs4", PRE_SPECS, 8, 2, 256, 4),
    ("a256_mixed_g32_bs4", MIXED_SPECS, 32, 1, 256, 4),
]


@pytest.mark.parametrize("name,specs,hq,hkv,a,bs", SMALL, ids=[c[0] for c in SMALL])
def test_small(kvc, orc, name, specs, hq, hkv, a, bs):
    _case(kvc, orc, name, specs, hq, hkv, a, bs)


def test_planner_over_several_passes(kvc, orc):
    """More sequences (2500) and prefill work items (4200) than the planner's
    1024 threads cover in one pass, in shuffled order, so its offsets carry
    from pass to pass (sequences, decode items, merge descriptors) and the
    cost sort spans several passes over the items."""
    rng = np.random.default_rng(11)
    specs = [(int(c), 33) for c in rng.integers(0, 40, 2100)]
    specs += [(int(c), 1) for c in rng.integers(0, 1500, 400)]
    specs = [specs[i] for i in rng.permutation(len(specs))]
    _case(kvc, orc, "many_seqs", specs, 8, 2, 128, 16)


def test_scale_variants(kvc, orc):
    _case(kvc, orc, "scale0", [(20, 1), (0, 40), (300, 1)], 4, 2, 128, 16, scale=0.0)
    _case(kvc, orc, "scale_big", [(20, 1), (0, 40), (300, 1)], 4, 2, 128, 16, scale=0.5)


# A scale <= 0 takes the kernels' other softmax order (scores scaled before the
# maximum); every decode and prefill instance, mixed and chunks-only calls.
@pytest.mark.parametrize("a", [16, 64, 128, 256])
@pytest.mark.parametrize("scale", [0.0, -0.09])
def test_nonpositive_scale(kvc, orc, a, scale):
    mixed = [(20, 1), (0, 40), (300, 1), (1100, 1), (70, 100)]
    _case(kvc, orc, f"scale{scale}_a{a}_mixed", mixed, 8, 2, a, 16, scale=scale)
    _case(kvc, orc, f"scale{scale}_a{a}_chunks", [(0, 70), (130, 70), (700, 70)], 8, 2, a, 4,
          scale=scale)


@pytest.mark.parametrize("a", [16, 64, 128, 256])
def test_prefill_beside_a_full_decode(kvc, orc, a):
    """Enough decode rows (300) for the decode to fill the chip, so the chunks
    run beside it on the side stream with the 4-wave prefill workgroups (at
    most one per compute unit at head_dim 128, by an LDS reservation); the
    small cases above, with a few decode rows, run the prefill first with the
    8-wave ones."""
    rng = np.random.default_rng(40 + a)
    specs = [(int(c), 1) for c in rng.integers(0, 300, 300)] + [(0, 100), (150, 70), (33, 129)]
    _case(kvc, orc, f"overlap_a{a}", specs, 8, 2, a, 16)


def _rising_keys(wl, top, seed=5):
    """Every K row of every sequence becomes s_p * w: one fixed unit direction w
    per kv head and a magnitude s_p rising linearly with the position p up to
    `top` at the longest sequence's end.  A query's scores then rise (or fall)
    steadily along its keys, so the running maximum moves many times inside
    each tile, partition and work item and the split-K partials carry very
    different maxima."""
    import dataclasses
    rng = np.random.default_rng(seed)
    st = wl.steps[0]
    hkv, a, bs = wl.num_kv_heads, wl.head_dim, wl.block_size
    w = rng.standard_normal((hkv, a))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    cu, ctx = st.cu_seqlens_q, st.context_lens
    lmax = int((ctx + np.diff(cu)).max())
    kp, kn = wl.k_pool.copy(), st.k_new.copy()
    for s_ in range(st.num_seqs):
        c, n = int(ctx[s_]), int(cu[s_ + 1] - cu[s_])
        pos = np.arange(c + n)
        rows = W.bf16_bits((top * (pos + 1) / lmax)[:, None, None] * w[None].astype(np.float32))
        kp[st.block_table[s_, pos[:c] // bs], :, pos[:c] % bs, :] = rows[:c]
        kn[cu[s_]:cu[s_] + n] = rows[c:]
    return dataclasses.replace(wl, k_pool=kp, steps=[dataclasses.replace(st, k_new=kn)])


@pytest.mark.parametrize("a", [16, 64, 128, 256])
def test_rising_scores(kvc, orc, a):
    """Scores that climb by about 100 (log2 units) along each sequence: the
    lazy rescale fires again and again in every kernel, and the merge combines
    partials whose maxima differ by far more than the rescale slack."""
    specs = [(5000, 1), (1500, 1), (300, 1), (0, 90), (600, 150), (4100, 1)]
    wl = W.make_step_workload(f"rising_a{a}", specs, num_q_heads=8, num_kv_heads=2,
                              head_dim=a, block_size=16, seed=9)
    wl = _rising_keys(wl, top=800.0 * math.sqrt(a / 128))
    (g,), _, _ = run_steps(kvc, wl)
    (r,), _, _ = oracle_run(orc, wl)
    compare(g, r, what=wl.name)


def test_toy_chunked_then_decode(kvc, orc):
    """Chunks of 4 and 3 tokens (block size 4), then 8 decode calls; every call
    against the oracle and the chunked rows against the unchunked prefill."""
    wl = W.toy(0)
    g, _, _ = run_steps(kvc, wl)
    r, _, _ = oracle_run(orc, wl)
    for i, (gi, ri) in enumerate(zip(g, r)):
        compare(gi, ri, what=f"toy call {i}")
    qb, kb, vb = wl.extra["full"]
    un = W.Step(q=qb[:7].copy(), k_new=kb[:7].copy(), v_new=vb[:7].copy(),
                cu_seqlens_q=np.array([0, 7], np.int32), context_lens=np.array([0], np.int32),
                block_table=wl.extra["table"])
    (ru,), _, _ = oracle_run(orc, wl, [un])
    compare(np.concatenate(g[:2]), ru, what="toy chunked vs unchunked")
    # decode step t equals the last row of the unchunked prefill over t+1 tokens
    for t in range(7, 15):
        un = W.Step(q=qb[:t + 1].copy(), k_new=kb[:t + 1].copy(), v_new=vb[:t + 1].copy(),
                    cu_seqlens_q=np.array([0, t + 1], np.int32),
                    context_lens=np.array([0], np.int32), block_table=wl.extra["table"])
        (ru,), _, _ = oracle_run(orc, wl, [un])
        compare(g[2 + t - 7], ru[t:t + 1], what=f"toy decode {t}")


@pytest.mark.parametrize("cfg", ["decode_mha", "decode_gqa", "decode_mqa", "mixed"])
def test_full_workload(kvc, orc, cfg):
    wl = getattr(W, cfg)()
    (g,), _, _ = run_steps(kvc, wl)
    (r,), _, _ = oracle_run(orc, wl)
    mx, mean = compare(g, r, what=cfg)
    print(f"{cfg}: max {mx:.3e} mean {mean:.3e}", flush=True)


def _tile_edge_rows(n, tile=32):
    """First and last row of every `tile`-position block of an n-row chunk:
    each prefill wave (and so each workgroup) of the chunk writes at least
    two compared rows."""
    sel = np.zeros(n, dtype=bool)
    sel[0::tile] = True
    sel[tile - 1::tile] = True
    sel[n - 1] = True
    return sel


@pytest.mark.timeout(900)
def test_long_prefill_chunks(kvc, orc):
    """32768-token prompt in 16 chunks of 2048 (cached length 2048*k): every
    row of chunks 0 and 1, the first and last row of every 32-position tile
    of chunks 2-15 (128 rows each), and the K/V pools after the 16 chunks bit
    for bit against the oracle's appends."""
    wl = W.long_prefill()
    g, kc, vc = run_steps(kvc, wl)
    sels = [np.ones(st.total_q, dtype=bool) if k < 2 else _tile_edge_rows(st.total_q)
            for k, st in enumerate(wl.steps)]
    r, kp, vp = oracle_run(orc, wl, row_select=sels)
    total = 0
    for k, (gk, rk, sel) in enumerate(zip(g, r, sels)):
        mx, mean = compare(gk, rk, rows=sel, what=f"chunk {k}")
        total += int(sel.sum())
        print(f"chunk {k}: {int(sel.sum())} of {sel.size} rows compared, max {mx:.3e} "
              f"mean {mean:.3e}", flush=True)
    assert np.array_equal(host_bits(kc), kp), "K pool after 16 chunks differs from the oracle's"
    assert np.array_equal(host_bits(vc), vp), "V pool after 16 chunks differs from the oracle's"
    print(f"long prompt: {total} rows compared; pools bit-exact ({kp.nbytes * 2} bytes)",
          flush=True)


@pytest.mark.timeout(900)
def test_shared_prefix_all_rows_product_allocator(kvc, orc):
    """16 sequences over one refcounted 2048-token prefix, 256-token suffixes.
    The table comes from the product allocator: sequence 0 takes the prefix
    blocks just in time, the other 15 share them by reference, and every
    sequence then grows by its suffix blocks (kvc_extend_tables).  Checked
    before any GPU work: 384 blocks in use instead of 2304, refcount 16 on
    every prefix block, 1 on every suffix block.  Then every row of both
    calls against the oracle, pools bit-exact, and every block freed."""
    S, prefix, suffix, bs = 16, 2048, 256, 16
    n_prefix, n_suffix = prefix // bs, suffix // bs
    nb = n_prefix + S * n_suffix + 8
    alloc = kvc.Allocator(nb, bs)
    table = np.full((S, n_prefix + n_suffix), -1, dtype=np.int32)
    held = np.zeros(S, dtype=np.int32)
    held[0] = kvc.kvc_extend_table(alloc, table[0], 0, prefix)       # written once
    for s in range(1, S):                                              # shared by reference
        kvc.kvc_share_blocks(alloc, table[0, :n_prefix])
        table[s, :n_prefix] = table[0, :n_prefix]
        held[s] = n_prefix
    kvc.kvc_extend_tables(alloc, table, held, np.full(S, prefix + suffix, dtype=np.int64))
    used = nb - kvc.kvc_num_free_blocks(alloc)
    assert used == 384 and S * (n_prefix + n_suffix) == 2304, used
    assert all(kvc.kvc_block_refcount(alloc, int(b)) == S for b in table[0, :n_prefix])
    assert all(kvc.kvc_block_refcount(alloc, int(b)) == 1 for b in table[:, n_prefix:].ravel())
    assert len(np.unique(table[:, n_prefix:])) == S * n_suffix
    wl = W.shared_prefix(table=table, num_blocks=nb)
    g, kc, vc = run_steps(kvc, wl)
    r, kp, vp = oracle_run(orc, wl)
    for k, (gk, rk) in enumerate(zip(g, r)):
        mx, mean = compare(gk, rk, what=f"call {k}")
        print(f"shared prefix call {k}: all {gk.shape[0]} rows compared, max {mx:.3e} "
              f"mean {mean:.3e}", flush=True)
    assert np.array_equal(host_bits(kc), kp) and np.array_equal(host_bits(vc), vp)
    for s in range(S):
        kvc.kvc_free_blocks(alloc, table[s, :held[s]])
    assert kvc.kvc_num_free_blocks(alloc) == nb
    alloc.close()
