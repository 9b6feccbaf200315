"""Seeded random shapes against the oracle: many small ragged batches that mix
decode rows, prompt chunks and empty rows, chunks-only calls and wide decode
batches with a few chunks, over the supported head groupings
(G = 1, 2 or a multiple of 4), block sizes 4 and 16 and head dims 16, 64, 128
and 256,
with context lengths drawn around block, tile, partition and work-item boundaries.  Same
bar as the other parity tests (max |diff| <= 2e-2, mean <= 2e-3); the pools
after the call equal the oracle's bit for bit."""
import numpy as np
import pytest

import workloads as W
from gpu_util import compare, host_bits, oracle_run, run_steps

pytestmark = pytest.mark.gpu

N_CASES = 24
# context lengths near the edges the kernels care about: blocks (4, 16),
# prefill key tiles (64), decode wave shares (1024 per wave) and work items
# (4096)
EDGES = [0, 1, 3, 4, 5, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025,
         4095, 4096, 4097]


def _case(i, dims=None):
    rng = np.random.default_rng(1000 + i)
    g = int(rng.choice([1, 2, 4, 8, 12, 16, 32, 64]))
    hkv = int(rng.choice([1, 2, 3])) if g <= 16 else 1
    a = (16 if rng.random() < 0.25 else 128) if dims is None else int(rng.choice(dims))
    bs = int(rng.choice([4, 16]))
    n = int(rng.integers(1, 13))
    specs = []
    for _ in range(n):
        c = int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(0, 1500))
        r = rng.random()
        if r < 0.45:
            q = 1                          # decode row
        elif r < 0.55:
            q = 0                          # sequence with no new rows
        else:
            q = int(rng.integers(2, 131))  # prompt chunk
        specs.append((c, q))
    if sum(q for _, q in specs) == 0:
        specs[0] = (specs[0][0], 1)
    return dict(name=f"rand{i:02d}_g{g}_hkv{hkv}_a{a}_bs{bs}", specs=specs, hq=g * hkv,
                hkv=hkv, a=a, bs=bs, seed=2000 + i)


def _chunks_only_case(i):
    """Every sequence brings the same number of rows (>= 2), so the host sizes
    rule decode rows out and the call takes the 8-wave prefill workgroups."""
    rng = np.random.default_rng(3000 + i)
    g = int(rng.choice([1, 2, 4, 8, 32]))
    hkv = int(rng.choice([1, 2])) if g <= 8 else 1
    a = int(rng.choice([16, 64, 128, 128]))
    bs = int(rng.choice([4, 16]))
    q = int(rng.integers(2, 200))
    n = int(rng.integers(1, 7))
    specs = [(int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(0, 3000)), q)
             for _ in range(n)]
    return dict(name=f"chunks{i:02d}_g{g}_hkv{hkv}_a{a}_bs{bs}_q{q}", specs=specs, hq=g * hkv,
                hkv=hkv, a=a, bs=bs, seed=4000 + i)


def _wide_case(i):
    """300-500 sequences on 2 kv heads, nearly all decode rows plus a few
    chunks: enough decode work (at least one workgroup per compute unit) for
    the prefill to run beside it on the side stream."""
    rng = np.random.default_rng(5000 + i)
    g = int(rng.choice([1, 4, 8, 32]))
    hkv = 2
    a = int(rng.choice([16, 64, 128, 256]))
    bs = int(rng.choice([4, 16]))
    n = int(rng.integers(300, 500))
    specs = [(int(rng.integers(0, 600)), 1 if rng.random() < 0.97 else int(rng.integers(2, 200)))
             for _ in range(n)]
    specs[0] = (specs[0][0], 64)
    return dict(name=f"wide{i:02d}_g{g}_hkv{hkv}_a{a}_bs{bs}_n{n}", specs=specs, hq=g * hkv,
                hkv=hkv, a=a, bs=bs, seed=6000 + i)


CASES = [_case(i) for i in range(N_CASES)]
# head dims 64 and 256 (the matrix decode and prefill instances of those sizes)
CASES += [_case(i, dims=(64, 256)) for i in range(N_CASES, N_CASES + 12)]
# chunks only (the 8-wave prefill with P.V a tile late on half the waves)
CASES += [_chunks_only_case(i) for i in range(10)]
# wide decode batches with chunks (the prefill beside the decode)
CASES += [_wide_case(i) for i in range(8)]


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_random_shapes(kvc, orc, case):
    wl = W.make_step_workload(case["name"], case["specs"], num_q_heads=case["hq"],
                              num_kv_heads=case["hkv"], head_dim=case["a"],
                              block_size=case["bs"], seed=case["seed"])
    (g,), kc, vc = run_steps(kvc, wl)
    (r,), kp, vp = oracle_run(orc, wl)
    compare(g, r, what=case["name"])
    # the append is a bit copy: both pools equal the oracle's, untouched slots included
    assert np.array_equal(host_bits(kc), kp) and np.array_equal(host_bits(vc), vp)
