"""The benchmark's host-side accounting, checked on the CPU.

The roofline's `achieved` divides algorithmic work by kernel time, so the
work formulas are pinned here against brute force and against the closed form
of the mixed step's chunks; the single-GPU contract and the workload matching
of the counter summaries are checked too."""
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import workloads as W  # noqa: E402


@pytest.fixture(scope="module")
def bench():
    import bench as b
    return b


def _step(specs):
    ctx = np.array([c for c, _ in specs], dtype=np.int32)
    ql = np.array([q for _, q in specs], dtype=np.int32)
    return types.SimpleNamespace(context_lens=ctx, q_lens=ql)


def test_algorithmic_work_against_brute_force(bench):
    rng = np.random.default_rng(3)
    specs = [(int(c), int(q)) for c, q in zip(rng.integers(0, 3000, 40), rng.choice([0, 1, 1, 2, 7, 64, 300], 40))]
    wl = types.SimpleNamespace(num_kv_heads=8, num_q_heads=32, head_dim=128)
    alg = bench.algorithmic(wl, [_step(specs), _step(specs[:10])])
    dec_bytes = pairs = tokens = 0
    for st in (specs, specs[:10]):
        for c, q in st:
            tokens += q
            if q == 1:  # the row reads its c cached keys and its own, K and V, bf16
                dec_bytes += (c + 1) * 8 * 128 * 2 * 2
            elif q >= 2:
                for i in range(q):  # row i of a chunk sees keys 0 .. c + i
                    pairs += c + i + 1
    assert alg["tokens"] == tokens
    assert alg["decode_kv_bytes"] == dec_bytes
    assert alg["prefill_pairs"] == pairs
    assert alg["prefill_flops"] == 4 * 128 * 32 * pairs  # 2A for QK^T, 2A for P.V


def test_mixed_step_chunk_pairs_closed_form(bench):
    """4 chunks of 512 rows at cached lengths 0, 512, 1024, 3584: each chunk
    contributes 512 c + 512 * 513 / 2 visible (query, key) pairs per head."""
    specs = [(c, 512) for c in (0, 512, 1024, 3584)] + [(1000, 1)]
    wl = types.SimpleNamespace(num_kv_heads=8, num_q_heads=32, head_dim=128)
    alg = bench.algorithmic(wl, [_step(specs)])
    assert alg["prefill_pairs"] == 3_146_752
    assert alg["prefill_flops"] == 51_556_384_768


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr


def test_counter_summaries_match_their_workload_only(bench):
    for kernel in ("decode_mfma_kernel", "prefill_kernel"):
        assert bench.measured_traffic(kernel, "no_such_workload") is None


def test_chunks_only_step_keeps_the_prefill_work(bench):
    """The bench's stand-alone prefill timing runs the mixed step's chunks as
    a call of their own: the same rows in the same order, all of the step's
    prefill work and none of its decode work."""
    wl = W.make_step_workload("m", [(0, 40), (300, 1), (17, 5), (1000, 1), (64, 130), (5, 0)],
                              num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, seed=3)
    st = wl.steps[0]
    sub = bench.chunks_only_step(st)
    assert sub.num_seqs == 3 and list(sub.q_lens) == [40, 5, 130]
    assert list(sub.context_lens) == [0, 17, 64]
    full = bench.algorithmic(wl, [st])
    part = bench.algorithmic(wl, [sub])
    assert part["prefill_flops"] == full["prefill_flops"] and part["decode_kv_bytes"] == 0
    rows = np.r_[0:40, 41:46, 47:177]
    assert np.array_equal(sub.q, st.q[rows]) and np.array_equal(sub.k_new, st.k_new[rows])
    assert np.array_equal(sub.block_table, st.block_table[[0, 2, 4]])
