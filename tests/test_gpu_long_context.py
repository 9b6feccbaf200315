"""Contexts far past the benchmark workloads: decode rows at 65535 and 131071
cached tokens (16 and 32 work items of 4096 tokens, merged), a 128K row next
to short ones, and a 64-row chunk at cached length 65536 (1025 key tiles),
for GQA with 16-token blocks and MQA with 4-token blocks (whose waves walk up
to 256 table entries over four registers).  Same bar as the other parity
tests; the pools after the call equal the oracle's bit for bit."""
import numpy as np
import pytest

import workloads as W
from gpu_util import compare, host_bits, oracle_run, run_steps

pytestmark = pytest.mark.gpu

CASES = [
    ("long_gqa_bs16", [(131071, 1), (65535, 1), (5, 1), (65536, 64)], 32, 8, 16),
    ("long_mqa_bs4", [(131071, 1), (4097, 1), (65535, 1), (65536, 64)], 32, 1, 4),
]


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


@pytest.mark.parametrize("name,specs,hq,hkv,bs", CASES, ids=[c[0] for c in CASES])
def test_long_contexts(kvc, orc, name, specs, hq, hkv, bs):
    wl = W.make_step_workload(name, specs, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                              block_size=bs, seed=61)
    (g,), kc, vc = run_steps(kvc, wl)
    (r,), kp, vp = oracle_run(orc, wl)
    mx, mean = compare(g, r, what=name)
    assert np.array_equal(host_bits(kc), kp) and np.array_equal(host_bits(vc), vp)
    print(f"{name}: max {mx:.3e} mean {mean:.3e}", flush=True)
