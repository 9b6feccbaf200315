"""The no-allocation entry point (kvc_paged_attention_varlen_noalloc) against
the workspace entry point (kvc_paged_attention_varlen) on the same inputs.

Two calls in a row on one GPU share the library's static scratch: first the
full mixed continuous-batching step (4 prefill chunks of 512 rows plus 512
decode rows, 32/8 heads, 43 MB of scratch), then a smaller step (fewer
sequences, shorter contexts, a different head ratio), so the second call
runs over whatever the first left in the scratch.  Each output must equal
the workspace entry point's bit for bit (same kernels, same plan; the
no-allocation call runs them all on the caller's stream, which does not
change any result) and match the oracle within the attention tolerance; the
appended pools must equal the oracle's.  A step that needs more scratch than
the static array holds is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DevStep, compare, dev_bits, host_bits, oracle_run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def _call(kvc, wl, k_cache, v_cache, noalloc):
    st = wl.steps[0]
    d = DevStep(st)
    out = torch.empty_like(d.q)
    if noalloc:
        kvc.kvc_paged_attention_varlen_noalloc(out, d.q, d.k_new, d.v_new, k_cache, v_cache,
                                               d.table, d.cu, d.ctx, wl.scale,
                                               max_q_len=st.max_q_len,
                                               max_context_len=st.max_context_len)
    else:
        ws = kvc.new_workspace(st.num_seqs, st.total_q, st.max_q_len, st.max_context_len,
                               wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size)
        kvc.kvc_paged_attention_varlen(out, d.q, d.k_new, d.v_new, k_cache, v_cache, d.table,
                                       d.cu, d.ctx, wl.scale, max_q_len=st.max_q_len,
                                       max_context_len=st.max_context_len, workspace=ws)
        torch.cuda.synchronize()
        assert kvc.kvc_workspace_flags(ws) == 0
    torch.cuda.synchronize()
    return host_bits(out)


def test_noalloc_equals_workspace_entry_two_calls(kvc, orc):
    big = W.mixed()
    small = W.make_step_workload("small", [(40, 17), (700, 1), (0, 1), (129, 64), (2000, 1)],
                                 num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                                 seed=77)
    for wl in (big, small):
        st = wl.steps[0]
        need = kvc.kvc_workspace_size(st.num_seqs, st.total_q, st.max_q_len, st.max_context_len,
                                      wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size)
        assert 0 < need <= kvc.NOALLOC_SCRATCH_BYTES
        kc_w, vc_w = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
        kc_n, vc_n = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
        g_w = _call(kvc, wl, kc_w, vc_w, noalloc=False)
        g_n = _call(kvc, wl, kc_n, vc_n, noalloc=True)
        (r,), kp, vp = oracle_run(orc, wl)
        mx, mean = compare(g_n, r, what=f"{wl.name} no-alloc")
        assert np.array_equal(g_n, g_w), f"{wl.name}: no-alloc output differs from the workspace entry"
        assert np.array_equal(host_bits(kc_n), kp) and np.array_equal(host_bits(vc_n), vp)
        print(f"{wl.name}: {need} bytes of scratch, {st.total_q} rows, bitwise equal to the "
              f"workspace entry, max {mx:.3e} mean {mean:.3e}", flush=True)
        del kc_w, vc_w, kc_n, vc_n


def test_noalloc_refuses_a_step_beyond_the_scratch(kvc):
    """1024 sequences with contexts up to 131071 over 32 q heads need about
    546 MB of split-K partials, more than the static array: refused with
    KVC_ERR_WORKSPACE, nothing launched (the output keeps its contents)."""
    s, hq, hkv, a, bs = 1024, 32, 1, 128, 16
    need = kvc.kvc_workspace_size(s, s, 1, 131071, hq, hkv, a, bs)
    assert need > kvc.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(s, hq, a, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    cache = torch.zeros(4, hkv, bs, a, dtype=torch.bfloat16, device="cuda")
    table = torch.zeros(s, 1, dtype=torch.int32, device="cuda")
    cu = torch.arange(s + 1, dtype=torch.int32, device="cuda")
    ctx = torch.zeros(s, dtype=torch.int32, device="cuda")
    with pytest.raises(kvc.KvcError) as ei:
        kvc.kvc_paged_attention_varlen_noalloc(out, q, None, None, cache, cache, table, cu, ctx,
                                               0.1, max_q_len=1, max_context_len=131071)
    assert ei.value.status == kvc.KVC_ERR_WORKSPACE
    assert "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
