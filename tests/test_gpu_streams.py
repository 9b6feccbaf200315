"""The stream contract, exercised the way a caller uses it.

Three back-to-back calls on one non-default stream reuse one workspace and
one output tensor.  Each call mixes a long prefill chunk (2048 rows at a
cached length of 3072 and more, so the prefill on the library's side stream
outlasts the decode) with 120 decode rows (enough for the decode to fill the
chip, the condition for the side stream).  After each call the output is copied
to pinned host memory with a non-blocking copy on the same stream.  The test
then waits on one event recorded on that stream, never on the device, and
compares every row of every call with the oracle.  If a call returned before
its side-stream prefill was joined back, the next call's plan would overwrite
the workspace under the running prefill, or the copy would read a partly
written output, and rows would differ.  The same runs once more with
KVC_SERIAL=1 (every kernel on the caller's stream).

Pages: news.myit.tw continuous-batching article, "Chunked prefill" (chunks of
one prompt in successive steps, each over the K/V the earlier steps cached)
and "Continuous batching" (prefill chunks and decode rows in one step)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DevStep, compare, dev_bits, oracle_run

pytestmark = pytest.mark.gpu

HQ, HKV, A, BS = 4, 1, 128, 16
CALLS = 3
CHUNK = 2048


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


@pytest.fixture(scope="module")
def case(orc):
    rng = np.random.default_rng(31)
    # enough decode sequences that the decode fills the chip, so the library
    # runs the prefill on its side stream
    dec_ctx = [int(c) for c in rng.integers(100, 2000, 120)]
    specs = [(3072, CALLS * CHUNK)] + [(c, CALLS) for c in dec_ctx]
    wl = W.make_step_workload("streams", specs, num_q_heads=HQ, num_kv_heads=HKV, head_dim=A,
                              block_size=BS, seed=31)
    per_call = [[CHUNK] + [1] * len(dec_ctx) for _ in range(CALLS)]
    wl = W.split_into_calls(wl, per_call)
    ref, _, _ = oracle_run(orc, wl)
    return wl, ref


def _run_on_stream(kvc, wl):
    stream = torch.cuda.Stream()
    dev = [DevStep(st) for st in wl.steps]
    k_cache, v_cache = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
    st0 = wl.steps[0]
    ws = kvc.new_workspace(st0.num_seqs, st0.total_q, st0.max_q_len,
                           max(st.max_context_len for st in wl.steps), HQ, HKV, A, BS)
    out = torch.empty_like(dev[0].q)
    host = [torch.empty(out.shape, dtype=torch.bfloat16, pin_memory=True) for _ in wl.steps]
    torch.cuda.synchronize()  # set-up copies done; from here on only the stream orders work
    with torch.cuda.stream(stream):
        for d, h in zip(dev, host):
            assert d.q.shape == out.shape
            kvc.kvc_paged_attention_varlen(out, d.q, d.k_new, d.v_new, k_cache, v_cache, d.table,
                                           d.cu, d.ctx, wl.scale, max_q_len=d.st.max_q_len,
                                           max_context_len=max(s.max_context_len for s in wl.steps),
                                           workspace=ws, stream=stream)
            h.copy_(out, non_blocking=True)
        done = torch.cuda.Event()
        done.record(stream)
    done.synchronize()
    flags = kvc.kvc_workspace_flags(ws, stream=stream)
    assert flags == 0, f"kernel flags {flags}"
    outs = [h.view(torch.int16).numpy().view(np.uint16).copy() for h in host]
    del k_cache, v_cache
    return outs


@pytest.mark.parametrize("serial", [False, True], ids=["side_stream", "KVC_SERIAL"])
def test_back_to_back_calls_on_one_stream(kvc, case, serial, monkeypatch):
    wl, ref = case
    if serial:
        monkeypatch.setenv("KVC_SERIAL", "1")
    else:
        monkeypatch.delenv("KVC_SERIAL", raising=False)
    outs = _run_on_stream(kvc, wl)
    for k, (g, r) in enumerate(zip(outs, ref)):
        mx, mean = compare(g, r, what=f"call {k}")
        print(f"{'serial' if serial else 'overlapped'} call {k}: all {g.shape[0]} rows, "
              f"max {mx:.3e} mean {mean:.3e}", flush=True)


def test_streams_agree_bitwise(kvc, case, monkeypatch):
    """The overlapped and the serial launch orders compute the same bits."""
    wl, _ = case
    monkeypatch.delenv("KVC_SERIAL", raising=False)
    a = _run_on_stream(kvc, wl)
    monkeypatch.setenv("KVC_SERIAL", "1")
    b = _run_on_stream(kvc, wl)
    for k, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x, y), f"call {k} differs between launch orders"
