"""The layouts ragged paged batching replaces, run on the GPU and checked
against the oracle's ragged result.

* Left-padded batch (news.myit.tw continuous-batching article, "Continuous
  batching": the sequences of a static batch share one length, shorter ones
  are padded on the left, a padding mask hides the pads): every sequence
  holds n_max positions, its tokens right-aligned, the pad positions filled
  with NaN.  kvc_padded_decode_attention must give each row the oracle's
  attention over that sequence's own tokens (the pads get weight 0, NaN or
  not), and append the new token at position n_max - 1.
* Contiguous cache reserving the maximum length per sequence (klklkl10086
  kv_cache post, "连续内存分配"): the same tokens at the same positions, but
  each sequence's blocks consecutive instead of shuffled through the pool.
  The paged step must give the very same bits as with the shuffled table
  (placement is invisible), and match the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev_bits, dev_i32, host_bits, oracle_run, run_steps

pytestmark = pytest.mark.gpu

CTX = [0, 1, 15, 16, 17, 100, 255, 511, 1023, 1024, 1500, 3000]


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def _ragged(hq, hkv, bs, seed):
    return W.make_step_workload("ragged", [(c, 1) for c in CTX], num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=128, block_size=bs, seed=seed)


def _gather(wl, s, p):
    """(K, V) rows of cached position p of sequence s, through its table."""
    st = wl.steps[0]
    blk = st.block_table[s, p // wl.block_size]
    return wl.k_pool[blk, :, p % wl.block_size, :], wl.v_pool[blk, :, p % wl.block_size, :]


@pytest.mark.parametrize("geom", [(32, 8, 16), (8, 2, 4), (32, 1, 16), (32, 1, 4)],
                         ids=["gqa4", "gqa4_bs4", "mqa", "mqa_bs4"])
def test_left_padded_batch_matches_the_ragged_oracle(kvc, orc, geom):
    hq, hkv, bs = geom
    wl = _ragged(hq, hkv, bs, seed=51)
    st = wl.steps[0]
    (ref,), _, _ = oracle_run(orc, wl)
    b = len(CTX)
    n_max = -(-(max(CTX) + 1) // bs) * bs
    pages = n_max // bs
    pad = np.array([n_max - (c + 1) for c in CTX], dtype=np.int32)
    kd = np.full((b * pages, hkv, bs, 128), W.BF16_NAN, dtype=np.uint16)
    vd = kd.copy()
    for s, c in enumerate(CTX):
        for p in range(c):  # cached token p sits at padded position pad + p
            pp = pad[s] + p
            kd[s * pages + pp // bs, :, pp % bs, :], vd[s * pages + pp // bs, :, pp % bs, :] = \
                _gather(wl, s, p)
    k_cache, v_cache = dev_bits(kd), dev_bits(vd)
    q = dev_bits(st.q)
    out = torch.empty_like(q)
    ws = torch.empty(kvc.kvc_padded_workspace_size(b, n_max, hq, hkv, 128, bs), dtype=torch.uint8,
                     device="cuda")
    kvc.kvc_padded_decode_attention(out, q, dev_bits(st.k_new), dev_bits(st.v_new), k_cache,
                                    v_cache, dev_i32(pad), wl.scale, n_max=n_max, workspace=ws)
    torch.cuda.synchronize()
    mx, mean = compare(host_bits(out), ref, what=f"left-padded batch {geom}")
    kc = host_bits(k_cache)
    for s in range(b):  # the new token went to position n_max - 1
        assert np.array_equal(kc[s * pages + pages - 1, :, bs - 1, :], st.k_new[s])
    print(f"left-padded {geom}: n_max {n_max}, {int(pad.sum())} pad positions of "
          f"{b * n_max}, max {mx:.3e} mean {mean:.3e}", flush=True)


def test_contiguous_reserved_cache_equals_the_shuffled_pool(kvc, orc):
    hq, hkv, bs = 32, 8, 16
    wl = _ragged(hq, hkv, bs, seed=52)
    st = wl.steps[0]
    (g_paged,), _, _ = run_steps(kvc, wl)
    (ref,), _, _ = oracle_run(orc, wl)
    b = len(CTX)
    reserve = -(-(max(CTX) + 1) // bs)  # blocks per sequence: the longest one's
    kc = np.full((b * reserve, hkv, bs, 128), W.BF16_NAN, dtype=np.uint16)
    vc = kc.copy()
    table = (np.arange(b)[:, None] * reserve + np.arange(reserve)[None, :]).astype(np.int32)
    for s, c in enumerate(CTX):
        for p in range(c):
            kc[table[s, p // bs], :, p % bs, :], vc[table[s, p // bs], :, p % bs, :] = _gather(wl, s, p)
    contiguous = W.Workload("contiguous", hq, hkv, 128, bs, wl.scale, kc, vc,
                            [W.Step(q=st.q, k_new=st.k_new, v_new=st.v_new,
                                    cu_seqlens_q=st.cu_seqlens_q, context_lens=st.context_lens,
                                    block_table=table)])
    (g_contig,), _, _ = run_steps(kvc, contiguous)
    assert np.array_equal(g_contig, g_paged), "contiguous layout changes the result"
    mx, mean = compare(g_contig, ref, what="contiguous reserved cache")
    used = sum(-(-(c + 1) // bs) for c in CTX)
    print(f"contiguous: {b * reserve} blocks reserved, {used} used; bitwise equal to the "
          f"shuffled pool; max {mx:.3e} mean {mean:.3e}", flush=True)


def test_padded_batch_rejects_before_launch(kvc):
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros(2 * 4, 2, 16, 128, dtype=torch.bfloat16, device="cuda")
    pad = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    assert kvc.kvc_padded_workspace_size(2, 60, 8, 2, 128, 16) == 0   # n_max not whole pages
    assert kvc.kvc_padded_workspace_size(2, 64, 8, 2, 16, 16) == 0    # head_dim 16
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_padded_decode_attention(q, q, None, None, cache, cache, pad, 0.1, n_max=64,
                                        workspace=ws[:100])
    assert e.value.status == kvc.KVC_ERR_WORKSPACE
