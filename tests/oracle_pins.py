"""Pins for the CPU oracle: properties fixed by the pages and by mathematics.

Each ``pin_*`` function takes an ``oracle.Oracle`` handle and raises
``AssertionError`` when the oracle breaks the property.  The same functions
run against the real oracle (tests/test_oracle_pins.py) and against builds
with planted mistakes (tests/test_oracle_mutants.py), where at least one must
fail.  None of them re-types the oracle's formula: they compare against a
library routine (torch's scaled_dot_product_attention, matmul/softmax), a
closed form, a numpy reshape, an invariant the pages state, or the pages'
printed numbers.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# small helpers (input construction only)
# --------------------------------------------------------------------------

def f64(bits: np.ndarray) -> np.ndarray:
    return W.bits_to_f32(bits).astype(np.float64)


def run(orc, wl: W.Workload, steps=None, row_select=None):
    """Run the workload's steps in order through the oracle; return the list
    of outputs and the final pools."""
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    outs = []
    for st in (steps if steps is not None else wl.steps):
        orc.append(kp, vp, st.k_new, st.v_new, st.block_table, st.cu_seqlens_q,
                   st.context_lens)
        out, _ = orc.attention(st.q, kp, vp, st.block_table, st.cu_seqlens_q,
                               st.context_lens, wl.scale, row_select)
        outs.append(out)
    return outs, kp, vp


def fresh_prefill(n, hq, hkv, a, bs, seed, scale=None, ctx=0):
    return W.make_step_workload("pin", [(ctx, n)], num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=a, block_size=bs, seed=seed, scale=scale)


def sdpa(q, k, v, scale, causal=True, gqa=False):
    """torch's own attention in float64 on the CPU.  q [n,Hq,A], k/v [n,Hkv,A]."""
    tq = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    tk = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0)
    tv = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=gqa)
    return o.squeeze(0).permute(1, 0, 2).numpy()


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_sdpa_causal(orc):
    """c = 0, one sequence, MHA: equals torch SDPA with is_causal (the causal
    mask of the 'Attention' section of the continuous-batching article)."""
    wl = fresh_prefill(13, 2, 2, 16, 4, seed=11, scale=0.3)
    (out,), _, _ = run(orc, wl)
    st = wl.steps[0]
    ref = sdpa(f64(st.q), f64(st.k_new), f64(st.v_new), 0.3)
    err = np.abs(out - ref).max()
    assert err <= 1e-12, f"SDPA causal mismatch {err}"


def pin_sdpa_gqa(orc):
    """GQA 8 q heads over 2 kv heads: equals SDPA with enable_gqa, whose kv
    head for query head h is h // (Hq/Hkv)."""
    wl = fresh_prefill(11, 8, 2, 16, 4, seed=12, scale=0.25)
    (out,), _, _ = run(orc, wl)
    st = wl.steps[0]
    ref = sdpa(f64(st.q), f64(st.k_new), f64(st.v_new), 0.25, gqa=True)
    err = np.abs(out - ref).max()
    assert err <= 1e-12, f"SDPA GQA mismatch {err}"


def pin_decode_listing(orc):
    """The batch-decode demo shape of the kv_cache post ('Batch Decode'):
    batch 4, hidden 128 over 4 heads (A = 32), 10 cached tokens; after the step
    each cache holds 11 tokens and the output equals
    softmax(q K^T / sqrt(A)) V computed with torch.matmul/softmax over the
    concatenated cache."""
    bsz, h, a, hist, bs = 4, 4, 32, 10, 4
    rng = np.random.default_rng(5)
    kh = W.bf16_bits(rng.standard_normal((bsz, hist, h, a)).astype(np.float32))
    vh = W.bf16_bits(rng.standard_normal((bsz, hist, h, a)).astype(np.float32))
    qn = W.bf16_bits(rng.standard_normal((bsz, h, a)).astype(np.float32))
    kn = W.bf16_bits(rng.standard_normal((bsz, h, a)).astype(np.float32))
    vn = W.bf16_bits(rng.standard_normal((bsz, h, a)).astype(np.float32))
    nblk = math.ceil((hist + 1) / bs)
    perm = rng.permutation(bsz * nblk + 3).astype(np.int32)
    table = perm[: bsz * nblk].reshape(bsz, nblk).copy()
    nb = len(perm)
    kp = np.full((nb, h, bs, a), W.BF16_NAN, dtype=np.uint16)
    vp = kp.copy()
    # history written by a prefill call of the oracle (c = 0, n = 10 each)
    cu_hist = (np.arange(bsz + 1) * hist).astype(np.int32)
    orc.append(kp, vp, kh.reshape(bsz * hist, h, a), vh.reshape(bsz * hist, h, a),
               table, cu_hist, np.zeros(bsz, dtype=np.int32))
    cu = np.arange(bsz + 1, dtype=np.int32)
    ctx = np.full(bsz, hist, dtype=np.int32)
    orc.append(kp, vp, kn, vn, table, cu, ctx)
    kg, vg = orc.gather(kp, vp, table, ctx + 1)
    assert kg.shape[0] == bsz * (hist + 1), "cache length after the step is not 11"
    out, _ = orc.attention(qn, kp, vp, table, cu, ctx, 1.0 / math.sqrt(a))
    # the listing: K_cache = cat([K_hist, k_new]); scores = q K^T / sqrt(d)
    K = torch.cat([torch.from_numpy(f64(kh)), torch.from_numpy(f64(kn))[:, None]], dim=1)
    V = torch.cat([torch.from_numpy(f64(vh)), torch.from_numpy(f64(vn))[:, None]], dim=1)
    K = K.permute(0, 2, 1, 3)  # [b, h, 11, a]
    V = V.permute(0, 2, 1, 3)
    qq = torch.from_numpy(f64(qn))[:, :, None, :]  # [b, h, 1, a]
    scores = torch.matmul(qq, K.transpose(-2, -1).contiguous()) / (a ** 0.5)
    ref = torch.matmul(torch.softmax(scores, dim=-1), V)[:, :, 0, :].numpy()
    err = np.abs(out - ref).max()
    assert err <= 1e-12, f"decode listing mismatch {err}"
    # the gathered cache is exactly the concatenation
    assert np.array_equal(kg.reshape(bsz, hist + 1, h, a)[:, :hist], kh)
    assert np.array_equal(kg.reshape(bsz, hist + 1, h, a)[:, hist], kn)


def pin_layout_identity(orc):
    """With the identity block table, the pool is the contiguous cache cut
    into blocks: pool = K.reshape(blocks, bs, Hkv, A).transpose(0, 2, 1, 3)
    (the [batch, heads, seq, head_dim] cache of the notes, paged)."""
    L, hkv, a, bs = 24, 3, 8, 4
    rng = np.random.default_rng(7)
    k = W.bf16_bits(rng.standard_normal((L, hkv, a)).astype(np.float32))
    v = W.bf16_bits(rng.standard_normal((L, hkv, a)).astype(np.float32))
    nb = L // bs
    table = np.arange(nb, dtype=np.int32)[None, :]
    kp = np.zeros((nb, hkv, bs, a), dtype=np.uint16)
    vp = kp.copy()
    orc.append(kp, vp, k, v, table, np.array([0, L], np.int32), np.array([0], np.int32))
    assert np.array_equal(kp, k.reshape(nb, bs, hkv, a).transpose(0, 2, 1, 3)), "K layout"
    assert np.array_equal(vp, v.reshape(nb, bs, hkv, a).transpose(0, 2, 1, 3)), "V layout"
    kg, vg = orc.gather(kp, vp, table, np.array([L], np.int32))
    assert np.array_equal(kg, k) and np.array_equal(vg, v), "gather of identity layout"


def pin_append_touches_only_new_slots(orc):
    """Append is a pure write of the new rows (the kv_cache post models it as
    torch.cat): the number of changed pool elements is exactly Tq*Hkv*A for
    K and for V (old slots hold the 8192 poison, new values never equal it)."""
    wl = W.make_step_workload("pin", [(5, 3), (0, 4), (9, 1), (16, 2)], num_q_heads=4,
                              num_kv_heads=2, head_dim=8, block_size=4, seed=13)
    st = wl.steps[0]
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    orc.append(kp, vp, st.k_new, st.v_new, st.block_table, st.cu_seqlens_q, st.context_lens)
    n = st.total_q * wl.num_kv_heads * wl.head_dim
    same = lambda x, y: (x == y) | (np.isnan(W.bits_to_f32(x)) & np.isnan(W.bits_to_f32(y)))
    assert (~same(kp, wl.k_pool)).sum() == n, "K: wrong number of slots written"
    assert (~same(vp, wl.v_pool)).sum() == n, "V: wrong number of slots written"
    # and each sequence's cache is its old cache followed by its new rows
    lens = st.context_lens + st.q_lens
    kg, _ = orc.gather(kp, vp, st.block_table, lens)
    kg0, _ = orc.gather(wl.k_pool, wl.v_pool, st.block_table, st.context_lens)
    off, off0 = 0, 0
    for s in range(st.num_seqs):
        c, q = int(st.context_lens[s]), int(st.q_lens[s])
        assert np.array_equal(kg[off:off + c], kg0[off0:off0 + c])
        assert np.array_equal(kg[off + c:off + c + q],
                              st.k_new[st.cu_seqlens_q[s]:st.cu_seqlens_q[s + 1]])
        off += c + q
        off0 += c


def pin_chunked_equals_unchunked(orc):
    """The chunked-prefill example (n = 7, m = 4: chunks of 4 then 3 tokens)
    gives the same rows as the unchunked prefill — bit for bit, since each row
    sums over the same keys in the same order."""
    wl = W.toy(0)
    outs, _, _ = run(orc, wl, wl.steps[:2])
    chunked = np.concatenate(outs, axis=0)
    qb, kb, vb = wl.extra["full"]
    un = W.Step(q=qb[:7].copy(), k_new=kb[:7].copy(), v_new=vb[:7].copy(),
                cu_seqlens_q=np.array([0, 7], np.int32), context_lens=np.array([0], np.int32),
                block_table=wl.extra["table"])
    (full,), _, _ = run(orc, wl, [un])
    assert np.array_equal(chunked, full), "chunked prefill differs from unchunked"


def pin_decode_equals_last_row(orc):
    """The KV-cache argument: a decode step for token t equals the last row of
    a full prefill over t+1 tokens (the new token does not change earlier rows
    and needs only its own q with the cached K/V)."""
    wl = W.toy(0)
    outs, _, _ = run(orc, wl)
    qb, kb, vb = wl.extra["full"]
    for t in range(7, 15):
        un = W.Step(q=qb[:t + 1].copy(), k_new=kb[:t + 1].copy(), v_new=vb[:t + 1].copy(),
                    cu_seqlens_q=np.array([0, t + 1], np.int32),
                    context_lens=np.array([0], np.int32), block_table=wl.extra["table"])
        (full,), _, _ = run(orc, wl, [un])
        dec = outs[2 + (t - 7)]
        assert np.array_equal(dec[0], full[t]), f"decode step {t} != last prefill row"


def _mixed_small(seed=21, hq=4, hkv=2, a=16, bs=4):
    specs = [(7, 5), (0, 1), (12, 1), (3, 6), (0, 3), (21, 1)]
    return W.make_step_workload("pin", specs, num_q_heads=hq, num_kv_heads=hkv, head_dim=a,
                                block_size=bs, seed=seed, scale=0.35, spare_blocks=5)


def pin_permutation_invariance(orc):
    """Block-table indirection: relabelling the physical blocks (table and pool
    together) leaves the output bit-for-bit unchanged."""
    wl = _mixed_small()
    (out,), kp, vp = run(orc, wl)
    st = wl.steps[0]
    rng = np.random.default_rng(99)
    pi = rng.permutation(wl.num_blocks).astype(np.int32)
    k2 = np.empty_like(wl.k_pool)
    v2 = np.empty_like(wl.v_pool)
    k2[pi] = wl.k_pool
    v2[pi] = wl.v_pool
    st2 = W.Step(q=st.q, k_new=st.k_new, v_new=st.v_new, cu_seqlens_q=st.cu_seqlens_q,
                 context_lens=st.context_lens, block_table=pi[st.block_table])
    wl2 = W.Workload("pin", wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                     wl.scale, k2, v2, [st2])
    (out2,), kp2, _ = run(orc, wl2)
    assert np.array_equal(out, out2), "output depends on physical placement"
    assert np.array_equal(kp2[pi], kp), "appended pool not the relabelled pool"


def pin_ragged_equals_separate(orc):
    """Ragged batching: concatenating sequences with a block-diagonal mask
    equals running each sequence alone."""
    wl = _mixed_small()
    (out,), _, _ = run(orc, wl)
    st = wl.steps[0]
    for s in range(st.num_seqs):
        lo, hi = int(st.cu_seqlens_q[s]), int(st.cu_seqlens_q[s + 1])
        one = W.Step(q=st.q[lo:hi].copy(), k_new=st.k_new[lo:hi].copy(),
                     v_new=st.v_new[lo:hi].copy(),
                     cu_seqlens_q=np.array([0, hi - lo], np.int32),
                     context_lens=st.context_lens[s:s + 1].copy(),
                     block_table=st.block_table[s:s + 1].copy())
        (o1,), _, _ = run(orc, wl, [one])
        assert np.array_equal(o1, out[lo:hi]), f"sequence {s} differs alone"


def pin_gqa_equals_repeated_mha(orc):
    """GQA equals MHA whose kv heads are each repeated Hq/Hkv times."""
    wl = _mixed_small(hq=6, hkv=2)
    (out,), _, _ = run(orc, wl)
    st = wl.steps[0]
    g = 3
    rep = lambda x, ax: np.ascontiguousarray(np.repeat(x, g, axis=ax))
    st2 = W.Step(q=st.q, k_new=rep(st.k_new, 1), v_new=rep(st.v_new, 1),
                 cu_seqlens_q=st.cu_seqlens_q, context_lens=st.context_lens,
                 block_table=st.block_table)
    wl2 = W.Workload("pin", 6, 6, wl.head_dim, wl.block_size, wl.scale,
                     rep(wl.k_pool, 1), rep(wl.v_pool, 1), [st2])
    (out2,), _, _ = run(orc, wl2)
    assert np.array_equal(out, out2), "GQA differs from repeated-head MHA"


def pin_closed_forms(orc):
    """Closed forms of softmax(z)·V: the first row of a fresh sequence sees one
    key, so its output is v_0 exactly; with scale = 0 every visible key has the
    same weight, so row i is the mean of v_0..v_i; with every value equal to
    one vector the output is that vector."""
    wl = fresh_prefill(9, 2, 1, 16, 4, seed=17, scale=0.5)
    (out,), _, _ = run(orc, wl)
    st = wl.steps[0]
    v = f64(st.v_new)
    for h in range(2):
        assert np.array_equal(out[0, h], v[0, 0]), "first row is not v_0"
    wl0 = fresh_prefill(9, 2, 1, 16, 4, seed=17, scale=0.0)
    (out0,), _, _ = run(orc, wl0)
    means = np.cumsum(v[:, 0], axis=0) / np.arange(1, 10)[:, None]
    err = np.abs(out0[:, 0] - means).max()
    assert err <= 1e-14, f"scale=0 is not the running mean ({err})"
    wlc = _mixed_small(seed=23)
    kappa = W.bf16_bits(np.linspace(-3, 3, 16).astype(np.float32))
    wlc.k_pool = wlc.k_pool.copy()
    wlc.v_pool = np.broadcast_to(kappa, wlc.v_pool.shape).copy()
    stc = wlc.steps[0]
    stc.v_new = np.broadcast_to(kappa, stc.v_new.shape).copy()
    (outc,), _, _ = run(orc, wlc)
    kv = f64(kappa)
    err = np.abs(outc - kv).max()
    assert err <= 1e-14, f"constant V not reproduced ({err})"


def pin_key_shift(orc):
    """Adding one vector u to every key adds scale*q.u to every score of a
    row, which softmax ignores.  Small integers keep K+u exact in bf16."""
    rng = np.random.default_rng(31)
    specs = [(6, 3), (0, 5)]
    wl = W.make_step_workload("pin", specs, num_q_heads=2, num_kv_heads=1, head_dim=8,
                              block_size=4, seed=31, scale=0.125)
    st = wl.steps[0]
    ints = lambda shape: W.bf16_bits(rng.integers(-3, 4, size=shape).astype(np.float32))
    st.q = ints(st.q.shape)
    st.k_new = ints(st.k_new.shape)
    kp = wl.k_pool.copy()
    live = W.bits_to_f32(kp) != 8192.0
    live &= ~np.isnan(W.bits_to_f32(kp))
    kp[live] = ints(int(live.sum()))
    wl.k_pool = kp
    (out,), _, _ = run(orc, wl)
    u = rng.integers(-2, 3, size=8).astype(np.float32)
    kp2 = kp.copy()
    kp2[live] = W.bf16_bits((W.bits_to_f32(kp) + u[None, None, None, :])[live])
    st2 = W.Step(q=st.q, k_new=W.bf16_bits(W.bits_to_f32(st.k_new) + u), v_new=st.v_new,
                 cu_seqlens_q=st.cu_seqlens_q, context_lens=st.context_lens,
                 block_table=st.block_table)
    wl2 = W.Workload("pin", 2, 1, 8, 4, 0.125, kp2, wl.v_pool, [st2])
    (out2,), _, _ = run(orc, wl2)
    err = np.abs(out - out2).max()
    assert err <= 1e-12, f"output changes when every key is shifted ({err})"


def pin_cache_bytes(orc):
    """The pages' cache-size numbers (tests/golden/page_numbers.json)."""
    with open(os.path.join(GOLDEN, "page_numbers.json")) as f:
        g = json.load(f)
    for case in g["kv_bytes_per_token"]:
        got = orc.kv_bytes_per_token(case["layers"], case["kv_heads"], case["head_dim"],
                                     case["elem_bytes"])
        assert got == case["bytes"], f"{case['cite']}: {got} != {case['bytes']}"
    n7 = g["notes_formula_7b_2048"]
    got = orc.kv_bytes_per_token(n7["layers"], n7["heads"], n7["head_dim"], 2) * n7["tokens"]
    assert got == n7["bytes"], f"notes formula, 7B at 2048 tokens: {got}"
    c13 = g["llama13b_sequence"]
    tot = orc.kv_bytes_per_token(c13["layers"], c13["kv_heads"], c13["head_dim"], 2) * c13["tokens"]
    assert round(tot / 1e9, 1) == c13["gb_rounded"], f"13B sequence: {tot} B"
    for r in g["ratios_vs_mha"]:
        mha = orc.kv_bytes_per_token(1, r["q_heads"], 128, 2)
        got = orc.kv_bytes_per_token(1, r["kv_heads"], 128, 2) / mha
        assert abs(got - r["ratio"]) < 1e-15, f"{r['cite']}: ratio {got}"


ALL_PINS = [
    pin_sdpa_causal, pin_sdpa_gqa, pin_decode_listing, pin_layout_identity,
    pin_append_touches_only_new_slots, pin_chunked_equals_unchunked,
    pin_decode_equals_last_row, pin_permutation_invariance, pin_ragged_equals_separate,
    pin_gqa_equals_repeated_mha, pin_closed_forms, pin_key_shift, pin_cache_bytes,
]
