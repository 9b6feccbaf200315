#!/usr/bin/env python3
"""Benchmark of one ragged paged-attention step on one MI355X.

Default workload: the mixed continuous-batching step (token budget 2560):
4 prefill chunks of 512 rows at cached lengths {0, 512, 1024, 3584} plus 512
decode rows with context U{128..4096}; 32 q heads / 8 kv heads, head_dim 128,
bf16, block size 16, physical blocks shuffled.  One step = one call of
kvc_paged_attention_varlen: append of the 2560 new K/V rows, the MFMA prefill
kernel, the split-K decode kernel and its merge (plus the planning kernel).
Inputs are seeded synthetic data already resident in HBM.

Prints one JSON line: whole-step tokens/s (K steps timed back to back), the
roofline of the dominant kernel (its launches timed with HIP events on the
stream they run on, during a second pass over the same K steps), the
decode KV-read bandwidth, the prefill MFMA utilisation, and the CPU oracle
timed on a bounded sample of the same step on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "mixed-step tokens/s; decode KV-read GB/s vs HBM peak; prefill MFMA util"
HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure

WORKLOADS = {
    "mixed": ("mixed continuous-batching step: 4 prefill chunks x 512 rows at cached "
              "lengths {0,512,1024,3584} + 512 decode rows with context U{128..4096}; "
              "32 q / 8 kv heads, head_dim 128, bf16, block 16", W.mixed),
    "decode_mha": ("decode batch, Llama-2-7B layer: 64 sequences, 32/32 heads, head_dim 128, "
                   "context U{512..4096}, block 16", W.decode_mha),
    "decode_gqa": ("GQA decode: 256 sequences, 32/8 heads, head_dim 128, context lognormal "
                   "(median 1024, sigma 0.8, clip [16, 8192]), block 16", W.decode_gqa),
    "decode_mqa": ("MQA decode: 256 sequences, 32 q heads on 1 kv head, head_dim 128, context "
                   "lognormal (median 4096, sigma 0.8, clip [64, 32768]), block 16", W.decode_mqa),
    "long_prefill": ("32768-token prompt as 16 sequential 2048-token chunks; 32/8 heads, "
                     "head_dim 128, block 16", W.long_prefill),
    "shared_prefix": ("16 x 256-token suffix chunks over one shared 2048-token prefix; "
                      "32/8 heads, head_dim 128, block 16", W.shared_prefix),
}


SERVE_DESC = ("continuous-batching serve loop: host scheduler (token budget 2560 rows, <= 1024 "
              "sequences per step) over a seeded trace of 4096 requests, prompts U{128..4096}, "
              "new tokens U{32..512}; 32 q / 8 kv heads, head_dim 128, bf16, block 16; one "
              "layer's attention per step")


def run_serve(args, kvc):
    """Sustained throughput of scheduler-driven steps: every step the host
    scheduler plans the rows (decode rows, prompt chunks, admissions, blocks
    just in time), the plan is copied into one of two device buffer sets, and
    the library runs the step; planning the next step overlaps the GPU."""
    budget, max_seqs, bs, hq, hkv, a = 2560, 1024, 16, 32, 8, 128
    n_req, max_prompt, max_new = 4096, 4096, 512
    rng = np.random.default_rng(6 if args.seed is None else args.seed)
    prompts = rng.integers(128, max_prompt, n_req, endpoint=True)
    news = rng.integers(32, max_new, n_req, endpoint=True)
    mb = -(-(max_prompt + max_new) // bs)
    nb = 131072  # 8.6 GB of K/V pool
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    alloc = kvc.Allocator(nb, bs)
    sched = kvc.Scheduler(alloc, budget, max_seqs, mb)
    for i in range(n_req):
        sched.add(i, int(prompts[i]), int(news[i]))
    g = torch.Generator(device="cuda").manual_seed(0)
    k_cache = torch.randn(nb, hkv, bs, a, generator=g, device="cuda").to(torch.bfloat16)
    v_cache = torch.randn(nb, hkv, bs, a, generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn(budget, hq, a, generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn(budget, hkv, a, generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn(budget, hkv, a, generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    ws = kvc.new_workspace(max_seqs, budget, budget, max_prompt + max_new, hq, hkv, a, bs)
    scale = 1.0 / math.sqrt(a)
    # two buffer sets: step i uses set i % 2 once step i - 2 has finished with it
    pin = [dict(cu=torch.empty(max_seqs + 1, dtype=torch.int32).pin_memory(),
                ctx=torch.empty(max_seqs, dtype=torch.int32).pin_memory(),
                table=torch.empty(max_seqs, mb, dtype=torch.int32).pin_memory()) for _ in range(2)]
    dev = [{k: torch.empty(v.shape, dtype=torch.int32, device="cuda") for k, v in b.items()}
           for b in pin]
    done = [torch.cuda.Event() for _ in range(2)]
    state = dict(i=0, finished=0)
    alg = dict(tokens=0, decode_rows=0, decode_bytes=0, pairs=0)

    def one_step():
        p = sched.step()
        if p.num_seqs == 0:
            return False
        k = state["i"] % 2
        done[k].synchronize()
        n, t = p.num_seqs, p.total_q
        pin[k]["cu"][:n + 1].numpy()[:] = p.cu_seqlens_q
        pin[k]["ctx"][:n].numpy()[:] = p.context_lens
        pin[k]["table"][:n].numpy()[:] = p.block_table
        for key, m in (("cu", n + 1), ("ctx", n), ("table", n)):
            dev[k][key][:m].copy_(pin[k][key][:m], non_blocking=True)
        kvc.kvc_paged_attention_varlen(out[:t], q[:t], kn[:t], vn[:t], k_cache, v_cache,
                                       dev[k]["table"][:n], dev[k]["cu"][:n + 1], dev[k]["ctx"][:n],
                                       scale, max_q_len=p.max_q_len,
                                       max_context_len=p.max_context_len, workspace=ws,
                                       stream=stream)
        done[k].record(stream)
        ql = np.diff(p.cu_seqlens_q).astype(np.int64)
        c = p.context_lens.astype(np.int64)
        alg["tokens"] += t
        d = ql == 1  # decode rows, and one-row chunks, read like decode rows
        alg["decode_rows"] += int(d.sum())
        alg["decode_bytes"] += int((c[d] + 1).sum()) * hkv * a * 2 * 2
        pr = ql >= 2
        alg["pairs"] += int((ql[pr] * c[pr] + ql[pr] * (ql[pr] + 1) // 2).sum())
        state["finished"] += len(sched.complete())
        state["i"] += 1
        return True

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    assert kvc.kvc_workspace_flags(ws) == 0
    for key in alg:
        alg[key] = 0
    fin0 = state["finished"]
    t0 = time.perf_counter()
    steps = 0
    while steps < args.steps and one_step():
        steps += 1
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    headline = dict(alg)
    fin = state["finished"] - fin0
    # kernel durations: the next K steps with HIP events around every launch
    for key in alg:
        alg[key] = 0
    kvc.kvc_profile_begin(args.steps)
    steps2 = 0
    while steps2 < args.steps and one_step():
        steps2 += 1
    torch.cuda.synchronize()
    phase_ms, ncalls = kvc.kvc_profile_end()
    dec_us = phase_ms["decode"] * 1e3 / max(steps2, 1)
    pre_us = phase_ms["prefill"] * 1e3 / max(steps2, 1)
    dec_bytes = alg["decode_bytes"] / max(steps2, 1)
    pre_flops = 4 * a * hq * alg["pairs"] / max(steps2, 1)
    if dec_us >= pre_us:
        gbps = dec_bytes / (dec_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": "decode_mfma_kernel (split-K partials)",
                    "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                    "algorithmic_bytes_per_launch": dec_bytes, "avg_launch_us": dec_us}
    else:
        tf = pre_flops / (pre_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": "prefill_kernel (bf16 MFMA)", "achieved": tf,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                    "algorithmic_flops_per_launch": pre_flops, "avg_launch_us": pre_us}
    result = {
        "metric": METRIC, "value": headline["tokens"] / elapsed, "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / max(steps, 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded request trace; random K/V and rows)",
        "config": {"workload": SERVE_DESC, "name": "serve", "requests": n_req,
                   "token_budget": budget, "max_seqs": max_seqs, "num_q_heads": hq,
                   "num_kv_heads": hkv, "head_dim": a, "block_size": bs, "pool_blocks": nb},
        "roofline": roofline,
        "serve": {"tokens_per_step": headline["tokens"] / max(steps, 1),
                  "decode_rows_per_step": headline["decode_rows"] / max(steps, 1),
                  "requests_finished_in_timed_steps": fin,
                  "running_after": sched.num_running, "waiting_after": sched.num_waiting},
        "kernels_us_per_step": {k: v * 1e3 / max(steps2, 1) for k, v in phase_ms.items()},
    }
    print(json.dumps(result), flush=True)


BASELINES_DESC = ("GQA decode batch (256 sequences, 32/8 heads, head_dim 128, context lognormal "
                  "median 1024, clip [16, 8192], block 16) run ragged and paged, against the "
                  "same rows as a left-padded batch (every sequence padded on the left to the "
                  "longest, pad positions read and masked) and on a contiguous cache reserving "
                  "8192 slots per sequence")


def time_decode_batch(kvc, ctx, hq, hkv, a, bs, steps, warmup, seed=0, reserve_len=None,
                      padded=False, phases=False):
    """Microseconds per call of one decode batch (one new token per sequence at
    the given contexts) on random GPU-drawn data.  Paged: each sequence holds
    just the blocks it needs, in shuffled pool order.  reserve_len set: a
    contiguous cache that reserves reserve_len slots per sequence (sequence i
    owns the consecutive blocks i*R .. i*R+R-1, R = reserve_len / block).
    padded: the left-padded batch (kvc_padded_decode_attention): every
    sequence holds n_max = the longest one's length, rounded up to whole
    blocks, its tokens right-aligned after pad positions that are read and
    masked.  phases: also time each kernel with HIP events in a second pass
    and return (us, {phase: us per call})."""
    s = len(ctx)
    nblk = [-(-(int(c) + 1) // bs) for c in ctx]
    g = torch.Generator(device="cuda").manual_seed(seed)
    if padded:
        n_max = max(nblk) * bs
        nb = s * max(nblk)
    elif reserve_len is None:
        nb, mb = sum(nblk), max(nblk)
        perm = torch.randperm(nb, generator=g, device="cuda").to(torch.int32).cpu().numpy()
        table = np.full((s, mb), -1, np.int32)
        o = 0
        for i, n in enumerate(nblk):
            table[i, :n] = perm[o:o + n]
            o += n
    else:
        mb = -(-int(reserve_len) // bs)
        assert max(nblk) <= mb
        nb = s * mb
        table = (np.arange(s, dtype=np.int64)[:, None] * mb + np.arange(mb)[None, :]).astype(np.int32)
    kc = torch.randn(nb, hkv, bs, a, generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn(nb, hkv, bs, a, generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn(s, hq, a, generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn(s, hkv, a, generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn(s, hkv, a, generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(a)
    if padded:
        pad = dev_i32(np.array([n_max - (int(c) + 1) for c in ctx]))
        ws = torch.empty(kvc.kvc_padded_workspace_size(s, n_max, hq, hkv, a, bs), dtype=torch.uint8,
                         device="cuda")
        call = lambda: kvc.kvc_padded_decode_attention(  # noqa: E731
            out, q, kn, vn, kc, vc, pad, scale, n_max=n_max, workspace=ws)
    else:
        cu = dev_i32(np.arange(s + 1))
        cx = dev_i32(np.asarray(ctx))
        tb = dev_i32(table)
        mc = int(max(ctx))
        ws = kvc.new_workspace(s, s, 1, mc, hq, hkv, a, bs)
        call = lambda: kvc.kvc_paged_attention_varlen(  # noqa: E731
            out, q, kn, vn, kc, vc, tb, cu, cx, scale, max_q_len=1, max_context_len=mc,
            workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / steps
    ph = None
    if phases:
        kvc.kvc_profile_begin(steps)
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        ms, n = kvc.kvc_profile_end()
        ph = {k: v * 1e3 / n for k, v in ms.items()}
    if not padded:
        assert kvc.kvc_workspace_flags(ws) == 0
    del kc, vc
    return (us, ph) if phases else us


HEADDIMS_DESC = ("decode batches of 256 sequences (one new token each) at head_dim 16, 64, 128 "
                 "and 256, block 16: GQA 32/8 heads with decode_gqa's contexts and MQA 32/1 "
                 "with decode_mqa's")


def run_headdims(args, kvc):
    """Decode kernel bandwidth per head size, GQA and MQA (random GPU-drawn
    data, shuffled paged blocks)."""
    torch.cuda.set_device(0)
    table = []
    for name, hq, hkv, seed, med, lo, hi in [("gqa", 32, 8, 2, 1024.0, 16, 8192),
                                             ("mqa", 32, 1, 5, 4096.0, 64, 32768)]:
        rng = np.random.default_rng(seed)
        ctx = [int(c) for c in np.clip(np.rint(np.exp(rng.normal(math.log(med), 0.8, size=256))),
                                       lo, hi)]
        for a in (16, 64, 128, 256):
            us, ph = time_decode_batch(kvc, ctx, hq, hkv, a, 16, args.steps, args.warmup,
                                       phases=True)
            kv_bytes = float(sum(c + 1 for c in ctx)) * hkv * a * 2 * 2
            gbps = kv_bytes / (ph["decode"] * 1e-6) / 1e9
            table.append({"heads": f"{hq}/{hkv}", "head_dim": a, "kv_bytes": kv_bytes,
                          "step_us": us, "decode_us": ph["decode"], "merge_us": ph["merge"],
                          "decode_gbps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS})
            print(f"# {name} head_dim {a}: decode {ph['decode']:.1f} us, {gbps:.0f} GB/s "
                  f"({gbps / HBM_PEAK_GBPS:.2f} of peak)", file=sys.stderr, flush=True)
    ref = next(r for r in table if r["heads"] == "32/8" and r["head_dim"] == 128)
    result = {
        "metric": METRIC, "value": 256 / (ref["step_us"] * 1e-6), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ref["step_us"] / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded lengths; GPU-drawn random K/V and rows)",
        "config": {"workload": HEADDIMS_DESC, "name": "headdims"},
        "roofline": {"bound": "hbm", "kernel": "decode kernels (GQA head_dim 128 batch)",
                     "achieved": ref["decode_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": ref["frac_hbm_peak"], "traffic": None,
                     "algorithmic_bytes_per_launch": ref["kv_bytes"],
                     "avg_launch_us": ref["decode_us"]},
        "head_dims": table,
    }
    print(json.dumps(result), flush=True)


def run_baselines(args, kvc):
    """The decode batch ragged and paged vs left-padded; paged vs contiguous
    max-length cache footprint (helpers in batching_kv_append_amd.baselines)."""
    from batching_kv_append_amd import baselines as base
    torch.cuda.set_device(0)
    hq, hkv, a, bs, max_len = 32, 8, 128, 16, 8192
    rng = np.random.default_rng(2 if args.seed is None else args.seed)
    ctx = np.clip(np.rint(np.exp(rng.normal(math.log(1024.0), 0.8, size=256))), 16, max_len)
    ctx = [int(c) for c in ctx]
    lens = [c + 1 for c in ctx]  # cached tokens after the step's append
    ragged_us = time_decode_batch(kvc, ctx, hq, hkv, a, bs, args.steps, args.warmup)
    padded_us = time_decode_batch(kvc, ctx, hq, hkv, a, bs, args.steps, args.warmup, padded=True)
    contiguous_us = time_decode_batch(kvc, ctx, hq, hkv, a, bs, args.steps, args.warmup,
                                      reserve_len=max_len + 1)
    useful, pads = base.left_padded_tokens(lens)
    paged = base.paged_cache_bytes(lens, bs, hkv, a)
    contiguous = base.contiguous_cache_bytes(len(lens), max_len, hkv, a)  # as the pages size it
    # how many such sequences fit in 64 GiB of cache, drawn from the same law
    lens_many = np.clip(np.rint(np.exp(rng.normal(math.log(1024.0), 0.8, size=200000))), 16,
                        max_len).astype(np.int64) + 1
    budget = 64 << 30
    per_token = 2 * hkv * a * 2
    fit_paged = base.sequences_that_fit(budget, (-(-int(x) // bs) * bs * per_token for x in lens_many))
    fit_contig = base.sequences_that_fit(budget, (max_len * per_token for _ in lens_many))
    kv_bytes = sum(lens) * per_token
    result = {
        "metric": METRIC, "value": len(ctx) / (ragged_us * 1e-6), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ragged_us / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded lengths; GPU-drawn random K/V and rows)",
        "config": {"workload": BASELINES_DESC, "name": "baselines", "num_seqs": len(ctx),
                   "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": a, "block_size": bs},
        "roofline": {"bound": "hbm", "kernel": "decode step (prep + decode + merge)",
                     "achieved": kv_bytes / (ragged_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": kv_bytes / (ragged_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                     "traffic": None, "algorithmic_bytes_per_launch": kv_bytes,
                     "avg_launch_us": ragged_us},
        "baselines": {
            "ragged_paged_us": ragged_us, "left_padded_us": padded_us,
            "padded_over_ragged_time": padded_us / ragged_us,
            "contiguous_max_len_cache_us": contiguous_us,
            "contiguous_over_paged_time": contiguous_us / ragged_us,
            "useful_cached_tokens": useful, "pad_tokens": pads,
            "pad_fraction_of_padded_batch": pads / (useful + pads),
            "paged_cache_bytes": paged, "contiguous_max_len_cache_bytes": contiguous,
            "contiguous_waste_fraction": 1 - kv_bytes / contiguous,
            "paged_waste_fraction": 1 - kv_bytes / paged,
            "sequences_in_64GiB_paged": fit_paged, "sequences_in_64GiB_contiguous": fit_contig,
            "insert_prompt_padding_B8_n100": base.insert_padding_tokens(8, 100),
        },
    }
    print(json.dumps(result), flush=True)


def dev_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def algorithmic(wl, steps):
    """Algorithmic work of the timed calls (per step = all calls below)."""
    hkv, hq, a = wl.num_kv_heads, wl.num_q_heads, wl.head_dim
    dec_bytes = 0
    pairs = 0
    tokens = 0
    for st in steps:
        ql = st.q_lens.astype(np.int64)
        c = st.context_lens.astype(np.int64)
        tokens += int(ql.sum())
        d = ql == 1
        dec_bytes += int((c[d] + 1).sum()) * hkv * a * 2 * 2  # K and V, bf16
        p = ql >= 2
        # row i of a chunk sees c + i + 1 keys
        pairs += int((ql[p] * c[p] + ql[p] * (ql[p] + 1) // 2).sum())
    return {"tokens": tokens, "decode_kv_bytes": dec_bytes, "prefill_pairs": pairs,
            "prefill_flops": 4 * a * hq * pairs,
            "append_bytes": tokens * hkv * a * 2 * 2 * 2}


def chunks_only_step(st):
    """The rows of the sequences of a step that bring >= 2 new tokens (its
    prefill chunks), as a step of their own."""
    ql = st.q_lens
    keep = np.nonzero(ql >= 2)[0]
    rows = np.concatenate([np.arange(st.cu_seqlens_q[s], st.cu_seqlens_q[s + 1]) for s in keep])
    cu = np.zeros(len(keep) + 1, dtype=np.int32)
    np.cumsum(ql[keep], out=cu[1:])
    return W.Step(q=st.q[rows], k_new=st.k_new[rows], v_new=st.v_new[rows], cu_seqlens_q=cu,
                  context_lens=st.context_lens[keep].copy(), block_table=st.block_table[keep].copy())


def time_prefill_calls(kvc, wl, steps, stream, k_cache=None, v_cache=None, reps=2):
    """The prefill kernel alone over chunks-only calls (no decode row, so the
    prefill runs on the caller's stream with nothing beside it): its summed
    duration per pass from HIP events around each launch, after one warm-up
    pass.  Appending the chunks' rows again writes the same bytes."""
    if k_cache is None:
        k_cache, v_cache = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
    calls = []
    for st in steps:
        q = dev_bits(st.q)
        calls.append(dict(out=torch.empty_like(q), q=q, k_new=dev_bits(st.k_new),
                          v_new=dev_bits(st.v_new), table=dev_i32(st.block_table),
                          cu=dev_i32(st.cu_seqlens_q), ctx=dev_i32(st.context_lens),
                          ws=kvc.new_workspace(st.num_seqs, st.total_q, st.max_q_len,
                                               st.max_context_len, wl.num_q_heads,
                                               wl.num_kv_heads, wl.head_dim, wl.block_size),
                          max_q=st.max_q_len, max_c=st.max_context_len))

    def one_pass():
        for c in calls:
            kvc.kvc_paged_attention_varlen(c["out"], c["q"], c["k_new"], c["v_new"], k_cache,
                                           v_cache, c["table"], c["cu"], c["ctx"], wl.scale,
                                           max_q_len=c["max_q"], max_context_len=c["max_c"],
                                           workspace=c["ws"], stream=stream)

    one_pass()
    torch.cuda.synchronize()
    kvc.kvc_profile_begin(reps * len(calls))
    for _ in range(reps):
        one_pass()
    torch.cuda.synchronize()
    phase_ms, n = kvc.kvc_profile_end()
    assert n == reps * len(calls)
    for c in calls:
        assert kvc.kvc_workspace_flags(c["ws"]) == 0
    flops = algorithmic(wl, steps)["prefill_flops"]
    us = phase_ms["prefill"] * 1e3 / reps
    tf = flops / (us * 1e-6) / 1e12
    return {"calls": len(calls), "flops": flops, "kernel_us": us, "tflops": tf,
            "frac_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(wl, steps, every, min_seconds=10.0, max_passes=8):
    """The oracle as it stands on a row sample of the same step(s), repeated
    until at least min_seconds of host time have been measured (appending the
    same rows again writes the same values, so every pass does the same work)."""
    import oracle
    orc = oracle.get()
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()   # harness copy, not timed
    t_total, rows_total, used, passes = 0.0, 0, 1, 0
    while passes < max_passes and (passes == 0 or t_total < min_seconds):
        for st in steps:
            sel = np.zeros(st.total_q, dtype=bool)
            sel[::every] = True
            t0 = time.perf_counter()
            orc.append(kp, vp, st.k_new, st.v_new, st.block_table, st.cu_seqlens_q, st.context_lens)
            _, used = orc.attention(st.q, kp, vp, st.block_table, st.cu_seqlens_q, st.context_lens,
                                    wl.scale, row_select=sel,
                                    nthreads=len(os.sched_getaffinity(0)))
            t_total += time.perf_counter() - t0
            rows_total += int(sel.sum())
        passes += 1
    return rows_total / t_total, used, rows_total, t_total, passes


def stream_read_ceiling(gib=4):
    """Practical HBM read ceiling: best GB/s of plain streaming-read kernels
    (libkvc_probe.so) over a small sweep of launch shapes, sequential and in
    random 4 KiB blocks (the decode kernel's pattern), each with plain loads
    and with non-temporal loads; the ceiling is the best of the block reads.
    None without the probe library."""
    import ctypes
    path = os.path.join(ROOT, "batching_kv_append_amd", "libkvc_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.kvcp_seq_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.kvcp_block_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    nblk = nbytes // 4096
    g = torch.Generator(device="cpu").manual_seed(0)
    perm = torch.randperm(nblk, generator=g).to(torch.int32).cuda()
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)

    def best(run, shapes, reps=5):
        out_gbps = 0.0
        for grid, unroll in shapes:
            out = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
            for _ in range(2):
                assert run(out, grid, unroll) == 0
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            for _ in range(reps):
                run(out, grid, unroll)
            e.record(stream)
            torch.cuda.synchronize()
            out_gbps = max(out_gbps, nbytes * reps / (s.elapsed_time(e) * 1e-3) / 1e9)
        return out_gbps

    res = {}
    for nt, tag in ((0, ""), (1, "_nontemporal")):
        res["sequential" + tag + "_gbps"] = best(
            lambda o, gr, u: lib.kvcp_seq_read(buf.data_ptr(), nbytes // 16, o.data_ptr(), gr, u,
                                               nt, st),
            [(2048, 8), (4096, 8), (4096, 16), (8192, 8)])
        res["random_4kib_blocks" + tag + "_gbps"] = best(
            lambda o, gr, u: lib.kvcp_block_read(buf.data_ptr(), perm.data_ptr(), nblk,
                                                 o.data_ptr(), gr, u, nt, st),
            [(1024, 4), (2048, 4), (4096, 4), (2048, 8), (4096, 2)])
    del buf, perm
    res["ceiling_gbps"] = max(res["random_4kib_blocks_gbps"],
                              res["random_4kib_blocks_nontemporal_gbps"])
    res["buffer_gib"] = gib
    return res


def mfma_ceiling():
    """Practical bf16 matrix rate: back-to-back v_mfma_f32_32x32x16_bf16 on
    register operands with 2 or 3 waves per SIMD on every CU (libkvc_probe.so),
    best TFLOP/s.  None without the probe library."""
    import ctypes
    path = os.path.join(ROOT, "batching_kv_append_amd", "libkvc_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.kvcp_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters, best = 8192, 0.0
    for per_cu in (2, 3):
        grid = cus * per_cu
        out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
        assert lib.kvcp_mfma_loop(out.data_ptr(), grid, iters, st) == 0
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(3):
            assert lib.kvcp_mfma_loop(out.data_ptr(), grid, iters, st) == 0
        e.record(stream)
        torch.cuda.synchronize()
        flops = 3 * grid * 4 * iters * 4 * 2 * 32 * 32 * 16
        best = max(best, flops / (s.elapsed_time(e) * 1e-3) / 1e12)
    return {"bf16_32x32x16_tflops": best}


def host_alloc_cost(wl, steps, reps=20):
    """Host block allocation for the step (just-in-time table growth of every
    sequence by its new tokens, one kvc_extend_tables call for all rows),
    timed on the product allocator; the blocks are released after each
    repetition so every repetition sees the same state."""
    import batching_kv_append_amd as kvc
    bs = wl.block_size
    st = steps[0]
    need = int(((st.context_lens.astype(np.int64) + st.q_lens + bs - 1) // bs).sum())
    alloc = kvc.Allocator(need + 64, bs)
    mb = st.block_table.shape[1]
    table = np.full((st.num_seqs, mb), -1, dtype=np.int32)
    held = np.zeros(st.num_seqs, dtype=np.int32)
    kvc.kvc_extend_tables(alloc, table, held, st.context_lens.astype(np.int64))
    new_lens = (st.context_lens.astype(np.int64) + st.q_lens).astype(np.int64)
    ts = []
    for _ in range(reps):
        h2 = held.copy()
        t0 = time.perf_counter()
        kvc.kvc_extend_tables(alloc, table, h2, new_lens)
        ts.append(time.perf_counter() - t0)
        new = np.concatenate([table[s, held[s]:h2[s]] for s in range(st.num_seqs)])
        kvc.kvc_free_blocks(alloc, new)
        table[h2 > held] = np.where(np.arange(mb)[None, :] < held[h2 > held][:, None],
                                    table[h2 > held], -1)
    alloc.close()
    return float(np.median(ts) * 1e6)


KERNEL_SOURCES = {
    "decode_mfma_kernel": ["batching_kv_append_amd/csrc/decode.hip", "batching_kv_append_amd/csrc/kvc_device.h"],
    "prefill_kernel": ["batching_kv_append_amd/csrc/prefill.hip", "batching_kv_append_amd/csrc/kvc_device.h"],
}


def source_digest(kernel):
    """First 16 hex digits of a SHA-256 over the kernel's sources with the
    comments and blank lines removed (so a comment edit keeps the counters
    that were taken on the same code)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", "", text)                 # line comments
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode("utf-8"))
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summaries in profiles/,
    or None when none was taken on this workload with the kernel's current
    code."""
    import glob
    key = f"traffic {kernel} workload={workload} src_sha256_16={source_digest(kernel)} "
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                if line.startswith(key):
                    fields = dict(kv.split("=", 1) for kv in line.split()[2:])
                    return int(fields["bytes_per_launch"])
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed",
                    choices=sorted(WORKLOADS) + ["serve", "baselines", "headdims"],
                    help="serve: scheduler-driven steps over a request trace (use e.g. "
                         "--steps 300 --warmup 300)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-every", type=int, default=1,
                    help="oracle timing uses every n-th row of the step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device-to-device copies (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this library runs one GPU's share of the step; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported — run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")

    import batching_kv_append_amd as kvc

    if args.workload == "serve":
        run_serve(args, kvc)
        return
    if args.workload == "baselines":
        run_baselines(args, kvc)
        return
    if args.workload == "headdims":
        run_headdims(args, kvc)
        return
    desc, make = WORKLOADS[args.workload]
    t0 = time.perf_counter()
    wl = make() if args.seed is None else make(seed=args.seed)
    steps = wl.steps if args.workload != "shared_prefix" else wl.steps[1:]
    gen_s = time.perf_counter() - t0
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    # ---- device state --------------------------------------------------------
    k_cache, v_cache = dev_bits(wl.k_pool), dev_bits(wl.v_pool)
    if args.workload == "shared_prefix":
        # the prefix is written once (untimed); the timed step is the suffix call
        st0 = wl.steps[0]
        ws0 = kvc.new_workspace(st0.num_seqs, st0.total_q, st0.max_q_len, st0.max_context_len,
                                wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size)
        q0 = dev_bits(st0.q)
        kvc.kvc_paged_attention_varlen(torch.empty_like(q0), q0, dev_bits(st0.k_new),
                                       dev_bits(st0.v_new), k_cache, v_cache,
                                       dev_i32(st0.block_table), dev_i32(st0.cu_seqlens_q),
                                       dev_i32(st0.context_lens), wl.scale,
                                       max_q_len=st0.max_q_len,
                                       max_context_len=st0.max_context_len, workspace=ws0)
    calls = []
    for st in steps:
        q = dev_bits(st.q)
        ws = kvc.new_workspace(st.num_seqs, st.total_q, st.max_q_len, st.max_context_len,
                               wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size)
        calls.append(dict(out=torch.empty_like(q), q=q, k_new=dev_bits(st.k_new),
                          v_new=dev_bits(st.v_new), table=dev_i32(st.block_table),
                          cu=dev_i32(st.cu_seqlens_q), ctx=dev_i32(st.context_lens),
                          ws=ws, max_q=st.max_q_len, max_c=st.max_context_len))
    torch.cuda.synchronize()

    def one_step():
        for c in calls:
            kvc.kvc_paged_attention_varlen(c["out"], c["q"], c["k_new"], c["v_new"], k_cache,
                                           v_cache, c["table"], c["cu"], c["ctx"], wl.scale,
                                           max_q_len=c["max_q"], max_context_len=c["max_c"],
                                           workspace=c["ws"], stream=stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    for c in calls:
        assert kvc.kvc_workspace_flags(c["ws"]) == 0

    # ---- timed region -----------------------------------------------------------
    # Headline: K steps back to back, nothing but the library's own launches.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Kernel durations: the same K steps again with HIP events recorded around
    # every launch on the stream it runs on (the events themselves add a few
    # microseconds between kernels, so this pass does not give the headline).
    kvc.kvc_profile_begin(args.steps * len(calls))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    elapsed_events = time.perf_counter() - t1
    phase_ms, ncalls = kvc.kvc_profile_end()
    assert ncalls == args.steps * len(calls), (ncalls, args.steps * len(calls))
    per_step_us = {k: v * 1e3 / args.steps for k, v in phase_ms.items()}
    # Cold caches: each step after a read of a 1 GiB scratch buffer (more than
    # the L2s and the 256 MB last-level cache hold; read only, so no dirty
    # lines are left to be written back during the step), timed by events
    # around the step alone, as when other layers run between two steps of
    # one layer.  Everything is queued before one final wait, so the GPU runs
    # scratch pass, event, step, event, ... and no host launch latency is
    # timed.
    scratch = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    probe = None
    probe_path = os.path.join(ROOT, "batching_kv_append_amd", "libkvc_probe.so")
    if os.path.exists(probe_path):
        import ctypes
        probe = ctypes.CDLL(probe_path)
        probe.kvcp_seq_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]

    def read_scratch():
        if probe is None:
            scratch.sum()
        else:
            assert probe.kvcp_seq_read(scratch.data_ptr(), scratch.numel() // 4, sink.data_ptr(),
                                       4096, 8, 0, ctypes.c_void_p(stream.cuda_stream)) == 0

    torch.cuda.synchronize()
    cold_ev = []
    for _ in range(min(args.steps, 10)):
        read_scratch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        one_step()
        e1.record(stream)
        cold_ev.append((e0, e1))
    torch.cuda.synchronize()
    cold_ms = [a.elapsed_time(b) for a, b in cold_ev]
    del scratch, sink

    # Prefill alone: the step's chunks as a chunks-only call (the default
    # mixed step's four 512-row chunks), and the 32768-token prompt's 16
    # chunks, each with the prefill kernel timed by events around its launch.
    prefill_standalone = None
    if args.workload == "mixed":
        sub = [chunks_only_step(st) for st in steps]
        prefill_standalone = {
            "mixed_step_chunks": time_prefill_calls(kvc, wl, sub, stream, k_cache, v_cache)}
        lp = W.long_prefill()
        prefill_standalone["long_prompt_16_chunks"] = time_prefill_calls(kvc, lp, lp.steps, stream)
        del lp
        torch.cuda.synchronize()

    alg = algorithmic(wl, steps)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = alg["tokens"] * args.steps / elapsed

    dec_us = per_step_us["decode"]
    merge_us = per_step_us["merge"]
    pre_us = per_step_us["prefill"]
    ceiling = stream_read_ceiling()
    mfma_ceil = mfma_ceiling()
    decode = None
    if alg["decode_kv_bytes"]:
        gbps = alg["decode_kv_bytes"] / (dec_us * 1e-6) / 1e9
        decode = {"kv_bytes_per_step": alg["decode_kv_bytes"], "partial_us": dec_us,
                  "merge_us": merge_us, "kernel_gbps": gbps,
                  "with_merge_gbps": alg["decode_kv_bytes"] / ((dec_us + merge_us) * 1e-6) / 1e9,
                  "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
                  "frac_random_4kib_read_ceiling":
                      gbps / ceiling["ceiling_gbps"] if ceiling else None}
    prefill = None
    if alg["prefill_flops"]:
        tf = alg["prefill_flops"] / (pre_us * 1e-6) / 1e12
        prefill = {"flops_per_step": alg["prefill_flops"], "visible_pairs_per_head":
                   alg["prefill_pairs"], "kernel_us": pre_us, "tflops": tf,
                   "frac_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                   "frac_measured_mfma_ceiling":
                       tf / mfma_ceil["bf16_32x32x16_tflops"] if mfma_ceil else None}
        if decode:
            prefill["note"] = ("runs on the side stream under the decode: kernel_us is its "
                               "window beside the decode, not its own speed")

    launches = len(calls)  # per step; each call launches each kernel at most once
    if decode and (not prefill or dec_us >= pre_us):
        roofline = {"bound": "hbm", "kernel": "decode_mfma_kernel (split-K partials)",
                    "achieved": decode["kernel_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": decode["frac_hbm_peak"], "traffic": measured_traffic("decode_mfma_kernel", args.workload),
                    "algorithmic_bytes_per_launch": alg["decode_kv_bytes"] / launches,
                    "avg_launch_us": dec_us / launches}
    else:
        roofline = {"bound": "mfma", "kernel": "prefill_kernel (bf16 MFMA)",
                    "achieved": prefill["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": prefill["frac_mfma_peak"],
                    "traffic": measured_traffic("prefill_kernel", args.workload),
                    "algorithmic_flops_per_launch": alg["prefill_flops"] / launches,
                    "avg_launch_us": pre_us / launches}

    # The step's own floor: its decode bytes at the HBM peak plus its prefill
    # flops at the matrix peak (the two overlap in the step, so this is a
    # lower bound on its time), against the measured step.
    floor_us = (alg["decode_kv_bytes"] / (HBM_PEAK_GBPS * 1e9)
                + alg["prefill_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
    step_roofline = {"decode_kv_bytes": alg["decode_kv_bytes"],
                     "prefill_flops": alg["prefill_flops"], "floor_us": floor_us,
                     "measured_us": ms_per_step * 1e3, "frac": floor_us / (ms_per_step * 1e3)}
    st0 = steps[0]
    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "ms_per_step_kernel_events_pass": elapsed_events * 1e3 / args.steps,
        "ms_per_step_cold_cache": float(np.median(cold_ms)),
        "ms_per_step_cold_cache_p90": float(np.percentile(cold_ms, 90)),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the pages' workloads)",
        "config": {"workload": desc, "name": args.workload, "calls_per_step": len(calls),
                   "num_seqs": int(st0.num_seqs), "tokens_per_step": alg["tokens"],
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "pool_blocks": wl.num_blocks},
        "roofline": roofline,
        "decode": decode, "prefill": prefill,
        "prefill_standalone": prefill_standalone,
        "step_roofline": step_roofline,
        # a phase with no work in this workload reports null: its empty launch
        # can sit behind the other stream's kernels, so its events time a wait
        "kernels_us_per_step": {
            k: (None if (k in ("decode", "merge") and not alg["decode_kv_bytes"])
                or (k == "prefill" and not alg["prefill_flops"]) else v)
            for k, v in per_step_us.items()},
        "host_alloc_us_per_step": host_alloc_cost(wl, steps),
        # measured streaming-read ceiling beside the data-sheet 8 TB/s
        "stream_read_ceiling": ceiling,
        # measured matrix-core rate beside the data-sheet 2.5 PFLOP/s
        "mfma_ceiling": mfma_ceil,
        "input_gen_s": gen_s,
    }
    if not args.no_cpu_baseline:
        every = max(1, args.cpu_sample_every)
        if args.workload == "long_prefill":
            every = max(every, 64)
        rate, used, nrows, secs, passes = cpu_baseline(wl, steps, every)
        rows = "every row" if every == 1 else f"every {every}-th row"
        result["cpu_baseline"] = {
            "value": rate, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{rows} of the step, {passes} pass(es): {nrows} rows in {secs:.1f} s, "
                      f"fp64 append + attention, OpenMP; host CPU {cpu_model()}"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
