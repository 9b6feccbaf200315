"""Seeded synthetic inputs for the ragged paged-attention step.

This module only draws inputs: sequence lengths, a shuffled physical block
numbering, block tables, and bf16 values for q, cached K/V and new K/V.  It
holds none of the attention arithmetic and imports neither the product package
nor the oracle, so both sides can be fed the same bytes from here.

Recipe (fixed draw order per workload: lengths, block permutation, q, cached
K, cached V, k_new, v_new):
  * lengths and the permutation come from ``numpy.random.default_rng(seed)``;
  * tensor values are fp32 N(0,1) rounded once to bf16 (round-to-nearest-even,
    ``torch.Tensor.to(torch.bfloat16)``), drawn in fixed 4 Mi-element chunks,
    each from its own ``torch.Generator`` seeded from (seed, tensor, chunk), so
    the bytes do not depend on how many threads draw them;
  * physical block ids are a seeded permutation of ``arange(num_blocks)``,
    handed to each sequence's logical blocks in order; a few spare blocks are
    left unreferenced;
  * pool slots of positions already cached hold random values; every other
    slot of a referenced block (the new tokens' slots and the tail of the last
    block) holds 8192.0; unreferenced blocks hold NaN.  A correct step never
    lets either poison reach an output.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os

import numpy as np
import torch

BF16_NAN = np.uint16(0x7FC0)
BF16_8192 = np.uint16(0x4600)  # 8192.0 = 2^13: sign 0, exponent 127+13, mantissa 0

_CHUNK = 1 << 22
_STREAMS = {"q": 1, "k_cache": 2, "v_cache": 3, "k_new": 4, "v_new": 5}


def bf16_bits(x: torch.Tensor | np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE) and return the raw bits as uint16."""
    t = torch.as_tensor(x, dtype=torch.float32)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(n: int, seed: int, stream: str, threads: int | None = None) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(j):
        lo, hi = j * _CHUNK, min(n, (j + 1) * _CHUNK)
        g = torch.Generator().manual_seed((seed * 1_000_003 + _STREAMS[stream] * 7_919 + j)
                                          & 0x7FFF_FFFF_FFFF)
        vals = torch.randn(hi - lo, generator=g, dtype=torch.float32)
        out[lo:hi] = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    workers = threads or min(16, os.cpu_count() or 1)
    if nchunks <= 1 or workers <= 1:
        for j in range(nchunks):
            fill(j)
    else:
        with _cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


@dataclasses.dataclass
class Step:
    """Host arrays of one call: rows of every sequence in cu_seqlens_q order."""
    q: np.ndarray             # [Tq, Hq, A] uint16 (bf16 bits)
    k_new: np.ndarray         # [Tq, Hkv, A]
    v_new: np.ndarray         # [Tq, Hkv, A]
    cu_seqlens_q: np.ndarray  # [S+1] int32
    context_lens: np.ndarray  # [S] int32, tokens cached before the call
    block_table: np.ndarray   # [S, max_blocks] int32

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q).astype(np.int32)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


@dataclasses.dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    k_pool: np.ndarray  # [NB, Hkv, bs, A] uint16, state before the first step
    v_pool: np.ndarray
    steps: list
    extra: dict = dataclasses.field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])


def _tables(final_lens, block_size, rng, spare, shared=None):
    """Block tables covering each sequence's final length.

    ``shared``: optional (num_shared_blocks, list of sequence indices) — those
    sequences' first num_shared_blocks logical blocks map to one common set of
    physical blocks (a refcounted prefix)."""
    nblk = [(int(L) + block_size - 1) // block_size for L in final_lens]
    max_blocks = max(1, max(nblk) if nblk else 1)
    n_shared, sharers = shared if shared else (0, [])
    sharers = set(sharers)
    needed = n_shared + sum(n - (n_shared if s in sharers else 0) for s, n in enumerate(nblk))
    num_blocks = needed + spare
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((len(final_lens), max_blocks), -1, dtype=np.int32)
    nxt = 0
    prefix_ids = perm[:n_shared]
    nxt = n_shared
    for s, n in enumerate(nblk):
        start = 0
        if s in sharers:
            table[s, :n_shared] = prefix_ids
            start = n_shared
        k = n - start
        table[s, start:n] = perm[nxt:nxt + k]
        nxt += k
    # unreferenced tail entries of a row point at a valid block (never read)
    table[table < 0] = perm[0] if num_blocks else 0
    return table, num_blocks, nblk


def make_step_workload(name, specs, *, num_q_heads, num_kv_heads, head_dim,
                       block_size, seed, scale=None, spare_blocks=None,
                       shared=None, rng=None):
    """One-call workload: ``specs`` is a list of (context_len, q_len) pairs.

    ``shared`` = (num_prefix_blocks, [sequence indices]) makes those sequences
    share their first blocks (the cached prefix must cover them).  ``rng`` is
    the generator the lengths were drawn from (the permutation comes next from
    the same stream)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    ctx = np.array([c for c, _ in specs], dtype=np.int32)
    ql = np.array([n for _, n in specs], dtype=np.int32)
    final = ctx + ql
    spare = spare_blocks if spare_blocks is not None else max(2, len(specs) // 8)
    table, nb, nblk = _tables(final, block_size, rng, spare, shared)
    tq = int(ql.sum())
    q = _normal_bf16(tq * num_q_heads * head_dim, seed, "q").reshape(tq, num_q_heads, head_dim)
    k_pool = _normal_bf16(nb * num_kv_heads * block_size * head_dim, seed, "k_cache")
    v_pool = _normal_bf16(nb * num_kv_heads * block_size * head_dim, seed, "v_cache")
    k_pool = k_pool.reshape(nb, num_kv_heads, block_size, head_dim)
    v_pool = v_pool.reshape(nb, num_kv_heads, block_size, head_dim)
    valid = np.zeros((nb, block_size), dtype=bool)
    ref = np.zeros(nb, dtype=bool)
    for s in range(len(specs)):
        ids = table[s, :nblk[s]]
        ref[ids] = True
        c = int(ctx[s])
        full = min(c // block_size, nblk[s])
        valid[ids[:full]] = True
        if full < nblk[s] and c % block_size:
            valid[ids[full], : c % block_size] = True
    for pool in (k_pool, v_pool):
        np.copyto(pool, BF16_8192,
                  where=np.broadcast_to((~valid)[:, None, :, None], pool.shape))
        np.copyto(pool, BF16_NAN,
                  where=np.broadcast_to((~ref)[:, None, None, None], pool.shape))
    k_new = _normal_bf16(tq * num_kv_heads * head_dim, seed, "k_new").reshape(tq, num_kv_heads, head_dim)
    v_new = _normal_bf16(tq * num_kv_heads * head_dim, seed, "v_new").reshape(tq, num_kv_heads, head_dim)
    cu = np.zeros(len(specs) + 1, dtype=np.int32)
    np.cumsum(ql, out=cu[1:])
    step = Step(q=q, k_new=k_new, v_new=v_new, cu_seqlens_q=cu, context_lens=ctx,
                block_table=table)
    return Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=block_size,
                    scale=scale if scale is not None else 1.0 / math.sqrt(head_dim),
                    k_pool=k_pool, v_pool=v_pool, steps=[step])


# ----------------------------------------------------------------------------
# The five configurations.
# ----------------------------------------------------------------------------

def toy(seed: int = 0) -> Workload:
    """1 sequence, 7-token prompt, 1 head, A=16, block size 4: chunks of 4 and
    3 tokens, then 8 decode steps (15 tokens, 4 blocks, at the end).

    extra["f32"] holds the unrounded fp32 q/k/v of all 15 tokens and
    extra["full"] the bf16 bits [15, 1, 16] of each, for unchunked
    comparisons."""
    rng = np.random.default_rng(seed)
    n_prompt, n_dec, bs, a = 7, 8, 4, 16
    total = n_prompt + n_dec
    nb = 8
    perm = rng.permutation(nb).astype(np.int32)
    table = perm[:4].reshape(1, 4).copy()
    g = torch.Generator().manual_seed(seed)
    q32 = torch.randn(total, 1, a, generator=g)
    k32 = torch.randn(total, 1, a, generator=g)
    v32 = torch.randn(total, 1, a, generator=g)
    qb, kb, vb = bf16_bits(q32), bf16_bits(k32), bf16_bits(v32)
    pool_k = np.full((nb, 1, bs, a), BF16_NAN, dtype=np.uint16)
    pool_k[table[0]] = BF16_8192
    pool_v = pool_k.copy()
    steps = []
    spans = [(0, 4), (4, 7)] + [(t, t + 1) for t in range(7, total)]
    for lo, hi in spans:
        steps.append(Step(q=qb[lo:hi].copy(), k_new=kb[lo:hi].copy(), v_new=vb[lo:hi].copy(),
                          cu_seqlens_q=np.array([0, hi - lo], dtype=np.int32),
                          context_lens=np.array([lo], dtype=np.int32),
                          block_table=table.copy()))
    return Workload(name="toy", num_q_heads=1, num_kv_heads=1, head_dim=a, block_size=bs,
                    scale=0.25, k_pool=pool_k, v_pool=pool_v, steps=steps,
                    extra={"f32": (q32.numpy(), k32.numpy(), v32.numpy()),
                           "full": (qb, kb, vb), "table": table})


def decode_mha(seed: int = 1, num_seqs: int = 64) -> Workload:
    """Decode-only batch, Llama-2-7B layer shape: 32/32 heads, A=128, bs=16,
    context U{512..4096}, one new token per sequence."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(512, 4096, size=num_seqs, endpoint=True)
    return make_step_workload("decode_mha", [(int(c), 1) for c in ctx], num_q_heads=32,
                              num_kv_heads=32, head_dim=128, block_size=16, seed=seed, rng=rng)


def decode_gqa(seed: int = 2, num_seqs: int = 256) -> Workload:
    """GQA decode: 32/8 heads, A=128, bs=16, context lognormal with median
    1024 and sigma 0.8, rounded and clipped to [16, 8192]."""
    rng = np.random.default_rng(seed)
    ctx = np.clip(np.rint(np.exp(rng.normal(math.log(1024.0), 0.8, size=num_seqs))), 16, 8192)
    return make_step_workload("decode_gqa", [(int(c), 1) for c in ctx], num_q_heads=32,
                              num_kv_heads=8, head_dim=128, block_size=16, seed=seed, rng=rng)


def decode_mqa(seed: int = 5, num_seqs: int = 256) -> Workload:
    """MQA decode (one kv head for all 32 q heads, 1/32 of the MHA cache per
    token): 32/1 heads, A=128, bs=16, context lognormal with median 4096 and
    sigma 0.8, rounded and clipped to [64, 32768]."""
    rng = np.random.default_rng(seed)
    ctx = np.clip(np.rint(np.exp(rng.normal(math.log(4096.0), 0.8, size=num_seqs))), 64, 32768)
    return make_step_workload("decode_mqa", [(int(c), 1) for c in ctx], num_q_heads=32,
                              num_kv_heads=1, head_dim=128, block_size=16, seed=seed, rng=rng)


def mixed(seed: int = 3, num_decode: int = 512, chunk: int = 512,
          chunk_ctx=(0, 512, 1024, 3584)) -> Workload:
    """Mixed continuous-batching step, token budget 2560: 4 prefill chunks of
    512 rows at cached lengths {0, 512, 1024, 3584} followed by 512 decode rows
    with context U{128..4096}; 32/8 heads, A=128, bs=16."""
    rng = np.random.default_rng(seed)
    dctx = rng.integers(128, 4096, size=num_decode, endpoint=True)
    specs = [(int(c), chunk) for c in chunk_ctx] + [(int(c), 1) for c in dctx]
    return make_step_workload("mixed", specs, num_q_heads=32, num_kv_heads=8,
                              head_dim=128, block_size=16, seed=seed, rng=rng)


def long_prefill(seed: int = 4, prompt: int = 32768, chunk: int = 2048) -> Workload:
    """One sequence with a 32768-token prompt fed as sequential 2048-token
    chunks (cached length 2048*k for chunk k); 32/8 heads, A=128, bs=16."""
    rng = np.random.default_rng(seed)
    nb_seq = prompt // 16
    spare = 16
    nb = nb_seq + spare
    perm = rng.permutation(nb).astype(np.int32)
    table = perm[:nb_seq].reshape(1, nb_seq).copy()
    hq, hkv, a, bs = 32, 8, 128, 16
    q = _normal_bf16(prompt * hq * a, seed, "q").reshape(prompt, hq, a)
    k_new = _normal_bf16(prompt * hkv * a, seed, "k_new").reshape(prompt, hkv, a)
    v_new = _normal_bf16(prompt * hkv * a, seed, "v_new").reshape(prompt, hkv, a)
    k_pool = np.full((nb, hkv, bs, a), BF16_NAN, dtype=np.uint16)
    k_pool[table[0]] = BF16_8192
    v_pool = k_pool.copy()
    steps = []
    for k in range(prompt // chunk):
        lo, hi = k * chunk, (k + 1) * chunk
        steps.append(Step(q=q[lo:hi], k_new=k_new[lo:hi], v_new=v_new[lo:hi],
                          cu_seqlens_q=np.array([0, chunk], dtype=np.int32),
                          context_lens=np.array([lo], dtype=np.int32),
                          block_table=table))
    return Workload(name="long_prefill", num_q_heads=hq, num_kv_heads=hkv, head_dim=a,
                    block_size=bs, scale=1.0 / math.sqrt(a), k_pool=k_pool, v_pool=v_pool,
                    steps=steps)


def shared_prefix(seed: int = 4, num_seqs: int = 16, prefix: int = 2048,
                  suffix: int = 256, table: np.ndarray | None = None,
                  num_blocks: int | None = None) -> Workload:
    """16 sequences share a 2048-token prefix (128 blocks, written once by the
    first call, a prefill of sequence 0 alone); the second call runs the 16
    suffix chunks of 256 rows at cached length 2048 over the shared blocks.

    ``table`` / ``num_blocks``: a block table [num_seqs, prefix/16 + suffix
    blocks] built elsewhere (for instance by a block allocator, the prefix
    blocks shared by every row) over a pool of num_blocks blocks, used
    instead of the seeded permutation."""
    rng = np.random.default_rng(seed + 1000)
    hq, hkv, a, bs = 32, 8, 128, 16
    n_prefix = prefix // bs
    n_suffix = (suffix + bs - 1) // bs
    mb = n_prefix + n_suffix
    if table is None:
        nb = n_prefix + num_seqs * n_suffix + 8
        perm = rng.permutation(nb).astype(np.int32)
        table = np.empty((num_seqs, mb), dtype=np.int32)
        table[:, :n_prefix] = perm[:n_prefix]
        for s in range(num_seqs):
            table[s, n_prefix:] = perm[n_prefix + s * n_suffix: n_prefix + (s + 1) * n_suffix]
    else:
        table = np.ascontiguousarray(table, dtype=np.int32)
        nb = int(num_blocks)
        if table.shape != (num_seqs, mb) or table.min() < 0 or table.max() >= nb:
            raise ValueError("table must be [num_seqs, prefix + suffix blocks] of ids < num_blocks")
        if not (table[:, :n_prefix] == table[:1, :n_prefix]).all():
            raise ValueError("every row must start with the same prefix blocks")
    tq = prefix + num_seqs * suffix
    q = _normal_bf16(tq * hq * a, seed + 1000, "q").reshape(tq, hq, a)
    k_new = _normal_bf16(tq * hkv * a, seed + 1000, "k_new").reshape(tq, hkv, a)
    v_new = _normal_bf16(tq * hkv * a, seed + 1000, "v_new").reshape(tq, hkv, a)
    k_pool = np.full((nb, hkv, bs, a), BF16_NAN, dtype=np.uint16)
    k_pool[np.unique(table)] = BF16_8192
    v_pool = k_pool.copy()
    first = Step(q=q[:prefix], k_new=k_new[:prefix], v_new=v_new[:prefix],
                 cu_seqlens_q=np.array([0, prefix], dtype=np.int32),
                 context_lens=np.array([0], dtype=np.int32),
                 block_table=table[:1].copy())
    cu = np.arange(num_seqs + 1, dtype=np.int32) * suffix
    second = Step(q=q[prefix:], k_new=k_new[prefix:], v_new=v_new[prefix:],
                  cu_seqlens_q=cu, context_lens=np.full(num_seqs, prefix, dtype=np.int32),
                  block_table=table)
    return Workload(name="shared_prefix", num_q_heads=hq, num_kv_heads=hkv, head_dim=a,
                    block_size=bs, scale=1.0 / math.sqrt(a), k_pool=k_pool, v_pool=v_pool,
                    steps=[first, second],
                    extra={"prefix_blocks": n_prefix, "suffix_blocks": n_suffix})


def split_into_calls(wl: Workload, per_call) -> Workload:
    """The one step of ``wl`` fed as successive calls: ``per_call[k][s]`` new
    rows of sequence s in call k (0 allowed), taken in order from the step's
    rows of s, with the cached length advanced by the rows of earlier calls.
    The pool and the table are unchanged (the table already covers the final
    lengths)."""
    st = wl.steps[0]
    ql = st.q_lens
    per_call = np.asarray(per_call, dtype=np.int64)
    if per_call.ndim != 2 or per_call.shape[1] != st.num_seqs or (per_call < 0).any() \
            or not (per_call.sum(axis=0) == ql).all():
        raise ValueError("per_call must be [calls, num_seqs] and sum to each sequence's rows")
    done = np.zeros(st.num_seqs, dtype=np.int64)
    steps = []
    for k in range(per_call.shape[0]):
        rows = np.concatenate([np.arange(st.cu_seqlens_q[s] + done[s],
                                         st.cu_seqlens_q[s] + done[s] + per_call[k, s])
                               for s in range(st.num_seqs)]).astype(np.int64)
        cu = np.zeros(st.num_seqs + 1, dtype=np.int32)
        np.cumsum(per_call[k], out=cu[1:])
        steps.append(Step(q=st.q[rows].copy(), k_new=st.k_new[rows].copy(),
                          v_new=st.v_new[rows].copy(), cu_seqlens_q=cu,
                          context_lens=(st.context_lens + done).astype(np.int32),
                          block_table=st.block_table.copy()))
        done += per_call[k]
    return dataclasses.replace(wl, steps=steps)


CONFIGS = {1: toy, 2: decode_mha, 3: decode_gqa, 4: mixed, 5: long_prefill, "5b": shared_prefix}
