"""Host continuous-batching scheduler (CPU): the step plans follow the
policy (decode rows first, then prompt chunks, then first-come first-served
admissions under the token budget), every request is served exactly
prompt_len prefill rows and max_new_tokens - 1 decode rows, tables always
cover the planned rows, and every block returns to the allocator."""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def test_small_trace_by_hand(kvc):
    """Budget 8, block size 4: A (prompt 6, 3 tokens), B (prompt 5, 1 token)."""
    alloc = kvc.Allocator(16, 4)
    s = kvc.Scheduler(alloc, token_budget=8, max_seqs=4, max_blocks_per_seq=4)
    s.add(100, 6, 3)
    s.add(200, 5, 1)
    # step 1: A's whole prompt (6) and B's first 2 prompt rows
    p = s.step()
    assert p.request_ids.tolist() == [100, 200]
    assert p.cu_seqlens_q.tolist() == [0, 6, 8] and p.context_lens.tolist() == [0, 0]
    assert (p.block_table[0] >= 0).sum() == 2 and (p.block_table[1] >= 0).sum() == 1
    assert s.complete() == []
    # step 2: A decodes (its first token came from the last prompt chunk),
    # B finishes its prompt (3 rows) and with it its only token
    p = s.step()
    assert p.request_ids.tolist() == [100, 200]
    assert p.cu_seqlens_q.tolist() == [0, 1, 4] and p.context_lens.tolist() == [6, 2]
    assert s.complete() == [200]
    # step 3: A's last decode row, then A is done
    p = s.step()
    assert p.request_ids.tolist() == [100] and p.context_lens.tolist() == [7]
    assert s.complete() == [100]
    assert s.step().num_seqs == 0
    assert kvc.kvc_num_free_blocks(alloc) == 16


def model_plan(state, waiting, budget, max_seqs, free_blocks, reserved, bs):
    """Independent model of one step: returns [(id, rows, context)]."""
    rows = []
    left = budget
    for r in state:  # decode rows, oldest first
        if left and len(rows) < max_seqs and r["cached"] >= r["prompt"]:
            rows.append((r["id"], 1, r["cached"]))
            left -= 1
    for r in state:  # prompt chunks
        if left and len(rows) < max_seqs and r["cached"] < r["prompt"]:
            n = min(r["prompt"] - r["cached"], left)
            rows.append((r["id"], n, r["cached"]))
            left -= n
    admitted = []
    while waiting and left and len(rows) < max_seqs:
        w = waiting[0]
        need = -(-(w["prompt"] + w["max_new"] - 1) // bs)
        if free_blocks - reserved < need:
            break
        waiting.pop(0)
        admitted.append(dict(w, cached=0, generated=0, need=need))
        n = min(w["prompt"], left)
        rows.append((w["id"], n, 0))
        left -= n
    return rows, admitted


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_trace_against_model(kvc, seed):
    rng = np.random.default_rng(seed)
    bs, nb, budget, max_seqs, mb = 16, 400, 96, 12, 40
    alloc = kvc.Allocator(nb, bs)
    s = kvc.Scheduler(alloc, budget, max_seqs, mb)
    reqs = [dict(id=int(1000 + i), prompt=int(rng.integers(1, 300)),
                 max_new=int(rng.integers(1, 40))) for i in range(60)]
    for r in reqs:
        s.add(r["id"], r["prompt"], r["max_new"])
    waiting = [dict(r) for r in reqs]
    state = []            # model: running requests in admission order
    served = {r["id"]: [0, 0] for r in reqs}  # prefill rows, decode rows
    finished = []
    for step in range(10000):
        # model bookkeeping of free blocks / reservations
        taken = sum(-(-(r["cached"]) // bs) for r in state)
        reserved = sum(r["need"] for r in state) - taken
        free_blocks = kvc.kvc_num_free_blocks(alloc)
        want, admitted = model_plan(state, waiting, budget, max_seqs, free_blocks, reserved, bs)
        state += admitted
        p = s.step()
        got = [(int(i), int(p.cu_seqlens_q[k + 1] - p.cu_seqlens_q[k]), int(p.context_lens[k]))
               for k, i in enumerate(p.request_ids)]
        assert got == want, f"step {step}"
        if not got:
            break
        assert p.total_q <= budget and p.num_seqs <= max_seqs
        # tables cover the planned rows with allocated, unshared blocks
        used = []
        for k in range(p.num_seqs):
            need = -(-(p.context_lens[k] + (p.cu_seqlens_q[k + 1] - p.cu_seqlens_q[k])) // bs)
            row = p.block_table[k]
            assert (row[:need] >= 0).all() and (row[need:] == -1).all()
            used += row[:need].tolist()
            assert all(kvc.kvc_block_refcount(alloc, int(b)) == 1 for b in row[:need])
        assert len(used) == len(set(used))
        # advance the model
        by_id = {r["id"]: r for r in state}
        for rid, n, _ in got:
            r = by_id[rid]
            pre = r["cached"] < r["prompt"]
            served[rid][0 if pre else 1] += n
            r["cached"] += n
            if not pre or r["cached"] == r["prompt"]:
                r["generated"] += 1
        done = [r["id"] for r in state if r["generated"] >= r["max_new"]]
        state = [r for r in state if r["generated"] < r["max_new"]]
        fin = s.complete()
        assert sorted(fin) == sorted(done)
        finished += fin
    assert sorted(finished) == sorted(r["id"] for r in reqs)
    for r in reqs:
        assert served[r["id"]] == [r["prompt"], r["max_new"] - 1]
    assert s.num_waiting == 0 and s.num_running == 0
    assert kvc.kvc_num_free_blocks(alloc) == nb


def test_rejects_requests_that_can_never_fit(kvc):
    alloc = kvc.Allocator(8, 16)
    s = kvc.Scheduler(alloc, 64, 4, 4)
    with pytest.raises(kvc.KvcError):
        s.add(1, 60, 10)   # 69 tokens > 4 blocks of 16
    with pytest.raises(kvc.KvcError):
        s.add(2, 0, 5)
    s2 = kvc.Scheduler(alloc, 64, 4, 16)
    with pytest.raises(kvc.KvcError):
        s2.add(3, 200, 1)  # more blocks than the pool
    s.add(4, 10, 2)
    s.step()
    with pytest.raises(kvc.KvcError):  # the planned step must be completed first
        s.step()
    s.complete()
    s.close()  # held blocks go back
    assert kvc.kvc_num_free_blocks(alloc) == 8
