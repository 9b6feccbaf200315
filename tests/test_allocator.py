"""Host block allocator: free list, reference counts, all-or-nothing
allocation, just-in-time table growth (CPU only)."""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kvc():
    import batching_kv_append_amd as m
    return m


def test_alloc_share_free_cycle(kvc):
    a = kvc.Allocator(16, 16)
    ids = kvc.kvc_alloc_blocks(a, 10)
    assert len(set(ids.tolist())) == 10 and kvc.kvc_num_free_blocks(a) == 6
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_alloc_blocks(a, 7)
    assert e.value.status == kvc.KVC_ERR_OOM and kvc.kvc_num_free_blocks(a) == 6
    kvc.kvc_share_blocks(a, ids[:4])
    assert [kvc.kvc_block_refcount(a, i) for i in ids[:5]] == [2, 2, 2, 2, 1]
    kvc.kvc_free_blocks(a, ids)
    assert kvc.kvc_num_free_blocks(a) == 12
    kvc.kvc_free_blocks(a, ids[:4])
    assert kvc.kvc_num_free_blocks(a) == 16
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_free_blocks(a, ids[:1])
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG


def test_just_in_time_growth(kvc):
    """A sequence takes a new block exactly when its last block is full."""
    a = kvc.Allocator(64, 16)
    row = np.full(8, -1, dtype=np.int32)
    held = 0
    taken = []
    for L in range(1, 129):
        before = kvc.kvc_num_free_blocks(a)
        held = kvc.kvc_extend_table(a, row, held, L)
        taken.append(before - kvc.kvc_num_free_blocks(a))
        assert held == (L + 15) // 16
    assert [i + 1 for i, t in enumerate(taken) if t] == [1, 17, 33, 49, 65, 81, 97, 113]
    with pytest.raises(kvc.KvcError):
        kvc.kvc_extend_table(a, row, held, 129)


def test_extend_tables_batch(kvc):
    """One call grows every row exactly as one call per row does, and is all
    or nothing: too few free blocks or a row too short change nothing."""
    rng = np.random.default_rng(5)
    s, mb, bs = 40, 12, 16
    ctx = rng.integers(0, 150, size=s)
    new = ctx + rng.integers(0, 40, size=s)
    a1, a2 = kvc.Allocator(600, bs), kvc.Allocator(600, bs)
    t1 = np.full((s, mb), -1, np.int32)
    t2 = t1.copy()
    h1 = np.zeros(s, np.int32)
    h2 = np.zeros(s, np.int32)
    for i in range(s):  # the cached contexts first, row by row in both
        h1[i] = kvc.kvc_extend_table(a1, t1[i], 0, int(ctx[i]))
        h2[i] = kvc.kvc_extend_table(a2, t2[i], 0, int(ctx[i]))
    for i in range(s):
        h1[i] = kvc.kvc_extend_table(a1, t1[i], int(h1[i]), int(new[i]))
    kvc.kvc_extend_tables(a2, t2, h2, new.astype(np.int64))
    assert np.array_equal(t1, t2) and np.array_equal(h1, h2)
    assert kvc.kvc_num_free_blocks(a1) == kvc.kvc_num_free_blocks(a2)
    assert (h2 == (new + bs - 1) // bs).all()
    # too few free blocks for the batch: nothing changes
    free0, t_before, h_before = kvc.kvc_num_free_blocks(a2), t2.copy(), h2.copy()
    more = new + 16 * (free0 // s + 1)
    more = np.minimum(more, mb * bs).astype(np.int64)
    if int(((more + bs - 1) // bs - h2).sum()) > free0:
        with pytest.raises(kvc.KvcError):
            kvc.kvc_extend_tables(a2, t2, h2, more)
        assert kvc.kvc_num_free_blocks(a2) == free0
        assert np.array_equal(t2, t_before) and np.array_equal(h2, h_before)
    # a row that would need more than max_blocks entries: nothing changes
    bad = new.astype(np.int64).copy()
    bad[-1] = mb * bs + 1
    with pytest.raises(kvc.KvcError):
        kvc.kvc_extend_tables(a2, t2, h2, bad)
    assert np.array_equal(t2, t_before) and np.array_equal(h2, h_before)
    assert kvc.kvc_num_free_blocks(a2) == free0


def test_prefix_sharing_footprint(kvc):
    """16 sequences share a 2048-token prefix (128 blocks) written once, each
    with a 256-token suffix: 128 + 16*16 = 384 blocks instead of 16*144."""
    a = kvc.Allocator(4096, 16)
    prefix = np.full(128, -1, dtype=np.int32)
    kvc.kvc_extend_table(a, prefix, 0, 2048)
    tables = []
    for s in range(16):
        row = np.full(144, -1, dtype=np.int32)
        row[:128] = prefix
        if s > 0:
            kvc.kvc_share_blocks(a, prefix)
        kvc.kvc_extend_table(a, row, 128, 2048 + 256)
        tables.append(row)
    assert 4096 - kvc.kvc_num_free_blocks(a) == 384
    assert all(kvc.kvc_block_refcount(a, int(b)) == 16 for b in prefix)
    assert kvc.kvc_block_refcount(a, int(tables[3][130])) == 1
    for row in tables:
        kvc.kvc_free_blocks(a, row)
    assert kvc.kvc_num_free_blocks(a) == 4096


def test_copy_on_write(kvc):
    """A block with one owner is written in place; a shared one is replaced by
    a fresh block for the writer, and the other sharers keep theirs."""
    a = kvc.Allocator(4, 16)
    (b,) = kvc.kvc_alloc_blocks(a, 1)
    assert kvc.kvc_cow_block(a, b) == (b, False)
    kvc.kvc_share_blocks(a, [b])
    nb, copied = kvc.kvc_cow_block(a, b)
    assert copied and nb != b
    assert kvc.kvc_block_refcount(a, b) == 1 and kvc.kvc_block_refcount(a, nb) == 1
    assert kvc.kvc_num_free_blocks(a) == 2
    for bad in (-1, 4, 3):  # out of range, out of range, free
        with pytest.raises(kvc.KvcError) as e:
            kvc.kvc_cow_block(a, bad)
        assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    # no free block: OOM and nothing changes
    kvc.kvc_alloc_blocks(a, 2)
    kvc.kvc_share_blocks(a, [b])
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_cow_block(a, b)
    assert e.value.status == kvc.KVC_ERR_OOM and kvc.kvc_block_refcount(a, b) == 2


@pytest.mark.parametrize("length", [0, 1, 15, 16, 17, 37, 48])
def test_fork_table(kvc, length):
    """Fork of a sequence holding `length` tokens (block size 16): full blocks
    shared, a partial last block copied on write, all or nothing."""
    a = kvc.Allocator(16, 16)
    parent = np.full(4, -1, dtype=np.int32)
    held = kvc.kvc_extend_table(a, parent, 0, length)
    free0 = kvc.kvc_num_free_blocks(a)
    child = np.full(4, -1, dtype=np.int32)
    ch, copies = kvc.kvc_fork_table(a, parent, length, child)
    nb = -(-length // 16)
    full = length // 16
    assert ch == nb == held
    assert child[:full].tolist() == parent[:full].tolist()
    for i in range(full):
        assert kvc.kvc_block_refcount(a, int(parent[i])) == 2
    if length % 16:
        assert copies == [(int(parent[full]), int(child[full]))]
        assert child[full] != parent[full]
        assert kvc.kvc_block_refcount(a, int(parent[full])) == 1
        assert kvc.kvc_block_refcount(a, int(child[full])) == 1
        assert kvc.kvc_num_free_blocks(a) == free0 - 1
    else:
        assert copies == [] and kvc.kvc_num_free_blocks(a) == free0
    # freeing both tables returns every block
    kvc.kvc_free_blocks(a, parent[:held])
    kvc.kvc_free_blocks(a, child[:ch])
    assert kvc.kvc_num_free_blocks(a) == 16


def test_fork_table_all_or_nothing(kvc):
    a = kvc.Allocator(3, 16)
    parent = np.full(4, -1, dtype=np.int32)
    kvc.kvc_extend_table(a, parent, 0, 40)  # 3 blocks, the last one partial
    child = np.full(4, -1, dtype=np.int32)
    with pytest.raises(kvc.KvcError) as e:  # the copy needs a free block
        kvc.kvc_fork_table(a, parent, 40, child)
    assert e.value.status == kvc.KVC_ERR_OOM
    assert [kvc.kvc_block_refcount(a, int(i)) for i in parent[:3]] == [1, 1, 1]
    with pytest.raises(kvc.KvcError) as e:  # child row too short
        kvc.kvc_fork_table(a, parent, 32, np.full(1, -1, dtype=np.int32))
    assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    assert [kvc.kvc_block_refcount(a, int(i)) for i in parent[:3]] == [1, 1, 1]


def test_native_driver_under_sanitizers(tmp_path):
    exe = tmp_path / "allocator_driver"
    srcs = [os.path.join(ROOT, "tests", "native", "allocator_driver.cpp"),
            os.path.join(ROOT, "batching_kv_append_amd", "csrc", "allocator.cpp"),
            os.path.join(ROOT, "batching_kv_append_amd", "csrc", "status.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "batching_kv_append_amd", "csrc"), *srcs, "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "allocator driver ok" in r.stdout
