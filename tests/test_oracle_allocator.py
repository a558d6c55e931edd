"""Pins for the oracle's block-manager model (CPU only)."""
import numpy as np
import pytest

import workloads
from oracle.allocator import BlockManagerModel, OutOfBlocks
from oracle.state import build_state
from tests.conftest import golden


def _model(nb, bs, order=None):
    return BlockManagerModel(nb, bs, list(range(nb)) if order is None else order)


def test_blocks_needed_worked_examples():
    for c in golden("pages_needed.json")["cases"]:
        m = _model(c["blocks"] + 3, c["block_size"])
        sid = m.add_seq()
        m.append(sid, c["tokens"])
        assert len(m.block_table(sid)) == c["blocks"]


def test_block_table_example_from_free_order():
    g = golden("block_table_example.json")
    order = g["block_table"] + [b for b in range(8) if b not in g["block_table"]]
    m = _model(8, g["block_size"], order)
    sid = m.add_seq()
    slots, _ = m.append(sid, g["num_tokens"])
    assert m.block_table(sid) == g["block_table"]
    for t, b, o in g["lookups"]:
        assert slots[t] == b * g["block_size"] + o


def test_parallel_sampling_sharing_example():
    g = golden("cow_example.json")
    order = g["shared_physical"] + g["exclusive_physical"]
    order += [b for b in range(16) if b not in order]
    m = _model(16, g["block_size"], order)
    parent = m.add_seq()
    m.append(parent, g["prompt_tokens"])
    seqs = [parent] + [m.fork(parent) for _ in range(g["candidates"] - 1)]
    for s in seqs:
        _, cow = m.append(s, 1)       # prompt ends on a block boundary: new block, no copy
        assert cow == []
    for b in g["shared_physical"]:
        assert m.ref[b] == g["shared_ref_count"]
    assert [m.block_table(s)[-1] for s in seqs] == g["exclusive_physical"]
    for b in g["exclusive_physical"]:
        assert m.ref[b] == g["exclusive_ref_count"]


def test_copy_on_write_steps():
    """Writing into a shared partly filled block: take a free block, copy,
    decrement the old count, repoint the table; the last sharer writes in place."""
    m = _model(10, 4)
    p = m.add_seq()
    m.append(p, 6)                                  # blocks [0, 1]; block 1 half full
    c1, c2 = m.fork(p), m.fork(p)
    assert m.ref[0] == 3 and m.ref[1] == 3
    slots, cow = m.append(c1, 1)
    assert cow == [(1, 2)] and m.block_table(c1) == [0, 2] and slots == [2 * 4 + 2]
    assert m.ref[1] == 2 and m.ref[2] == 1
    _, cow = m.append(c2, 3)                        # fills block 3 then opens block 4
    assert cow == [(1, 3)] and m.block_table(c2) == [0, 3, 4]
    slots, cow = m.append(p, 1)                     # last sharer: in place
    assert cow == [] and slots == [1 * 4 + 2] and m.ref[1] == 1
    assert m.ref[0] == 3


def test_out_of_blocks_is_atomic():
    m = _model(4, 4)
    a = m.add_seq()
    m.append(a, 10)                                 # 3 blocks
    b = m.add_seq()
    before = (list(m.free), list(m.ref), dict(m.lens))
    with pytest.raises(OutOfBlocks):
        m.append(b, 5)                              # needs 2, 1 free
    assert (list(m.free), list(m.ref), dict(m.lens)) == before
    assert m.block_table(b) == []
    # copy-on-write needs a block too
    c = m.fork(a)
    m.append(b, 4)                                  # takes the last free block
    with pytest.raises(OutOfBlocks):
        m.append(c, 1)
    assert m.ref[m.block_table(a)[-1]] == 2


def test_free_returns_blocks_to_the_back_of_the_queue():
    m = _model(6, 2, [5, 4, 3, 2, 1, 0])
    a = m.add_seq()
    m.append(a, 3)                                   # 5, 4
    b = m.fork(a)
    m.free_seq(a)
    assert m.num_free() == 4                         # shared blocks survive
    m.free_seq(b)
    assert list(m.free) == [3, 2, 1, 0, 5, 4]


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(11)
    nb, bs = 64, 8
    m = _model(nb, bs, list(rng.permutation(nb)))
    live = []
    for step in range(3000):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                s = m.add_seq()
                m.append(s, int(rng.integers(0, 40)))
                live.append(s)
            elif op == 1:
                live.append(m.fork(live[rng.integers(len(live))]))
            elif op == 2:
                m.append(live[rng.integers(len(live))], int(rng.integers(1, 20)))
            else:
                m.free_seq(live.pop(rng.integers(len(live))))
        except OutOfBlocks:
            pass
        held = [b for s in live for b in m.block_table(s)]
        assert sum(m.ref) == len(held)
        assert m.num_free() + len(set(held)) == nb
        assert not set(held) & set(m.free)
        for s in live:
            assert len(m.block_table(s)) == -(-m.lens[s] // bs)
    for s in live:
        m.free_seq(s)
    assert m.num_free() == nb and sum(m.ref) == 0


def test_mean_internal_fragmentation_is_half_a_block():
    """[k4i] memory utilization: the last block is on average half full."""
    rng = np.random.default_rng(2)
    bs = 16
    lens = rng.integers(1, 1000, 6000)
    m = _model(int(sum(-(-L // bs) for L in lens)), bs)
    waste = []
    for L in lens:
        s = m.add_seq()
        m.append(s, int(L))
        waste.append(len(m.block_table(s)) * bs - L)
    assert abs(np.mean(waste) - (bs - 1) / 2) < 0.3


def test_shared_prefix_workload_refcounts():
    """100 sequences over one 2000-token prefix at block_size 256: the 7 full
    prefix blocks end with refcount 100; the partly filled 8th is copied by 99
    sequences and written in place by the last one."""
    w = workloads.make("5c")
    st = build_state(w)
    m = st.model
    full = st.block_tables[0, :7]
    assert all(m.ref[b] == 100 for b in full)
    assert len(st.copies) == 99
    for s in range(w.S):
        assert np.array_equal(st.block_tables[s, :7], full)
    assert len({int(st.block_tables[s, 7]) for s in range(w.S)}) == 100


# ------------------------------------------------------------ prefix cache
def _cache_model(nb=64, bs=4):
    return BlockManagerModel(nb, bs, list(range(nb)))


def test_prefix_cache_reuses_a_shared_system_prompt():
    """[k4i] #prefix-caching: a 4096-token system prompt at block_size 16 is
    256 blocks, all reusable by a second request with the same prompt
    (golden/pages_needed.json); each shared block's count is then 2."""
    case = [c for c in golden("pages_needed.json")["cases"] if c["tokens"] == 4096][0]
    m = BlockManagerModel(600, case["block_size"], list(range(600)))
    prompt = list(range(1000, 1000 + case["tokens"]))
    a, hit_a = m.add_seq_cached(prompt)
    b, hit_b = m.add_seq_cached(prompt)
    assert hit_a == 0 and hit_b == case["tokens"]
    assert m.block_table(a) == m.block_table(b) and len(m.block_table(b)) == case["blocks"]
    assert all(m.ref[x] == 2 for x in m.block_table(a))
    assert m.num_cached() == case["blocks"] and m.num_free() == 600 - case["blocks"]


def test_prefix_cache_stops_at_the_first_miss_and_skips_partial_blocks():
    m = _cache_model()
    p = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10]          # 2 full blocks + 2 tokens
    a, _ = m.add_seq_cached(p)
    assert m.num_cached() == 2                    # the partial block is not cached
    q = [1, 2, 3, 4, 0, 6, 7, 8, 9, 10]          # second block differs
    b, hit = m.add_seq_cached(q)
    assert hit == 4                               # only the first block is reused
    assert m.block_table(b)[0] == m.block_table(a)[0]
    assert m.block_table(b)[1] != m.block_table(a)[1]
    # a later block with equal tokens but a different parent chain is new too
    r = [9, 9, 9, 9, 5, 6, 7, 8]
    _, hit = m.add_seq_cached(r)
    assert hit == 0


def test_prefix_cache_extra_key_separates_caches():
    m = _cache_model()
    p = [1, 2, 3, 4, 5, 6, 7, 8]
    m.add_seq_cached(p, extra=1)
    _, hit = m.add_seq_cached(p, extra=2)
    assert hit == 0
    _, hit = m.add_seq_cached(p, extra=1)
    assert hit == 8


def test_freed_cached_blocks_are_revived_then_evicted_least_recently_freed_first():
    m = BlockManagerModel(6, 2, list(range(6)))
    a, _ = m.add_seq_cached([1, 1, 2, 2])        # blocks 0, 1
    b, _ = m.add_seq_cached([3, 3, 4, 4])        # blocks 2, 3
    m.free_seq(a)                                 # 0, 1 back (still cached)
    m.free_seq(b)                                 # then 2, 3
    assert list(m.free) == [4, 5, 0, 1, 2, 3] and m.num_cached() == 4
    c, hit = m.add_seq_cached([1, 1, 2, 2])      # revived from the middle of the queue
    assert hit == 4 and m.block_table(c) == [0, 1] and list(m.free) == [4, 5, 2, 3]
    d, _ = m.add_seq_cached([7, 7, 8, 8, 9, 9])  # takes 4, 5, then 2: 2's entry goes
    assert m.block_table(d) == [4, 5, 2]
    assert m.num_cached() == 4 - 1 + 3  # 2 lost its entry; 4, 5, 2 hold the new full blocks
    e, hit = m.add_seq_cached([3, 3])            # its block was evicted: a miss, which
    assert hit == 0 and m.block_table(e) == [3]   # takes 3 (the last free) and drops (3,3)->(4,4)
    assert m.num_free() == 0


def test_prefix_cache_out_of_blocks_is_atomic():
    m = BlockManagerModel(4, 2, list(range(4)))
    m.add_seq_cached([1, 1, 2, 2])
    before = (list(m.free), dict(m.cache), list(m.ref))
    try:
        m.add_seq_cached([5, 5, 6, 6, 7])         # needs 3 blocks, 2 free
        raise AssertionError("expected OutOfBlocks")
    except OutOfBlocks:
        pass
    assert (list(m.free), dict(m.cache), list(m.ref)) == before
