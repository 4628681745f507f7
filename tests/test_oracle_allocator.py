"""Pins for the oracle's host block pool (CPU only).

Each test drives the pool the way a page's program does and checks what the
page states (or what follows from its code where it prints nothing).  The
fixtures under tests/golden/ carry the citations.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import OracleError, Pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def status(pool):
    s = pool.stats()
    return {"total": s["n_blocks"], "free": s["n_free"], "active": s["n_active"]}


def test_p1_main_demo():
    """'PagedAttention实现' main(): two sequences, 24 and 16 tokens, then free seq 1."""
    g = golden("p1_main_demo.json")
    pool = Pool(g["num_blocks"], g["block_size"])
    s1 = pool.seq_new()
    b = [pool.seq_alloc_block(s1), pool.seq_alloc_block(s1)]
    assert b == g["seq1_blocks"]
    slots1 = [pool.seq_slot(s1, i) for i in range(g["seq1_tokens"])]
    s2 = pool.seq_new()
    assert [pool.seq_alloc_block(s2)] == g["seq2_blocks"]
    slots2 = [pool.seq_slot(s2, i) for i in range(g["seq2_tokens"])]
    assert status(pool) == g["status_after_writes"]
    assert slots1[-1] == g["seq1_last_token_slot"]
    # every write lands in the sequence's own blocks, at distinct slots
    assert len(set(slots1) | set(slots2)) == g["seq1_tokens"] + g["seq2_tokens"]
    pool.free(s1)
    assert status(pool) == g["status_after_free_seq1"]
    assert pool.alloc() == g["next_alloc_after_free"]


def test_p1_write_beyond_table_is_an_error():
    pool = Pool(8, 16)
    s = pool.seq_new()
    pool.seq_alloc_block(s)
    assert pool.seq_slot(s, 15) == 7 * 16 + 15
    with pytest.raises(OracleError):
        pool.seq_slot(s, 16)        # the page leaves this access unchecked


def test_p2_demo1_block_table_growth():
    """Lecture 7 demo 1: the vLLM Fig. 6 example (7-token prompt, block size 4)."""
    g = golden("p2_demo1_block_table.json")
    st = g["stated_on_page"]
    pool = Pool(st["pool_blocks"], st["block_size"])
    junk = [pool.alloc() for _ in range(st["junk_allocs"])]
    for i in st["junk_freed_indices"]:
        pool.decref(junk[i])
    freed = {junk[i] for i in st["junk_freed_indices"]}
    seq = pool.seq_new()
    tables = []
    for _ in range(7):                  # prefill 7 tokens
        pool.append(seq)
    tables.append(pool.table(seq).tolist())
    for _ in range(2):                  # two decode steps
        pool.append(seq)
        tables.append(pool.table(seq).tolist())
    for row, tab in zip(st["rows"], tables):
        n = pool.seq_len(seq) if row is st["rows"][-1] else None
        assert len(tab) == row["n_blocks"]
        filled, size = map(int, row["last_block_fill"].split("/"))
        assert row["tokens"] - (row["n_blocks"] - 1) * size == filled
        if n is not None:
            assert n == row["tokens"]
    # the other (simulated) sequences still hold 2 blocks
    assert pool.stats()["n_used"] - len(tables[-1]) == st["blocks_held_by_other_sequences"]
    # freed blocks are handed out first; the ids are not contiguous
    assert set(tables[-1]) <= freed
    assert any(b2 - b1 != 1 for b1, b2 in zip(tables[-1], tables[-1][1:]))
    assert tables == g["derived_lifo_from_identity"]["tables"]


def test_p2_demo1_tokens_and_fill_per_step():
    """Tokens written and last-block fill after each step, as the demo 1 table lists."""
    pool = Pool(8, 4)
    seq = pool.seq_new()
    rows = []
    for n_new in (7, 1, 1):
        for _ in range(n_new):
            pool.append(seq)
        n, nb = pool.seq_len(seq), pool.seq_num_blocks(seq)
        rows.append((nb, n, n - (nb - 1) * 4))
    assert rows == [(2, 7, 3), (2, 8, 4), (3, 9, 1)]


@pytest.mark.parametrize("block_size", [1, 4, 16, 64])
def test_p2_demo2_blocks_used_and_waste(block_size):
    """Lecture 7 demo 2: prompts 5/17/33/64, prefill + 20 decode steps, pool 260//B+8."""
    g = golden("p2_demo2_waste.json")
    st, der = g["stated_on_page"], g["derived_closed_form"]
    pool = Pool(260 // block_size + 8, block_size)
    assert pool.num_blocks == der["pool_blocks"][str(block_size)]
    seqs = [pool.seq_new() for _ in st["prompt_lengths"]]
    for s, n in zip(seqs, st["prompt_lengths"]):        # prefill (the first of 21 passes)
        for _ in range(n):
            pool.append(s)
    for _ in range(st["decode_steps"]):                 # 20 decode passes, 1 token each
        for s in seqs:
            pool.append(s)
    used = pool.stats()["n_used"]
    need = sum(pool.seq_len(s) for s in seqs)
    waste = 1 - need / (used * block_size)
    assert need == sum(st["prompt_lengths"]) + 4 * st["decode_steps"] == 199
    assert used == der["blocks_used"][str(block_size)]
    assert waste == pytest.approx(der["waste"][str(block_size)], abs=1e-15)
    stated = st["waste_percent_rounded"].get(str(block_size))
    if stated is not None:
        assert round(100 * waste) == stated
    # every sequence wastes less than one block (lecture 7, demo 1 observations)
    for s in seqs:
        assert pool.seq_num_blocks(s) * block_size - pool.seq_len(s) < block_size


@pytest.mark.parametrize("n", [2, 4, 6])
def test_p2_demo3_parallel_sampling_cow(n):
    """Lecture 7 demo 3: n samples share a 100-token prompt; the first write into
    the half-full 7th block copies it for n-1 samples, the last writes in place."""
    g = golden("p2_demo3_cow.json")
    st = g["stated_on_page"]
    bs = st["block_size"]
    pool = Pool(st["pool_blocks"], bs)
    prompt = pool.seq_new()
    for _ in range(st["prompt_tokens"]):
        pool.append(prompt)
    tab = pool.table(prompt)
    assert len(tab) == st["shared_prompt_blocks"]
    assert st["prompt_tokens"] - st["full_prompt_blocks"] * bs == st["tokens_in_last_prompt_block"]
    samples = [prompt] + [pool.fork(prompt) for _ in range(n - 1)]
    assert all(pool.ref(b) == n for b in tab)
    cows = []
    for _ in range(st["new_tokens_per_sample"]):
        for s in samples:
            slot, src, dst = pool.append(s)
            if src >= 0:
                cows.append((s, src, dst))
    assert pool.stats()["n_copies"] == n - 1 == g["derived"]["cow_copies"][str(n)]
    # the copies all came from the shared 7th block, and the last sample kept it
    assert {c[1] for c in cows} == {int(tab[-1])}
    assert [c[0] for c in cows] == samples[:n - 1]
    assert pool.table(samples[-1])[6] == tab[-1]
    assert pool.ref(int(tab[-1])) == 1
    # blocks used vs each sample holding its own copy of the prompt
    per_sample = math.ceil((st["prompt_tokens"] + st["new_tokens_per_sample"]) / bs)
    used = pool.stats()["n_used"]
    assert used == 6 + n * (per_sample - 6)
    assert used < n * per_sample


def test_fork_then_free_returns_every_block():
    pool = Pool(32, 4)
    a = pool.seq_new()
    for _ in range(10):
        pool.append(a)
    kids = [pool.fork(a) for _ in range(3)]
    for k in kids:
        for _ in range(5):
            pool.append(k)
    for s in [a] + kids:
        pool.free(s)
    st = pool.stats()
    assert st["n_free"] == 32 and st["n_used"] == 0 and st["n_active"] == 0


def test_pool_exhaustion_is_reported_not_undefined():
    """'PagedAttention实现' allocate_block reports an empty free list; its
    copy-on-write path does not check.  The oracle reports both."""
    pool = Pool(2, 4)
    s = pool.seq_new()
    for _ in range(8):
        pool.append(s)
    with pytest.raises(OracleError) as e:
        pool.append(s)
    assert e.value.code == -1
    # copy-on-write on a full pool
    pool2 = Pool(1, 4)
    p = pool2.seq_new()
    pool2.append(p)
    c = pool2.fork(p)
    with pytest.raises(OracleError) as e:
        pool2.append(c)
    assert e.value.code == -1


def test_bad_ids_are_errors():
    pool = Pool(4, 4)
    with pytest.raises(OracleError):
        pool.free(3)
    with pytest.raises(OracleError):
        pool.decref(0)            # not held
    with pytest.raises(OracleError):
        pool.ref(9)
    with pytest.raises(OracleError):
        Pool(4, 4, free_order=np.array([0, 1, 1, 2]))   # not a permutation


def test_free_order_is_a_stack():
    order = np.array([5, 2, 7, 0, 1, 3, 6, 4])
    pool = Pool(8, 4, free_order=order)
    got = [pool.alloc() for _ in range(8)]
    assert got == order[::-1].tolist()
