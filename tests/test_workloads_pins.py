"""Caller-side bookkeeping and the workload generator, pinned to the pages' printed traces."""
import json
import math
import os

import numpy as np
import pytest

from conftest import GOLDEN
from workloads import (BlockManager, BlockPool, build_step_tensors, make_config, p2_length_pairs,
                       slot_mapping_for)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_block_pool_doctest():
    g = _golden("p2_block_pool_doctest.json")
    pool = BlockPool(g["num_blocks"])
    table = pool.allocate(3)
    assert table == g["first_allocation"]
    assert pool.num_free() == g["free_after_first"]
    other = pool.allocate(g["second_allocation_size"])
    assert other is not None
    pool.free(table)
    assert pool.allocate(4) == g["allocation_after_free"]
    got = slot_mapping_for(g["slot_mapping_block_table"], range(g["slot_mapping_positions"]),
                           g["slot_mapping_block_size"])
    assert got == g["slot_mapping"]


def test_pool_shortfall_returns_none_and_manager_raises():
    pool = BlockPool(2)
    assert pool.allocate(3) is None and pool.num_free() == 2
    mgr = BlockManager(2, 16)
    with pytest.raises(MemoryError):
        mgr.allocate("s", 33)


def test_round_robin_tables():
    g = _golden("p2_round_robin_tables.json")
    pool = BlockPool(g["num_blocks"])
    bs = g["block_size"]
    tables = [[] for _ in g["seq_lens"]]
    while any(len(t) * bs < s for t, s in zip(tables, g["seq_lens"])):
        for t, s in zip(tables, g["seq_lens"]):
            if len(t) * bs < s:
                t += pool.allocate(1)
    assert tables == g["tables"]


def test_int8ai_slot_trace():
    g = _golden("p3_slot_trace.json")
    bs = g["block_size"]
    # a pool whose next free block is the one the trace allocates
    pool = BlockPool(16)
    taken = pool.allocate(16)
    pool.free([g["next_free_block"]])
    mgr = BlockManager(16, bs, pool=pool)
    mgr.block_tables["r"] = list(g["initial_table"])
    assert len(taken) == 16
    for step in g["trace"]:
        t = step["token"]
        before = len(mgr.block_tables["r"])
        mgr.append_token("r", t)
        assert (len(mgr.block_tables["r"]) > before) == step["new_block"]
        slot = mgr.slot_index("r", t)
        assert divmod(slot, bs) == (step["physical_block"], step["slot_in_block"])
        assert t // bs == step["logical_block"]
    assert mgr.block_tables["r"] == g["final_table"]


def test_block_boundary_grow_before_write():
    g = _golden("p1_allocator_cases.json")["boundary"]
    mgr = BlockManager(g["num_blocks"], g["block_size"])
    mgr.allocate("s", g["prompt_len"])
    assert len(mgr.block_tables["s"]) == g["blocks_after_prefill"]
    for cur in g["decode_positions"]:
        mgr.append_token("s", cur)
        slot = mgr.slot_index("s", cur)
        assert slot % g["block_size"] == cur % g["block_size"]
    assert len(mgr.block_tables["s"]) == g["blocks_after_decode"]


def test_exercise5_can_allocate():
    g = _golden("p1_allocator_cases.json")["exercise5"]
    mgr = BlockManager(g["num_blocks"], g["block_size"])
    assert mgr.num_free_blocks() == g["free_blocks"]
    assert mgr.blocks_for(200) == g["blocks_needed_200"]
    assert mgr.can_allocate(200) == g["can_allocate_200"]
    assert mgr.can_allocate(100) == g["can_allocate_100"]


def test_fork_and_copy_on_write():
    mgr = BlockManager(8, 4)
    mgr.allocate("a", 6)                      # 2 blocks
    mgr.fork("a", "b")
    shared = mgr.block_tables["a"][1]
    assert mgr.pool.ref_cnt[shared] == 2
    src, dst = mgr.cow_append("b", 1)
    assert src == shared and dst != src
    assert mgr.block_tables["b"][1] == dst and mgr.block_tables["a"][1] == shared
    assert mgr.pool.ref_cnt[shared] == 1 and mgr.pool.ref_cnt[dst] == 1
    assert mgr.cow_append("a", 1) == (shared, shared)
    mgr.free_seq("a"); mgr.free_seq("b")
    assert mgr.num_free_blocks() == 8


def test_build_step_tensors():
    mgr = BlockManager(8, 4)
    mgr.allocate(0, 4)
    mgr.allocate(1, 2)
    cur = [4, 2]
    for s, n in zip([0, 1], cur):
        mgr.append_token(s, n)
    bt, slots, ctx = build_step_tensors([mgr.block_tables[0], mgr.block_tables[1]], cur, 4)
    assert bt.dtype == np.int32 and bt.shape == (2, 2)
    assert bt[1, 1] == 0                                   # right padding
    assert list(ctx) == [5, 3]
    assert slots[0] == mgr.block_tables[0][1] * 4 + 0
    assert slots[1] == mgr.block_tables[1][0] * 4 + 2


def test_p2_utilization_generator():
    g = _golden("p2_utilization.json")
    reqs = p2_length_pairs(g["num_requests"], g["seed"])
    used = sum(p + o for p, o in reqs)
    assert round(100 * used / (len(reqs) * g["max_len"]), 1) == g["reserve_max_percent"]
    for bs, pct in g["paged_percent"].items():
        bs = int(bs)
        alloc = sum(math.ceil((p + o) / bs) * bs for p, o in reqs)
        assert round(100 * used / alloc, 1) == pct


@pytest.mark.parametrize("name", ["tiny_f32", "llama3_8b_b64", "llama2_7b_mha"])
def test_config_tables_are_a_partition_of_the_pool(name):
    w = make_config(name)
    seen = []
    for b in range(w.num_seqs):
        n = -(-int(w.context_lens[b]) // w.block_size)
        seen.extend(w.block_tables[b, :n].tolist())
    assert len(seen) == len(set(seen))                    # no block used twice
    assert all(0 <= x < w.num_blocks for x in seen)
    assert w.num_blocks == (64 if name == "tiny_f32" else math.ceil(1.1 * len(seen)))


def test_config_sizes():
    c1 = make_config("tiny_f32")
    assert c1.context_lens.tolist() == [35, 146, 196, 17]
    c2 = make_config("llama3_8b_b64")
    assert c2.total_tokens == 121416 and c2.context_lens.min() == 732 and c2.context_lens.max() == 3360
    assert c2.num_blocks == 8382 and c2.max_blocks_per_seq == 210
    assert c2.scale == float(np.float32(1 / math.sqrt(128)))
    for bs, nb in [(1, 70002), (16, 4392), (64, 1110), (256, 290)]:
        w = make_config("llama2_7b_mha", bs)
        assert w.total_tokens == 63638 and w.num_blocks == nb


def test_shared_prefix_config():
    w = make_config("llama3_8b_fp8_prefix")
    assert w.num_blocks == 34074
    assert (w.block_tables[:8, :256] == w.block_tables[0, :256]).all()
    assert (w.ref_count[w.block_tables[0, :256]] == 8).all()
    used = np.concatenate([w.block_tables[b] for b in range(w.num_seqs)])
    assert len(np.unique(used)) == 30976
    # this step's write position lands in a privately owned block: no copy-on-write needed
    for b, s in enumerate(w.append_slots()):
        assert w.ref_count[s // w.block_size] == 1
    # positions owned by sequence 1 start after the shared prefix
    assert w.owned_positions(1)[0] == 4096 and w.owned_positions(0)[0] == 0


def test_block_size_sweep_shares_token_values():
    a = make_config("llama2_7b_mha", 1)
    b = make_config("llama2_7b_mha", 256)
    assert np.array_equal(a.seq_token_values("k", 3)[:5], b.seq_token_values("k", 3)[:5])
    assert np.array_equal(a.q_values(), b.q_values())
