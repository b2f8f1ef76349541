"""Copy-on-write: the harness allocator's decisions and the oracle's block copy.

The oracle's ``copy_blocks`` is pinned by what copy-on-write must guarantee
(LLM stack book, "Copy-on-write for shared prefixes"; ai-infra-handbooks "Paged
KV cache", exercise 2): after forking, copying the contested block and
writing, every sequence attends over exactly what a private, never-shared copy
of its tokens would hold -- so decoding the copy-on-write state must equal
decoding private pools built from scratch, bit for bit (the oracle reads the
same values in the same logical order).
"""
import numpy as np
import pytest

import oracle
from workloads import BlockManager, f32_to_bf16_bits


def test_walkthrough_allocation_decisions():
    """The events of the mohdvasim.com walkthrough ("Execution Walkthrough Simulation"): 10
    blocks of 16; a 24-token request, a second request sharing its prefix, the first
    appending at 32 tokens (a fresh block), the second appending at 24 (inside the shared
    block, so a copy).  Checked: this allocator's decisions and reference counts (the
    page prints no block ids; ours come from its first-free order)."""
    m = BlockManager(10, 16)
    m.allocate("u1", 24)
    assert m.block_tables["u1"] == [0, 1]
    m.fork("u1", "u2")
    assert [m.pool.ref_cnt[b] for b in (0, 1)] == [2, 2]
    m.append_token("u1", 32)                       # position 32: logical block 2, new
    assert m.block_tables["u1"] == [0, 1, 2]
    assert m.cow_append("u1", 32 // 16) == (2, 2)  # private: write in place
    m.append_token("u2", 24)                       # position 24: logical block 1, shared
    src, dst = m.cow_append("u2", 24 // 16)
    assert (src, dst) == (1, 3)
    assert m.block_tables["u2"] == [0, 3] and m.block_tables["u1"] == [0, 1, 2]
    assert [m.pool.ref_cnt[b] for b in (0, 1, 2, 3)] == [2, 1, 1, 1]
    m.free_seq("u1")
    m.free_seq("u2")
    assert m.num_free_blocks() == 10


def _rows(rng, n, hkv, d, fmt):
    x = rng.standard_normal((n, hkv, d)).astype(np.float32)
    return (x, "f32") if fmt == "f32" else (f32_to_bf16_bits(x), "bf16")


def cow_scenario(fmt="bf16", prefix=40, children=3, bs=16, hkv=2, d=64, seed=3, num_blocks=32):
    """Parent with ``prefix`` tokens forked ``children`` times; every sequence appends its own token.

    Returns (state, private, q, fmt, pre): the copy-on-write pools and tables after copy
    and write, the same sequences built in private blocks from scratch (each
    (kc, vc, tables, ctx, copies) with copies = the (src, dst) pairs copied), the query,
    the storage format, and pre = (kc, vc, new_k, new_v, slots, in_fmt): the pools just
    before the copy and the appended rows with their slots.
    """
    rng = np.random.default_rng(seed)
    store = {"f32": np.float32, "bf16": np.uint16}[fmt]
    poison = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0)}[fmt]
    pk, _ = _rows(rng, prefix, hkv, d, fmt)
    pv, kin = _rows(rng, prefix, hkv, d, fmt)
    seqs = ["p"] + [f"c{i}" for i in range(children)]
    newk = {s: _rows(rng, 1, hkv, d, fmt)[0] for s in seqs}
    newv = {s: _rows(rng, 1, hkv, d, fmt)[0] for s in seqs}

    # copy-on-write state
    kc = np.full((num_blocks, bs, hkv, d), poison, dtype=store)
    vc = np.full_like(kc, poison)
    m = BlockManager(num_blocks, bs)
    m.allocate("p", prefix)
    oracle.write_kv(kc, vc, pk, pv, [m.slot_index("p", t) for t in range(prefix)], fmt, kin)
    for s in seqs[1:]:
        m.fork("p", s)
    pre_k, pre_v = kc.copy(), vc.copy()
    copies = []
    for s in seqs:                                  # each appends at position `prefix`
        m.append_token(s, prefix)
        src, dst = m.cow_append(s, prefix // bs)
        if src != dst:
            copies.append((src, dst))
    src = [c[0] for c in copies]
    dst = [c[1] for c in copies]
    oracle.copy_blocks(kc, vc, src, dst)
    new_slots = [m.slot_index(s, prefix) for s in seqs]
    for s, slot in zip(seqs, new_slots):
        oracle.write_kv(kc, vc, newk[s], newv[s], [slot], fmt, kin)
    nbps = -(-(prefix + 1) // bs)
    tables = np.array([m.block_tables[s][:nbps] for s in seqs], dtype=np.int32)
    ctx = np.full(len(seqs), prefix + 1, dtype=np.int32)
    state = (kc, vc, tables, ctx, copies)

    # private pools: each sequence writes all its tokens into blocks of its own
    kp = np.full((len(seqs) * nbps, bs, hkv, d), poison, dtype=store)
    vp = np.full_like(kp, poison)
    ptab = np.arange(len(seqs) * nbps, dtype=np.int32).reshape(len(seqs), nbps)
    for i, s in enumerate(seqs):
        slots = [int(ptab[i, t // bs]) * bs + t % bs for t in range(prefix + 1)]
        oracle.write_kv(kp, vp, np.concatenate([pk, newk[s]]), np.concatenate([pv, newv[s]]), slots, fmt, kin)
    private = (kp, vp, ptab, ctx, [])
    q = _rows(rng, len(seqs), 2 * hkv, d, fmt)[0]                # two query heads per KV head
    pre = (pre_k, pre_v, np.concatenate([newk[s] for s in seqs]), np.concatenate([newv[s] for s in seqs]),
           np.array(new_slots, dtype=np.int32), kin)
    return state, private, q, fmt, pre


@pytest.mark.parametrize("prefix,bs", [(40, 16), (32, 16), (7, 4), (100, 64)])
def test_copy_on_write_equals_private_blocks(prefix, bs):
    state, private, q, fmt, _ = cow_scenario(prefix=prefix, bs=bs)
    kc, vc, tables, ctx, copies = state
    kp, vp, ptab, _, _ = private
    scale = 0.125
    a = oracle.decode(q, kc, vc, tables, ctx, scale, fmt, fmt)
    b = oracle.decode(q, kp, vp, ptab, ctx, scale, fmt, fmt)
    assert np.array_equal(a, b)
    # a block boundary before the appended token needs no copy; otherwise every
    # sharer but the last one copies, and the last writes in place
    assert len(copies) == (0 if prefix % bs == 0 else 3)
    # every sequence ends with a private last block
    assert len(set(tables[:, -1].tolist())) == len(tables)


def test_copy_blocks_reads_the_state_before_the_call():
    """A copy whose source another pair of the same call overwrites still copies the old block."""
    kc = np.arange(6 * 2 * 1 * 4, dtype=np.float32).reshape(6, 2, 1, 4)
    vc = -kc
    before = kc.copy()
    oracle.copy_blocks(kc, vc, [0, 1, -1, 2], [1, 3, 4, 9])     # (-1 -> 4) and (2 -> 9) are skipped
    assert np.array_equal(kc[1], before[0]) and np.array_equal(kc[3], before[1])
    assert np.array_equal(vc[3], -before[1])
    for blk in (0, 2, 4, 5):
        assert np.array_equal(kc[blk], before[blk])
