"""Pins for the oracle's multi-query paged attention (ai-infra-handbooks "Paged KV cache",
section "Paged attention").

The oracle is checked against things other than itself:
  * the page's own check -- three requests (a decode of 1 token over 37, a full prefill
    of 5, the last 8 tokens of a 20-token chunked prefill), heads 8/2, d 64, block 4,
    with the block tables the page prints -- against torch's fp64 scaled dot-product
    attention on contiguous K/V with the page's causal mask;
  * the one-token case, which must equal the (separately pinned) decode oracle;
  * a full prefill, whose first row can only see token 0 (so it returns v_0) and whose
    last row is the decode of the whole sequence;
  * invariance under where the blocks sit in the pool.
"""
import json
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def _pools(rng, tables, seq_lens, nb, bs, hkv, d):
    """Random f32 pools holding each sequence's tokens at its table's slots; the rest NaN."""
    kc = np.full((nb, bs, hkv, d), np.nan, dtype=np.float32)
    vc = np.full_like(kc, np.nan)
    ks, vs = [], []
    for t, s in zip(tables, seq_lens):
        k = rng.standard_normal((s, hkv, d)).astype(np.float32)
        v = rng.standard_normal((s, hkv, d)).astype(np.float32)
        slots = [t[p // bs] * bs + p % bs for p in range(s)]
        oracle.write_kv(kc, vc, k, v, slots, "f32", "f32")
        ks.append(k)
        vs.append(v)
    return kc, vc, ks, vs


def _table_array(tables):
    width = max(len(t) for t in tables)
    return np.array([list(t) + [0] * (width - len(t)) for t in tables], dtype=np.int32)


def test_printed_check_equals_contiguous_sdpa():
    import torch
    import torch.nn.functional as F
    g = json.load(open(os.path.join(GOLDEN, "p2_round_robin_tables.json")))
    hq, hkv, d, bs = g["num_heads"], g["num_kv_heads"], g["head_dim"], g["block_size"]
    seq_lens, qlens, tables = g["seq_lens"], g["query_lens"], g["tables"]
    rng = np.random.default_rng(0)
    kc, vc, ks, vs = _pools(rng, tables, seq_lens, g["num_blocks"], bs, hkv, d)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), hq, d)).astype(np.float32)
    scale = d ** -0.5
    out = oracle.paged_attention(q, kc, vc, _table_array(tables), np.array(seq_lens), qsl, scale, "f32", "f32")
    rep = hq // hkv
    for i, (s, n) in enumerate(zip(seq_lens, qlens)):
        qi = torch.from_numpy(q[qsl[i]:qsl[i + 1]]).double().transpose(0, 1)
        k = torch.from_numpy(ks[i]).double().repeat_interleave(rep, 1).transpose(0, 1)
        v = torch.from_numpy(vs[i]).double().repeat_interleave(rep, 1).transpose(0, 1)
        mask = torch.ones(n, s, dtype=torch.bool).tril(diagonal=s - n)
        ref = F.scaled_dot_product_attention(qi, k, v, attn_mask=mask, scale=float(np.float32(scale)))
        assert np.abs(out[qsl[i]:qsl[i + 1]] - ref.transpose(0, 1).numpy()).max() <= 1e-12


def test_one_new_token_is_decode():
    rng = np.random.default_rng(1)
    bs, hkv, d, hq = 16, 2, 64, 8
    seq_lens = [1, 17, 90, 33]
    nb = 20
    perm = rng.permutation(nb)
    tables, k = [], 0
    for s in seq_lens:
        m = -(-s // bs)
        tables.append(list(perm[k:k + m]))
        k += m
    kc, vc, _, _ = _pools(rng, tables, seq_lens, nb, bs, hkv, d)
    q = rng.standard_normal((len(seq_lens), hq, d)).astype(np.float32)
    bt = _table_array(tables)
    mq = oracle.paged_attention(q, kc, vc, bt, np.array(seq_lens), np.arange(5, dtype=np.int32), 0.125, "f32", "f32")
    dec = oracle.decode(q, kc, vc, bt, np.array(seq_lens), 0.125, "f32", "f32")
    assert np.abs(mq - dec).max() <= 1e-13


def test_full_prefill_first_and_last_rows():
    rng = np.random.default_rng(2)
    bs, hkv, d, hq, s = 4, 1, 64, 2, 23
    tables = [list(rng.permutation(8)[:6])]
    kc, vc, ks, vs = _pools(rng, tables, [s], 8, bs, hkv, d)
    q = rng.standard_normal((s, hq, d)).astype(np.float32)
    bt = _table_array(tables)
    out = oracle.paged_attention(q, kc, vc, bt, np.array([s]), np.array([0, s], dtype=np.int32), 0.3, "f32", "f32")
    assert np.array_equal(out[0], np.repeat(vs[0][0, 0].astype(np.float64)[None], hq, 0))   # only token 0 visible
    dec = oracle.decode(q[-1:], kc, vc, bt, np.array([s]), 0.3, "f32", "f32")
    assert np.abs(out[-1] - dec[0]).max() <= 1e-13


def test_invariant_under_block_placement():
    rng = np.random.default_rng(3)
    bs, hkv, d, hq = 4, 2, 64, 4
    seq_lens, qlens = [13, 30], [5, 30]
    vals = [(rng.standard_normal((s, hkv, d)).astype(np.float32),
             rng.standard_normal((s, hkv, d)).astype(np.float32)) for s in seq_lens]
    q = rng.standard_normal((sum(qlens), hq, d)).astype(np.float32)
    qsl = np.array([0, 5, 35], dtype=np.int32)
    outs = []
    for perm_seed in (0, 1):
        perm = np.random.default_rng(perm_seed).permutation(16)
        tables, k = [], 0
        for s in seq_lens:
            m = -(-s // bs)
            tables.append(list(perm[k:k + m]))
            k += m
        kc = np.full((16, bs, hkv, d), np.nan, dtype=np.float32)
        vc = np.full_like(kc, np.nan)
        for t, s, (kk, vv) in zip(tables, seq_lens, vals):
            oracle.write_kv(kc, vc, kk, vv, [t[p // bs] * bs + p % bs for p in range(s)], "f32", "f32")
        outs.append(oracle.paged_attention(q, kc, vc, _table_array(tables), np.array(seq_lens), qsl, 0.2,
                                           "f32", "f32"))
    assert np.array_equal(outs[0], outs[1])
