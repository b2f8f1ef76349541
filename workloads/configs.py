"""The five decode workloads and their seeded construction.

Shapes: a Llama-3-8B attention layer (32 query heads, 8 KV heads, head dim 128),
a Llama-2-7B-style MHA layer (32/32, 128) and a tiny GQA case.  Lengths come from
the ai-infra-handbooks "Paged KV cache" generator (section "Why paging");
physical blocks are a seeded random permutation of the pool dealt to the
sequences in batch order, so consecutive logical blocks land anywhere in the
pool (the LLM stack book, section "The OS-Paging Analogy").  A pool holds
ceil(1.1 * blocks needed) blocks; blocks no sequence uses stay unused and the
tests poison them.

Nothing here computes attention or writes a pool: it returns integer tables,
lengths, the slots each token is written to, and the random values.
"""
from __future__ import annotations

import math
import random
from dataclasses import dataclass, field

import numpy as np

from .lengths import p2_context_lens

# streams of the seeded value generator
_Q, _K, _V = 0, 1, 2


def deal_tables(ctx, block_size: int, perm: np.ndarray):
    """Deal the permuted physical block ids to sequences in batch order."""
    need = [-(-int(c) // block_size) for c in ctx]
    max_blocks = max(max(need), 1)
    bt = np.zeros((len(ctx), max_blocks), dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[k:k + n]
        k += n
    return bt, k


def shared_prefix_tables(ctx, block_size: int, perm: np.ndarray, sharers: int, prefix_blocks: int):
    """Tables where sequences 0..sharers-1 share their first ``prefix_blocks`` physical blocks.

    The shared blocks are the first ``prefix_blocks`` ids of ``perm`` (refcount =
    ``sharers``); every other logical block gets a private id, dealt in batch order.
    """
    need = [-(-int(c) // block_size) for c in ctx]
    bt = np.zeros((len(ctx), max(need)), dtype=np.int32)
    shared = perm[:prefix_blocks]
    k = prefix_blocks
    for b, n in enumerate(need):
        if b < sharers:
            bt[b, :prefix_blocks] = shared
            rest = n - prefix_blocks
            bt[b, prefix_blocks:n] = perm[k:k + rest]
            k += rest
        else:
            bt[b, :n] = perm[k:k + n]
            k += n
    return bt, k


@dataclass
class DecodeWorkload:
    """One decode step's integer inputs plus seeded value streams.

    Attributes follow the pages' notation: ``context_lens`` counts the tokens
    valid after this step's write, block tables are right-padded with 0.
    """
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str            # "f32" | "bf16" | "e4m3"
    q_dtype: str             # "f32" | "bf16"
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, max_blocks]
    num_blocks: int
    seed: int
    shared_prefix_tokens: int = 0   # sequences 0..sharers-1 share this many leading tokens
    sharers: int = 0
    ref_count: np.ndarray = field(default=None)
    query_lens: np.ndarray = field(default=None)  # multi-query workloads: new tokens per sequence

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d_h) as the float32 value the kernels receive."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.sum())

    def slots(self, b: int, positions: np.ndarray) -> np.ndarray:
        """Slot of each position of sequence b: table[p // B] * B + p % B (int64)."""
        positions = np.asarray(positions, dtype=np.int64)
        bs = self.block_size
        return self.block_tables[b, positions // bs].astype(np.int64) * bs + positions % bs

    def owned_positions(self, b: int) -> np.ndarray:
        """Positions whose slots sequence b writes (a shared prefix belongs to sequence 0)."""
        start = self.shared_prefix_tokens if (0 < b < self.sharers) else 0
        return np.arange(start, int(self.context_lens[b]), dtype=np.int64)

    # -- values ------------------------------------------------------------
    def q_values(self) -> np.ndarray:
        rng = np.random.default_rng([self.seed, _Q])
        return rng.standard_normal((self.num_seqs, self.num_q_heads, self.head_dim), dtype=np.float32)

    def seq_token_values(self, which: str, b: int) -> np.ndarray:
        """float32 [len(owned_positions(b)), H_kv, d] for K ('k') or V ('v') of sequence b."""
        stream = {"k": _K, "v": _V}[which]
        rng = np.random.default_rng([self.seed, stream, b])
        n = len(self.owned_positions(b))
        return rng.standard_normal((n, self.num_kv_heads, self.head_dim), dtype=np.float32)

    # -- multi-query (several new tokens per sequence) ------------------------------
    def query_start_loc(self) -> np.ndarray:
        """int32 [B + 1]: sequence b's new tokens are rows qsl[b] .. qsl[b+1]-1."""
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    def mq_q_values(self) -> np.ndarray:
        """float32 [sum(query_lens), H_q, d]: the new tokens' queries."""
        rng = np.random.default_rng([self.seed, _Q])
        n = int(np.sum(self.query_lens))
        return rng.standard_normal((n, self.num_q_heads, self.head_dim), dtype=np.float32)

    def append_slots(self) -> np.ndarray:
        """slot_mapping of this step's write: position ctx-1 of every sequence (int32)."""
        return np.array([self.slots(b, [int(c) - 1])[0] for b, c in enumerate(self.context_lens)],
                        dtype=np.int32)

    def with_dtypes(self, kv_dtype: str, q_dtype: str, name: str | None = None) -> "DecodeWorkload":
        """Same tables and value streams, other storage dtypes (the f32 shadows)."""
        w = DecodeWorkload(**{**self.__dict__})
        w.kv_dtype, w.q_dtype = kv_dtype, q_dtype
        w.name = name or f"{self.name}-{kv_dtype}"
        return w

    def kv_bytes_read(self, kv_elem_bytes: int) -> int:
        """Bytes of K and V one decode pass must read: sum(ctx) * H_kv * d * 2 * b."""
        return self.total_tokens * self.num_kv_heads * self.head_dim * 2 * kv_elem_bytes


def _refcounts(bt: np.ndarray, ctx, block_size: int, num_blocks: int) -> np.ndarray:
    rc = np.zeros(num_blocks, dtype=np.int32)
    for b, c in enumerate(ctx):
        n = -(-int(c) // block_size)
        np.add.at(rc, bt[b, :n], 1)
    return rc


def _pool_size(blocks_needed: int) -> int:
    return math.ceil(1.1 * blocks_needed)


def _paged(name, B, hq, hkv, d, bs, kv, q, ctx, seed_perm, seed_vals):
    ctx = np.asarray(ctx, dtype=np.int32)
    need = int(sum(-(-int(c) // bs) for c in ctx))
    nb = _pool_size(need)
    perm = np.random.default_rng(seed_perm).permutation(nb).astype(np.int32)
    bt, used = deal_tables(ctx, bs, perm)
    assert used == need
    return DecodeWorkload(name, B, hq, hkv, d, bs, kv, q, ctx, bt, nb, seed_vals,
                          ref_count=_refcounts(bt, ctx, bs, nb))


CONFIG_NAMES = ("tiny_f32", "llama3_8b_b64", "llama3_8b_long", "llama2_7b_mha", "llama3_8b_fp8_prefix")
MQ_CONFIG_NAMES = ("llama3_8b_chunk512",)


def make_mq_config(name: str) -> DecodeWorkload:
    """Multi-query workloads: several new tokens per sequence, causal over the paged context.

    llama3_8b_chunk512: 32 sequences with the lengths of the utilization experiment's
    first 32 (prompt, output) pairs, each computing its last min(512, len) tokens -- the
    final chunk of a chunked prefill -- on a Llama-3-8B layer (32/8 heads, d 128, bf16,
    block 16, pool +10 %).
    """
    if name == "llama3_8b_chunk512":
        ctx = p2_context_lens(32)
        w = _paged(name, 32, 32, 8, 128, 16, "bf16", "bf16", ctx, 16, 106)
        w.query_lens = np.minimum(512, w.context_lens).astype(np.int32)
        return w
    raise ValueError(f"unknown multi-query workload {name!r}")


def make_config(name: str, block_size: int | None = None) -> DecodeWorkload:
    """Build one of the five decode workloads (seeded, deterministic).

    * ``tiny_f32``: 4 sequences, 4 query / 2 KV heads, d 64, block 16, f32;
      lengths ``random.Random(1).randint(1, 200)`` x4 (post-write); pool of 64 blocks.
    * ``llama3_8b_b64``: Llama-3-8B layer, bf16, batch 64, lengths = first 64
      (prompt, output) pairs of the seed-0 stream; pool 1.1x the blocks needed.
    * ``llama3_8b_long``: same layer, batch 64, every context 8192.
    * ``llama2_7b_mha``: 32/32 heads, bf16, batch 32, first 32 pairs; ``block_size``
      in {1, 16, 64, 256} with identical token values for every block size.
    * ``llama3_8b_fp8_prefix``: e4m3 K/V pools, bf16 q, batch 16, context 32768;
      sequences 0..7 share their first 4096 tokens (256 blocks of 16).
    """
    if name == "tiny_f32":
        rng = random.Random(1)
        ctx = [rng.randint(1, 200) for _ in range(4)]
        B, bs, nb = 4, 16, 64
        ctx = np.asarray(ctx, dtype=np.int32)
        perm = np.random.default_rng(11).permutation(nb).astype(np.int32)
        bt, _ = deal_tables(ctx, bs, perm)
        return DecodeWorkload(name, B, 4, 2, 64, bs, "f32", "f32", ctx, bt, nb, 101,
                              ref_count=_refcounts(bt, ctx, bs, nb))
    if name == "llama3_8b_b64":
        return _paged(name, 64, 32, 8, 128, 16, "bf16", "bf16", p2_context_lens(64), 12, 102)
    if name == "llama3_8b_long":
        return _paged(name, 64, 32, 8, 128, 16, "bf16", "bf16", [8192] * 64, 13, 103)
    if name == "llama2_7b_mha":
        bs = 16 if block_size is None else int(block_size)
        w = _paged(f"{name}_bs{bs}", 32, 32, 32, 128, bs, "bf16", "bf16", p2_context_lens(32), 14, 104)
        return w
    if name == "llama3_8b_fp8_prefix":
        B, bs, ctxlen, sharers, prefix = 16, 16, 32768, 8, 4096
        ctx = np.full(B, ctxlen, dtype=np.int32)
        pb = prefix // bs
        per_seq = ctxlen // bs
        unique = pb + sharers * (per_seq - pb) + (B - sharers) * per_seq
        nb = _pool_size(unique)
        perm = np.random.default_rng(15).permutation(nb).astype(np.int32)
        bt, used = shared_prefix_tables(ctx, bs, perm, sharers, pb)
        assert used == unique
        return DecodeWorkload(name, B, 32, 8, 128, bs, "e4m3", "bf16", ctx, bt, nb, 105,
                              shared_prefix_tokens=prefix, sharers=sharers,
                              ref_count=_refcounts(bt, ctx, bs, nb))
    raise KeyError(name)
