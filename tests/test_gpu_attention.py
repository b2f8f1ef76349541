"""pa_paged_attention (several new tokens per sequence, causal) against the oracle."""
import json
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN
from pools import POISON, STORAGE, from_dev, out_to_f64, to_dev
from workloads import f32_to_bf16_bits, make_mq_config

pytestmark = pytest.mark.gpu


class MQ:
    """Host pools (written by the oracle), tables and queries for one multi-query call."""

    def __init__(self, seq_lens, qlens, hq, hkv, d, bs, kv="bf16", seed=0, tables=None, nb=None, kgrow=0.0):
        rng = np.random.default_rng(seed)
        self.seq_lens = np.asarray(seq_lens, dtype=np.int32)
        self.qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        need = [-(-int(s) // bs) for s in seq_lens]
        if tables is None:
            nb = sum(need) + 3
            perm = rng.permutation(nb)
            tables, k = [], 0
            for m in need:
                tables.append(list(perm[k:k + m]))
                k += m
        width = max(max(need), 1)
        self.bt = np.array([list(t) + [0] * (width - len(t)) for t in tables], dtype=np.int32)
        self.kv, self.bs, self.d = kv, bs, d
        self.kc = np.full((nb, bs, hkv, d), POISON[kv], dtype=STORAGE[kv])
        self.vc = np.full_like(self.kc, POISON[kv])
        self.ks = self.vs = 1.0
        kvals = [rng.standard_normal((int(s), hkv, d)).astype(np.float32) for s in seq_lens]
        if kgrow:                                     # key norms growing with the position
            kvals = [(x * (1.0 + kgrow * np.arange(len(x), dtype=np.float32))[:, None, None]).astype(np.float32)
                     for x in kvals]
        vvals = [rng.standard_normal((int(s), hkv, d)).astype(np.float32) for s in seq_lens]
        if kv in ("e4m3", "i8"):
            qmax = 448.0 if kv == "e4m3" else 127.0
            bf = lambda x: (f32_to_bf16_bits(x).astype(np.uint32) << 16).view(np.float32)
            self.ks = float(np.float32(max(np.abs(bf(x)).max() for x in kvals) / qmax))
            self.vs = float(np.float32(max(np.abs(bf(x)).max() for x in vvals) / qmax))
        for t, s, kk, vv in zip(tables, seq_lens, kvals, vvals):
            slots = [t[p // bs] * bs + p % bs for p in range(int(s))]
            oracle.write_kv(self.kc, self.vc, f32_to_bf16_bits(kk), f32_to_bf16_bits(vv), slots, kv, "bf16",
                            self.ks, self.vs)
        self.q = f32_to_bf16_bits(rng.standard_normal((int(self.qsl[-1]), hq, d)).astype(np.float32))

    def run(self, scale, max_q=None):
        import torch
        import paged_kv_cache_112_amd as pa
        qlens = np.diff(self.qsl)
        out = pa.paged_attention(to_dev(self.q), to_dev(self.kc), to_dev(self.vc), to_dev(self.bt),
                                 to_dev(self.seq_lens), to_dev(self.qsl), scale,
                                 int(qlens.max()) if max_q is None else max_q, k_scale=self.ks, v_scale=self.vs)
        torch.cuda.synchronize()
        return out

    def oracle(self, scale, rows=None):
        return oracle.paged_attention(self.q, self.kc, self.vc, self.bt, self.seq_lens, self.qsl, scale, self.kv,
                                      "bf16", self.ks, self.vs, rows=rows)


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "i8"])
def test_printed_check(kv):
    """The page's check: decode 1 of 37, a full prefill of 5, the last 8 of 20; its block tables."""
    g = json.load(open(os.path.join(GOLDEN, "p2_round_robin_tables.json")))
    m = MQ(g["seq_lens"], g["query_lens"], g["num_heads"], g["num_kv_heads"], g["head_dim"], g["block_size"],
           kv, tables=g["tables"], nb=g["num_blocks"])
    scale = g["head_dim"] ** -0.5
    assert np.abs(out_to_f64(m.run(scale)) - m.oracle(scale)).max() <= 2e-2


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (16, 8, 64), (32, 8, 128), (32, 4, 64), (32, 2, 128)])
@pytest.mark.parametrize("bs", [1, 4, 16, 64, 1024])
def test_mixed_query_lengths(hq, hkv, d, bs):
    seq_lens = [1, 5, 40, 300, 17, 130, 64]
    qlens = [1, 5, 3, 300, 16, 17, 1]
    m = MQ(seq_lens, qlens, hq, hkv, d, bs, seed=bs + hq + d)
    scale = float(np.float32(1 / np.sqrt(d)))
    assert np.abs(out_to_f64(m.run(scale)) - m.oracle(scale)).max() <= 2e-2


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "i8"])
@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 4), (16, 16), (32, 2)])
@pytest.mark.parametrize("bs", [16, 32])
def test_head128_group_sizes(kv, hq, hkv, bs):
    """head_dim 128 with blocks of 16 tokens or more (the kernel that shares K/V tiles through
    LDS, one-byte pools widened as they go to LDS): group sizes 2, 8, 1 and 16."""
    seq_lens = [1, 5, 40, 300, 17, 130, 64, 333]
    qlens = [1, 5, 40, 300, 16, 17, 1, 129]
    m = MQ(seq_lens, qlens, hq, hkv, 128, bs, kv, seed=hq + bs)
    scale = float(np.float32(1 / np.sqrt(128)))
    assert np.abs(out_to_f64(m.run(scale)) - m.oracle(scale)).max() <= 2e-2


@pytest.mark.parametrize("kv", ["e4m3", "i8"])
@pytest.mark.parametrize("hq,hkv,d,bs", [(16, 8, 64, 16), (32, 2, 128, 4), (8, 8, 64, 64), (32, 4, 64, 1)])
def test_one_byte_pools_across_shapes(kv, hq, hkv, d, bs):
    """e4m3 and int8 pools over group sizes 2, 16, 1, 8, both head sizes and small / large blocks."""
    seq_lens = [1, 40, 300, 17, 130]
    qlens = [1, 40, 100, 16, 3]
    m = MQ(seq_lens, qlens, hq, hkv, d, bs, kv, seed=hq + d + bs)
    scale = float(np.float32(1 / np.sqrt(d)))
    assert np.abs(out_to_f64(m.run(scale)) - m.oracle(scale)).max() <= 2e-2


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "i8"])
def test_peaky_scores(kv):
    """A large scale makes each row nearly one-hot: a wrong key or mask shows as an O(1) error."""
    m = MQ([70, 33, 129], [70, 9, 20], 32, 8, 128, 16, kv, seed=9)
    scale = float(np.float32(8 / np.sqrt(128)))
    assert np.abs(out_to_f64(m.run(scale)) - m.oracle(scale)).max() <= 2e-2


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, -0.7])
def test_negative_and_zero_scale(scale):
    """The kernel applies a negative scale as a sign flip of q; a zero scale gives the mean of visible rows."""
    m = MQ([50, 300, 33], [50, 70, 9], 32, 8, 128, 16, seed=13)
    scale = float(np.float32(scale))
    assert np.abs(out_to_f64(m.run(scale)) - m.oracle(scale)).max() <= 2e-2


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_scores_growing_along_the_context(kv):
    """Key norms growing with the position push the running maximum up step after step, so
    the output and sum are re-referenced many times within one query's pass."""
    m = MQ([600, 200, 97], [64, 200, 30], 32, 8, 128, 16, kv, seed=17, kgrow=0.05)
    scale = float(np.float32(1 / np.sqrt(128)))
    assert np.abs(out_to_f64(m.run(scale)) - m.oracle(scale)).max() <= 2e-2


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B", [63, 64, 65, 130])
def test_many_requests(B, d):
    """Up to 64 requests are ranked longest first inside the kernel, beyond that taken in order:
    both sides of the limit, with lengths that tie (head_dim 128 runs the LDS-sharing kernel)."""
    rng = np.random.default_rng(B)
    seq_lens = rng.integers(1, 200, B)
    seq_lens[::9] = 96                                # ties
    qlens = np.minimum(seq_lens, rng.integers(0, 40, B))
    m = MQ(seq_lens, qlens, 16, 4, d, 16, seed=B)
    scale = 0.125
    assert np.abs(out_to_f64(m.run(scale)) - m.oracle(scale)).max() <= 2e-2


def test_one_token_per_sequence_matches_decode():
    import torch
    import paged_kv_cache_112_amd as pa
    seq_lens = [1, 16, 17, 255, 700]
    m = MQ(seq_lens, [1] * len(seq_lens), 32, 8, 128, 16, seed=4)
    scale = float(np.float32(1 / np.sqrt(128)))
    mq = out_to_f64(m.run(scale))
    dq = to_dev(m.q)
    dec = pa.decode(dq, to_dev(m.kc), to_dev(m.vc), to_dev(m.bt), to_dev(m.seq_lens), scale,
                    max_context_len=max(seq_lens))
    torch.cuda.synchronize()
    ref = oracle.decode(m.q, m.kc, m.vc, m.bt, m.seq_lens, scale, "bf16", "bf16")
    assert np.abs(mq - ref).max() <= 2e-2
    assert np.abs(out_to_f64(dec) - ref).max() <= 2e-2


@pytest.mark.parametrize("d", [64, 128])
def test_sequences_with_no_new_tokens_and_bad_lengths_are_skipped(d):
    """A sequence with no rows writes nothing; one claiming more new tokens than its context is skipped."""
    import torch
    import paged_kv_cache_112_amd as pa
    m = MQ([40, 12, 30], [4, 0, 6], 16, 4, d, 16, seed=5)
    scale = 0.125
    ref = m.oracle(scale)
    out = m.run(scale)
    assert np.abs(out_to_f64(out) - ref).max() <= 2e-2
    bad = m.seq_lens.copy()
    bad[2] = 3                                        # 6 new tokens but a context of 3
    sentinel = torch.full_like(out, 7.0)
    pa.paged_attention(to_dev(m.q), to_dev(m.kc), to_dev(m.vc), to_dev(m.bt), to_dev(bad), to_dev(m.qsl), scale,
                       6, out=sentinel)
    torch.cuda.synchronize()
    got = out_to_f64(sentinel)
    assert np.all(got[4:10] == 7.0)                   # rows of the inconsistent sequence untouched
    assert np.abs(got[:4] - ref[:4]).max() <= 2e-2


def _chunk512_full_size(kv, peaky=False):
    """llama3_8b_chunk512 at full size; every row of three sequences and spread rows of all, vs the oracle.
    One-byte pools hold uniformly drawn codes (e4m3 NaN codes excluded) with scale 0.01."""
    import torch
    import paged_kv_cache_112_amd as pa
    w = make_mq_config("llama3_8b_chunk512")
    scale = float(np.float32(8 / np.sqrt(w.head_dim))) if peaky else w.scale
    rng = np.random.default_rng(w.seed)
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    ks = vs = 1.0
    if kv == "bf16":
        kc = f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
        vc = f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    elif kv == "e4m3":
        kc, vc = (rng.integers(0, 256, shape, dtype=np.uint8) for _ in range(2))
        for c in (kc, vc):
            c[(c & 0x7F) == 0x7F] -= 1
        ks = vs = 0.01
    else:
        kc, vc = (rng.integers(-127, 128, shape).astype(np.int8) for _ in range(2))
        ks = vs = 0.01
    q = f32_to_bf16_bits(w.mq_q_values())
    qsl = w.query_start_loc()
    out = pa.paged_attention(to_dev(q), to_dev(kc), to_dev(vc), to_dev(w.block_tables), to_dev(w.context_lens),
                             to_dev(qsl), scale, int(w.query_lens.max()), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    got = out_to_f64(out)
    rows = set(range(int(qsl[0]), int(qsl[0]) + 8)) | set(range(int(qsl[16]) + 500, int(qsl[17])))
    rows |= set(int(r) for r in rng.choice(int(qsl[-1]), 40, replace=False))
    rows |= {int(qsl[b + 1]) - 1 for b in range(w.num_seqs)}          # each sequence's last row
    ref = oracle.paged_attention(q, kc, vc, w.block_tables, w.context_lens, qsl, scale, kv, "bf16", ks, vs,
                                 rows=rows)
    idx = sorted(rows)
    err = float(np.abs(got[idx] - ref[idx]).max())
    print(f"chunk512 kv={kv} peaky={peaky}: {len(idx)} rows, max |out| {np.abs(ref[idx]).max():.3g}, "
          f"max abs err {err:.3g}", flush=True)
    assert err <= 2e-2
    return got[idx], ref[idx]


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "i8"])
def test_chunk512_full_size_sampled_rows(kv):
    _chunk512_full_size(kv)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_chunk512_full_size_peaky_scale(kv):
    """The same with scale 8/sqrt(d): a few keys carry each row's softmax, so a dropped, repeated
    or misplaced 32-key step moves a row by O(1), not by the ~1 % the standard scale would."""
    got, ref = _chunk512_full_size(kv, peaky=True)
    assert np.abs(ref).max() > 1.0                 # the outputs are single value rows, not averages
