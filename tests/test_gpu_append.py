"""pa_decode_append (the step's pa_write_kv done by the partition launch itself) against
pa_write_kv followed by pa_decode: outputs and pools bit for bit, and against the oracle."""
import numpy as np
import pytest

import oracle
from pools import append_step, build_host_inputs, custom_workload, from_dev, out_to_f64, to_dev
from workloads import make_config

pytestmark = pytest.mark.gpu

# lengths after the append: one token, tile and block edges, partition edges for 256/512/1024
EDGES = [1, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1000, 1024, 1025, 2049]


def _both(w, P, hq_scale=None):
    """Run unfused (write then decode) and fused on copies of the same pools; return both results."""
    import torch
    import paged_kv_cache_112_amd as pa
    h = build_host_inputs(w, skip_last=True)
    kn, vn, _, slots = append_step(w)
    q, bt, ctx = to_dev(h.q), to_dev(w.block_tables.astype(np.int32)), to_dev(w.context_lens.astype(np.int32))
    kn_d, vn_d = to_dev(kn), to_dev(vn)
    maxc = int(w.context_lens.max())
    kc_a, vc_a = to_dev(h.kc), to_dev(h.vc)
    kc_b, vc_b = kc_a.clone(), vc_a.clone()
    pa.write_kv(kn_d, vn_d, to_dev(slots.astype(np.int32)), kc_a, vc_a, h.k_scale, h.v_scale)
    out_a = pa.decode(q, kc_a, vc_a, bt, ctx, w.scale, max_context_len=maxc, partition_tokens=P,
                      k_scale=h.k_scale, v_scale=h.v_scale)
    out_b = pa.decode_append(q, kn_d, vn_d, kc_b, vc_b, bt, ctx, w.scale, max_context_len=maxc,
                             partition_tokens=P, k_scale=h.k_scale, v_scale=h.v_scale)
    torch.cuda.synchronize()
    return h, (from_dev(out_a), from_dev(kc_a), from_dev(vc_a)), (from_dev(out_b), from_dev(kc_b), from_dev(vc_b))


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "i8"])
@pytest.mark.parametrize("bs", [1, 16, 64, 1024])
@pytest.mark.parametrize("P", [256, 512, 1024])
def test_append_equals_write_then_decode(kv, bs, P):
    w = custom_workload(EDGES, 32, 8, 128, bs, kv=kv, seed=bs + P)
    _, a, b = _both(w, P)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "i8"])
def test_append_head_dim_64_group_2(kv):
    w = custom_workload([3, 16, 300, 700], 16, 8, 64, 16, kv=kv, seed=21)
    _, a, b = _both(w, 256)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("kv", ["bf16", "e4m3", "i8"])
def test_append_against_oracle(kv):
    """The fused call's pools equal the oracle's write, and its output the oracle's decode."""
    w = custom_workload([1, 17, 256, 257, 900], 32, 8, 128, 16, kv=kv, seed=33)
    h, _, (out, kc, vc) = _both(w, 256)
    kn, vn, kin, slots = append_step(w)
    kc_ref, vc_ref = h.kc.copy(), h.vc.copy()
    oracle.write_kv(kc_ref, vc_ref, kn, vn, slots, kv, kin, h.k_scale, h.v_scale)
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)
    ref = oracle.decode(h.q, kc_ref, vc_ref, w.block_tables, w.context_lens, w.scale, kv, "bf16",
                        h.k_scale, h.v_scale)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.abs(got - ref).max() <= 2e-2


def test_append_beyond_the_dense_grid():
    """More than 1024 sequences: the partition grid is (partitions x heads, sequences), not the
    dense numbering; fused and unfused still agree bit for bit."""
    rng = np.random.default_rng(8)
    ctx = rng.integers(1, 600, 1100)
    w = custom_workload(ctx, 8, 2, 64, 16, seed=9)
    _, a, b = _both(w, 256)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_append_llama3_8b_b64_full_size():
    """The batch-64 step at full size, fused against unfused, bit for bit."""
    w = make_config("llama3_8b_b64")
    _, a, b = _both(w, 256)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_empty_context_appends_nothing():
    """context_lens[b] == 0: zeros out, and no row of that sequence is written."""
    import torch
    import paged_kv_cache_112_amd as pa
    w = custom_workload([5, 3], 8, 2, 64, 16, seed=3)
    h = build_host_inputs(w, skip_last=True)
    kn, vn, _, _ = append_step(w)
    ctx = w.context_lens.astype(np.int32).copy()
    ctx[0] = 0
    kc, vc = to_dev(h.kc), to_dev(h.vc)
    out = pa.decode_append(to_dev(h.q), to_dev(kn), to_dev(vn), kc, vc, to_dev(w.block_tables.astype(np.int32)),
                           to_dev(ctx), w.scale, max_context_len=5)
    torch.cuda.synchronize()
    assert np.all(out_to_f64(out)[0] == 0.0)
    kc_h = from_dev(kc)
    changed = np.argwhere(np.any(kc_h.view(np.uint16) != h.kc.view(np.uint16), axis=(2, 3)))
    slot1 = w.append_slots()[1]
    assert [tuple(x) for x in changed] == [(slot1 // w.block_size, slot1 % w.block_size)]
