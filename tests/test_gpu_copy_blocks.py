"""pa_copy_blocks against the oracle: whole pools bit for bit, and copy-on-write end to end."""
import numpy as np
import pytest

import oracle
from pools import POISON, STORAGE, build_host_inputs, from_dev, out_to_f64, to_dev
from test_cow import cow_scenario
from workloads import f32_to_bf16_bits, make_config

pytestmark = pytest.mark.gpu


def _random_pool(rng, nb, bs, hkv, d, fmt):
    shape = (nb, bs, hkv, d)
    if fmt == "f32":
        return rng.standard_normal(shape).astype(np.float32)
    if fmt == "bf16":
        return rng.integers(0, 1 << 16, shape, dtype=np.uint16)
    return rng.integers(0, 256, shape, dtype=np.uint8)


def _pairs(rng, nb, n):
    """n pairs with distinct destinations that are never sources, plus padding and out-of-pool ids."""
    ids = rng.permutation(nb)
    src = ids[:n].astype(np.int32)
    dst = ids[n:2 * n].astype(np.int32)
    src[::7] = -1                                   # padding: skipped
    dst[3::11] = nb + 5                             # outside the pool: skipped
    return src, dst


@pytest.mark.parametrize("fmt", ["f32", "bf16", "e4m3"])
@pytest.mark.parametrize("bs,hkv,d", [(1, 8, 128), (16, 8, 128), (16, 2, 64), (256, 4, 64)])
@pytest.mark.parametrize("n", [1, 5, 40])
def test_copy_blocks_bit_exact(fmt, bs, hkv, d, n):
    import torch
    import paged_kv_cache_112_amd as pa
    rng = np.random.default_rng(bs * 131 + n + len(fmt))
    nb = 2 * n + 7
    kc, vc = _random_pool(rng, nb, bs, hkv, d, fmt), _random_pool(rng, nb, bs, hkv, d, fmt)
    src, dst = _pairs(rng, nb, n)
    dk, dv = to_dev(kc), to_dev(vc)
    pa.copy_blocks(dk, dv, to_dev(src), to_dev(dst))
    torch.cuda.synchronize()
    oracle.copy_blocks(kc, vc, src, dst)
    assert np.array_equal(from_dev(dk).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(from_dev(dv).view(np.uint8), vc.view(np.uint8))


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("prefix,bs", [(40, 16), (7, 4), (100, 64), (32, 16)])
def test_copy_on_write_decode(fmt, prefix, bs):
    """Fork, copy the contested block, write each sequence's token, decode: all on the GPU."""
    import torch
    import paged_kv_cache_112_amd as pa
    state, private, q, fmt, pre = cow_scenario(fmt=fmt, prefix=prefix, bs=bs)
    kc_ref, vc_ref, tables, ctx, copies = state
    pre_k, pre_v, new_k, new_v, slots, kin = pre
    dk, dv = to_dev(pre_k), to_dev(pre_v)
    src = np.array([c[0] for c in copies], dtype=np.int32)
    dst = np.array([c[1] for c in copies], dtype=np.int32)
    pa.copy_blocks(dk, dv, to_dev(src), to_dev(dst))
    pa.write_kv(to_dev(new_k), to_dev(new_v), to_dev(slots), dk, dv)
    out = pa.decode(to_dev(q), dk, dv, to_dev(tables), to_dev(ctx), 0.125, max_context_len=int(ctx.max()))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dk).view(np.uint8), kc_ref.view(np.uint8))
    assert np.array_equal(from_dev(dv).view(np.uint8), vc_ref.view(np.uint8))
    ref = oracle.decode(q, kc_ref, vc_ref, tables, ctx, 0.125, fmt, fmt)
    tol = 1e-5 if fmt == "f32" else 2e-2
    assert np.abs(out_to_f64(out) - ref).max() <= tol


def test_copy_blocks_full_size_fp8_pool():
    """4,000 block copies over the 34,074-block e4m3 pools of the shared-prefix workload."""
    import torch
    import paged_kv_cache_112_amd as pa
    w = make_config("llama3_8b_fp8_prefix")
    rng = np.random.default_rng(77)
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kc = rng.integers(0, 256, shape, dtype=np.uint8)
    vc = rng.integers(0, 256, shape, dtype=np.uint8)
    src, dst = _pairs(rng, w.num_blocks, 4000)
    dk, dv = to_dev(kc), to_dev(vc)
    pa.copy_blocks(dk, dv, to_dev(src), to_dev(dst))
    torch.cuda.synchronize()
    oracle.copy_blocks(kc, vc, src, dst)
    assert np.array_equal(from_dev(dk), kc)
    assert np.array_equal(from_dev(dv), vc)


@pytest.mark.parametrize("fmt", ["bf16", "e4m3", "i8"])
def test_multi_layer_pool_in_one_allocation(fmt):
    """Pools [L, nb, bs, H_kv, d] in one allocation: per-layer writes and decodes through layer views,
    and copy-on-write copies of every layer in one launch."""
    import torch
    import paged_kv_cache_112_amd as pa
    from pools import POISON, STORAGE
    L, nb, bs, hkv, d, hq = 3, 24, 16, 2, 128, 8
    rng = np.random.default_rng(21)
    kc = np.full((L, nb, bs, hkv, d), POISON[fmt], dtype=STORAGE[fmt])
    vc = np.full_like(kc, POISON[fmt])
    ctx = np.array([40, 17, 64], dtype=np.int32)
    bt = np.array([[3, 9, 1, 0], [5, 2, 0, 0], [7, 11, 13, 4]], dtype=np.int32)
    scale_k = scale_v = 1.0 if fmt == "bf16" else (0.02 if fmt == "e4m3" else 0.03)
    dk, dv = to_dev(kc), to_dev(vc)
    for l in range(L):                              # each layer's own values, written through its view
        for b, c in enumerate(ctx):
            pos = np.arange(c)
            kk = f32_to_bf16_bits(rng.standard_normal((c, hkv, d)).astype(np.float32))
            vv = f32_to_bf16_bits(rng.standard_normal((c, hkv, d)).astype(np.float32))
            slots = (bt[b, pos // bs] * bs + pos % bs).astype(np.int32)
            oracle.write_kv(kc[l], vc[l], kk, vv, slots, fmt, "bf16", scale_k, scale_v)
            pa.write_kv(to_dev(kk), to_dev(vv), to_dev(slots), dk[l], dv[l], scale_k, scale_v)
    src = np.array([9, 13], dtype=np.int32)
    dst = np.array([20, 21], dtype=np.int32)
    pa.copy_blocks(dk, dv, to_dev(src), to_dev(dst))
    for l in range(L):
        oracle.copy_blocks(kc[l], vc[l], src, dst)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dk).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(from_dev(dv).view(np.uint8), vc.view(np.uint8))
    # sequences 0 and 2 now read the copies: same values, other blocks
    bt2 = bt.copy()
    bt2[0, 1], bt2[2, 2] = 20, 21
    q = f32_to_bf16_bits(rng.standard_normal((3, hq, d)).astype(np.float32))
    for l in range(L):
        out = pa.decode(to_dev(q), dk[l], dv[l], to_dev(bt2), to_dev(ctx), 0.088, max_context_len=64,
                        k_scale=scale_k, v_scale=scale_v)
        torch.cuda.synchronize()
        ref = oracle.decode(q, kc[l], vc[l], bt, ctx, 0.088, fmt, "bf16", scale_k, scale_v)
        assert np.abs(out_to_f64(out) - ref).max() <= 2e-2
