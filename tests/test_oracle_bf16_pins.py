"""The oracle's bf16 decoding pinned to the format definition and to torch's own bf16 type.

A bf16 value has a sign bit, an 8-bit exponent with bias 127 and a 7-bit fraction:
the upper half of a binary32.  These tests derive every pattern's value from those
fields as an exact rational (no bit shifts, no float32 view), so a wrong shift, a
lower-half read or a lost sign in ``bf16_to_f64`` or in the bf16 branch of the
write's quantizer input fails here.  The identity-table case decodes its bf16
inputs through torch's bfloat16 dtype, an implementation that shares nothing with
the oracle, and compares with torch's float64 scaled_dot_product_attention
(ai-infra-handbooks "Paged KV cache", section "Paged attention": paged and
contiguous storage give the same attention).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from conftest import GOLDEN
from test_oracle_pins import _E4M3_CODE, _e4m3_rne_sat_reference, _fp_round, _golden, _rne_int
from workloads import slot_mapping_for

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _bf16_from_fields(bits: int):
    """Exact value of a bf16 pattern: None for NaN, +-inf as floats, else a Fraction (and its sign bit)."""
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    sign = -1 if s else 1
    if e == 0xFF:
        return None if m else sign * math.inf
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(1, 2 ** 126)       # subnormal: 0.m * 2^-126
    return sign * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def test_bf16_decode_every_pattern_from_fields():
    got = oracle.bf16_to_f64(ALL)
    via_to_f64 = oracle.to_f64(ALL, "bf16")
    assert np.array_equal(got, via_to_f64, equal_nan=True)
    n_sub = n_nan = 0
    for i in range(65536):
        ref = _bf16_from_fields(i)
        g = float(got[i])
        if ref is None:
            assert math.isnan(g), hex(i)
            n_nan += 1
        elif isinstance(ref, float):
            assert g == ref, hex(i)
        else:
            assert Fraction(g) == ref, hex(i)
            assert math.copysign(1.0, g) == (-1.0 if i & 0x8000 else 1.0), hex(i)   # -0 keeps its sign
            if (i >> 7) & 0xFF == 0 and i & 0x7F:
                n_sub += 1
    assert n_sub == 2 * 127 and n_nan == 2 * 127


def test_bf16_decode_known_values():
    known = {0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3F00: 0.5, 0x4049: 3.140625,
             0x7F7F: 3.3895313892515355e38, 0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x7F80: math.inf,
             0xFF80: -math.inf, 0xC2F7: -123.5}
    for bits, v in known.items():
        assert oracle.bf16_to_f64(np.array([bits], dtype=np.uint16))[0] == v, hex(bits)


def _rows(bits):
    return bits.reshape(-1, 4, 64)


@pytest.mark.parametrize("scale", [1.0, float(np.float32(5.0 / 448)), float(np.float32(1 / 3))])
def test_bf16_input_to_e4m3_pool_from_fields(scale):
    """The bf16 -> e4m3 write: each pattern's field-derived value, one fp32 multiply by fp32(1/scale),
    then nearest-even with saturation, must be the code the oracle stores."""
    kc = np.zeros((16, 16, 4, 64), dtype=np.uint8)
    vc = np.zeros_like(kc)
    slots = np.arange(256, dtype=np.int32)[::-1].copy()
    oracle.write_kv(kc, vc, _rows(ALL), _rows(ALL[::-1].copy()), slots, "e4m3", "bf16", scale, scale)
    stored = kc.reshape(256, 256)[slots].reshape(-1)          # row i went to slot slots[i]
    inv = _fp_round(Fraction(1) / Fraction(scale), 23, -126)
    for i in range(65536):
        ref = _bf16_from_fields(i)
        neg = bool(i & 0x8000)
        if ref is None:
            assert stored[i] & 0x7F == 0x7F, hex(i)
            continue
        if isinstance(ref, float):
            want = 0xFE if neg else 0x7E
        else:
            y = _fp_round(ref * inv, 23, -126)
            want = _E4M3_CODE[abs(_e4m3_rne_sat_reference(y))] | (0x80 if neg else 0)
        assert stored[i] == want, (hex(i), scale)


@pytest.mark.parametrize("scale", [1.0, float(np.float32(5.0 / 127))])
def test_bf16_input_to_int8_pool_from_fields(scale):
    kc = np.zeros((16, 16, 4, 64), dtype=np.int8)
    vc = np.zeros_like(kc)
    slots = np.arange(256, dtype=np.int32)
    oracle.write_kv(kc, vc, _rows(ALL), _rows(ALL), slots, "i8", "bf16", scale, scale)
    stored = kc.reshape(-1)
    inv = _fp_round(Fraction(1) / Fraction(scale), 23, -126)
    for i in range(65536):
        ref = _bf16_from_fields(i)
        if ref is None:
            want = 0
        elif isinstance(ref, float):
            want = 127 if ref > 0 else -127
        else:
            y = _fp_round(ref * inv, 23, -126)
            want = 127 if y > 2 ** 128 else -127 if y < -(2 ** 128) else max(-127, min(127, _rne_int(y)))
        assert int(stored[i]) == want, (hex(i), scale)


def test_bf16_pool_write_is_a_byte_copy():
    kc = np.full((16, 16, 4, 64), 0x7FC0, dtype=np.uint16)
    vc = kc.copy()
    slots = np.arange(256, dtype=np.int32)
    oracle.write_kv(kc, vc, _rows(ALL), _rows(ALL[::-1].copy()), slots, "bf16", "bf16")
    assert np.array_equal(kc.reshape(-1), ALL) and np.array_equal(vc.reshape(-1), ALL[::-1])


def _torch_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 patterns decoded by torch's bfloat16 dtype, widened to float64."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_bf16_identity_table_equals_torch_sdpa(kv):
    """The page's check shape (8 heads over 2 KV heads, head dim 64, blocks of 4 tokens, requests of
    37, 5 and 20 tokens, its printed tables) with bf16 q and a bf16 or e4m3 pool: the oracle equals
    torch's float64 SDPA on contiguous K/V decoded by torch's own bf16 / float8_e4m3fn types."""
    g = _golden("p2_round_robin_tables.json")
    hq, hkv, d, bs = g["num_heads"], g["num_kv_heads"], g["head_dim"], g["block_size"]
    ctx = g["seq_lens"]
    rng = np.random.default_rng(77)
    from workloads import f32_to_bf16_bits
    Ks = [f32_to_bf16_bits(rng.standard_normal((n, hkv, d), dtype=np.float32)) for n in ctx]
    Vs = [f32_to_bf16_bits(rng.standard_normal((n, hkv, d), dtype=np.float32)) for n in ctx]
    q = f32_to_bf16_bits(rng.standard_normal((len(ctx), hq, d), dtype=np.float32))
    mb = max(len(t) for t in g["tables"])
    bt = np.zeros((len(ctx), mb), dtype=np.int32)
    for i, t in enumerate(g["tables"]):
        bt[i, :len(t)] = t
    store = {"bf16": (np.uint16, 0x7FC0), "e4m3": (np.uint8, 0x7F)}[kv]
    kc = np.full((g["num_blocks"], bs, hkv, d), store[1], dtype=store[0])
    vc = kc.copy()
    ks, vs = (float(np.float32(0.0123)), float(np.float32(0.0101))) if kv == "e4m3" else (1.0, 1.0)
    for K, V, t in zip(Ks, Vs, g["tables"]):
        sl = np.asarray(slot_mapping_for(t, range(len(K)), bs), dtype=np.int32)
        oracle.write_kv(kc, vc, K, V, sl, kv, "bf16", ks, vs)
    scale = float(np.float32(d ** -0.5))
    got = oracle.decode(q, kc, vc, bt, np.array(ctx), scale, kv, "bf16", ks, vs)
    # the contiguous reference reads the stored codes back in logical order, decoded by torch
    rep = hq // hkv
    qt = _torch_bf16(q)
    for b, n in enumerate(ctx):
        t = np.arange(n)
        phys = bt[b, t // bs]
        if kv == "bf16":
            K = _torch_bf16(kc[phys, t % bs])
            V = _torch_bf16(vc[phys, t % bs])
        else:
            K = torch.from_numpy(kc[phys, t % bs]).view(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(ks))
            V = torch.from_numpy(vc[phys, t % bs]).view(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(vs))
        kt = K.repeat_interleave(rep, 1).transpose(0, 1).contiguous()        # [H, n, d]
        vt = V.repeat_interleave(rep, 1).transpose(0, 1).contiguous()
        ref = F.scaled_dot_product_attention(qt[b][:, None, :], kt, vt, scale=scale)[:, 0, :].numpy()
        assert np.abs(got[b] - ref).max() <= 1e-12, (kv, b)
