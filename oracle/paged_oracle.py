"""CPU oracle for the paged-KV hot path: slot-mapping write and paged decode attention.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never uses it, it shares no code with the library, and it imports
nothing from the library or from the input generators.

Everything is plain numpy in float64.  Storage formats are decoded here from
their definitions: bf16 as the upper half of a float32, OCP E4M3FN from its
sign/exponent/mantissa fields.  Arrays are passed as raw storage:

  * "f32"  -> float32 values
  * "bf16" -> uint16 bit patterns
  * "e4m3" -> uint8 codes (values are code * per-tensor scale)
  * "i8"   -> int8 codes (values are code * per-tensor scale)

Caches have the layout [num_blocks, block_size, H_kv, d_h] (LLM stack book
"4.6 PagedAttention & KV-Cache Memory Management", section "Block Tables, the
Allocator & Copy-on-Write"; ai-infra-handbooks "Paged KV cache", section
"Implementation").

What is computed (each function names its passage):

  * ``write_kv``: every new token i with slot_mapping[i] >= 0 lands in
    block slot // B at offset slot % B of the flat pool; a same-format write
    is a byte copy, an e4m3 pool stores the quantized value.
  * ``slot_mapping``: each new token's slot from its sequence's block table.
  * ``copy_blocks``: copy-on-write's device step, whole physical blocks of both
    pools copied as stored.
  * ``decode``: for every sequence and query head, softmax(scale * q . K^T) V
    over the context's tokens, gathering each token's K/V row through the
    block table.  Both the LLM stack book ("The PagedAttention Kernel") and the
    mohdvasim.com "PagedAttention - Explained" page ("The Custom CUDA Kernel
    Overview") state that the paged kernel computes exactly the values of plain
    attention, so the oracle computes the plain definition: gather the tokens in
    logical order, two-pass softmax, weighted sum.
  * ``paged_attention``: several new tokens per sequence, each attending causally
    to the context up to its own position (ai-infra-handbooks "Paged attention").
  * ``decode_partials`` / ``merge_partials``: the split-K decomposition of the
    same sum over token partitions (LLM stack book, "Performance
    considerations": long sequences are split across thread blocks and the
    pieces reduced afterwards), written with base-2 exponents.

Readings where the pages are silent are listed in the repository's design
notes; the ones that shape this file: context_len 0 gives a zero output; GQA
query head h uses KV head h // (H_q / H_kv); fp8 is OCP E4M3FN with one fp32
scale per pool, quantized as RNE-with-saturation of fp32(x * fp32(1/scale));
NaN quantizes to the NaN code with the input's sign.

Pins (tests marked "not gpu"): page-printed slot traces and sizes, the KV-size
closed form through the read-byte counter, equality with torch's CPU
scaled_dot_product_attention under an identity block table, invariance under
block permutation and block size, brute force at 50 digits on tiny inputs,
closed-form special cases, and an exhaustive check of the e4m3 codec against
exact rational rounding.
"""
from __future__ import annotations

import math

import numpy as np

FORMATS = ("f32", "bf16", "e4m3", "i8")
ELEM_BYTES = {"f32": 4, "bf16": 2, "e4m3": 1, "i8": 1}
E4M3_MAX = 448.0
LOG2E = 1.4426950408889634


# ---------------------------------------------------------------------------
# KV-size closed form
# ---------------------------------------------------------------------------
def kv_cache_bytes(num_layers: int, num_kv_heads: int, head_dim: int, seq_len: int,
                   bytes_per_elem: int, batch: int = 1) -> int:
    """2 * L * H_kv * d_h * s * b bytes per sequence, times the batch.

    LLM stack book, section "The size formula" (restated in its Exercise 1);
    mohdvasim.com "PagedAttention - Explained", section "Memory Consumption
    Formula" and Appendix A.  The 2 is one K and one V vector.
    """
    return 2 * num_layers * num_kv_heads * head_dim * seq_len * bytes_per_elem * batch


# ---------------------------------------------------------------------------
# storage codecs
# ---------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64: the pattern is the upper half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_values() -> np.ndarray:
    """Value of each of the 256 OCP E4M3FN codes (float64; NaN for S.1111.111).

    Fields: sign 1 bit, exponent 4 bits with bias 7, mantissa 3 bits.
    Exponent field 0 is subnormal: m/8 * 2^-6.  There is no infinity; the
    largest finite magnitude is 1.75 * 2^8 = 448.
    """
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = math.nan
        elif e == 0:
            out[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_E4M3_TABLE = e4m3_values()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3FN codes: nearest, ties to even, saturating at +-448.

    Inputs of magnitude >= 448 (infinities included) become +-448; NaN becomes
    the NaN code carrying the input's sign.  Zero keeps its sign.
    """
    y = np.ascontiguousarray(y, dtype=np.float32)
    sign = ((y.view(np.uint32) >> np.uint32(31)).astype(np.uint8) << np.uint8(7))
    nan = np.isnan(y)
    a = np.abs(y.astype(np.float64))
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    # spacing of representable values around a: 2^(floor(log2 a) - 3), never below 2^-9
    _, e = np.frexp(a)                       # a = f * 2^e with f in [0.5, 1)
    ex = np.maximum(e - 1, -6)
    quantum = np.ldexp(1.0, ex - 3)
    v = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)   # rint: half to even
    _, e2 = np.frexp(v)
    ex2 = e2 - 1
    normal = v >= 2.0 ** -6
    exp_field = np.where(normal, ex2 + 7, 0).astype(np.int64)
    mant = np.where(normal, v * np.ldexp(1.0, -ex2) * 8.0 - 8.0, v * 2.0 ** 9)
    code = (exp_field << 3) | mant.astype(np.int64)
    code = np.where(nan, 0x7F, code).astype(np.uint8)
    return code | sign


def e4m3_quantize(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Stored code of real value x for a pool with per-tensor scale: q8(fp32(x * fp32(1/scale)))."""
    inv = np.float32(1.0) / np.float32(scale)                 # one fp32 division
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.asarray(x_f32, dtype=np.float32) * inv         # one fp32 rounding
    return e4m3_encode(y)


def int8_quantize(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Stored int8 code of real value x for a pool with per-tensor scale.

    The pages say only that quantizing the cache to int8 halves the bytes per
    element (LLM stack book, "Why it matters"); the reading here is symmetric
    per-tensor quantization: y = fp32(x * fp32(1/scale)) (one fp32 rounding),
    then round to nearest with ties to even and clamp to [-127, 127]; NaN -> 0.
    """
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (np.asarray(x_f32, dtype=np.float32) * inv).astype(np.float64)
    code = np.clip(np.rint(np.nan_to_num(y, nan=0.0, posinf=127.0, neginf=-127.0)), -127, 127)
    return code.astype(np.int8)


def to_f64(arr: np.ndarray, fmt: str, scale: float = 1.0) -> np.ndarray:
    """Decode stored values to float64 (e4m3 codes are multiplied by their scale)."""
    if fmt == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_to_f64(arr)
    if fmt == "e4m3":
        return e4m3_to_f64(arr) * float(np.float32(scale))
    if fmt == "i8":
        return np.asarray(arr, dtype=np.int8).astype(np.float64) * float(np.float32(scale))
    raise ValueError(fmt)


def _as_f32(arr: np.ndarray, fmt: str) -> np.ndarray:
    """Exact float32 view of f32 or bf16 input values (the quantizer's input)."""
    if fmt == "f32":
        return np.asarray(arr, dtype=np.float32)
    if fmt == "bf16":
        return (np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# slot-mapping write
# ---------------------------------------------------------------------------
def write_kv(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray, v: np.ndarray,
             slot_mapping: np.ndarray, kv_format: str, in_format: str,
             k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Scatter new tokens' K and V rows into the pools, in place.

    Token i goes to flat slot s = slot_mapping[i]: block s // B, offset s % B
    (LLM stack book, "From Python bookkeeping to the tensors the kernel
    actually takes": the pool viewed as [num_blocks * B, H_kv, d_h]; "Putting It
    Together": divmod of the slot).  A negative slot skips the token.  When
    the pool format equals the input format the row is copied bit for bit;
    an e4m3 pool stores e4m3_quantize(row, scale), an int8 pool int8_quantize.
    """
    B = k_cache.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if kv_format == "e4m3":
        kq = e4m3_quantize(_as_f32(k, in_format), k_scale)
        vq = e4m3_quantize(_as_f32(v, in_format), v_scale)
    elif kv_format == "i8":
        kq = int8_quantize(_as_f32(k, in_format), k_scale)
        vq = int8_quantize(_as_f32(v, in_format), v_scale)
    else:
        if kv_format != in_format:
            raise ValueError("a non-fp8 pool takes input of its own format")
        kq, vq = np.asarray(k), np.asarray(v)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), B)
        k_cache[blk, off] = kq[i]
        v_cache[blk, off] = vq[i]


def slot_mapping(block_tables: np.ndarray, seq_lens, query_start_loc, block_size: int, num_tokens: int):
    """Slots of this step's new tokens (int64 [num_tokens]).

    New token j of sequence b sits at position p = seq_lens[b] - n_b + j and is
    stored in logical block p // B at offset p % B, i.e. at slot
    table[b][p // B] * B + p % B (ai-infra-handbooks "Paged KV cache", section
    "Block tables and slot mapping"; int8ai.com, "How the Block Table Works").
    ``query_start_loc`` None means one new token per sequence, in row b.  A
    position outside the table gets -1.
    """
    out = np.full(num_tokens, -1, dtype=np.int64)
    for b in range(len(seq_lens)):
        if query_start_loc is None:
            r0, n = b, 1
        else:
            r0, n = int(query_start_loc[b]), int(query_start_loc[b + 1]) - int(query_start_loc[b])
        S = int(seq_lens[b])
        for j in range(n):
            p = S - n + j
            lb, off = divmod(p, block_size)
            if 0 <= r0 + j < num_tokens and p >= 0 and lb < block_tables.shape[1]:
                out[r0 + j] = int(block_tables[b][lb]) * block_size + off
    return out


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, src, dst) -> None:
    """Copy-on-write's device step, in place: physical block src[i] -> dst[i] in both pools.

    LLM stack book, "Copy-on-write for shared prefixes": a sequence about to
    append into a block whose reference count exceeds one gets a fresh block, the
    contested block is copied into it, and the sequence's table entry is
    redirected; ai-infra-handbooks "Paged KV cache", exercise 2, describes the
    same steps.  A block is copied whole -- every offset, every KV head -- as
    stored.  Every copy reads the pools as they were before the call; a pair with
    an id outside the pool (negative padding included) is skipped.
    """
    nb = k_cache.shape[0]
    k_before, v_before = k_cache.copy(), v_cache.copy()
    for s, d in zip(np.asarray(src, dtype=np.int64), np.asarray(dst, dtype=np.int64)):
        if not (0 <= s < nb and 0 <= d < nb):
            continue
        k_cache[d] = k_before[s]
        v_cache[d] = v_before[s]


# ---------------------------------------------------------------------------
# paged decode
# ---------------------------------------------------------------------------
def _gather(cache: np.ndarray, table_row: np.ndarray, n: int, kvh: int, fmt: str, scale: float,
            counter: dict | None) -> np.ndarray:
    """Rows of tokens 0..n-1 of one sequence and KV head, in logical order (float64 [n, d]).

    Address translation per token t: physical block = table[t // B], offset t % B
    (mohdvasim.com "The Custom CUDA Kernel Overview"; int8ai.com "How the Block
    Table Works").
    """
    B = cache.shape[1]
    t = np.arange(n, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[t // B]
    rows = cache[phys, t % B, kvh, :]
    if counter is not None:
        counter["kv_bytes"] = counter.get("kv_bytes", 0) + rows.size * ELEM_BYTES[fmt]
    return to_f64(rows, fmt, scale)


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
           context_lens: np.ndarray, scale: float, kv_format: str, q_format: str,
           k_scale: float = 1.0, v_scale: float = 1.0, seqs=None,
           counter: dict | None = None) -> np.ndarray:
    """out[b, h] = softmax_t(scale * q[b, h] . K_t) . V_t over t < context_lens[b].

    q: [B, H_q, d] storage of ``q_format``; caches [nb, B, H_kv, d] of
    ``kv_format``; block_tables [B, max_blocks] int32; scale is taken as the
    float32 the kernels receive.  Query head h reads KV head h // (H_q / H_kv)
    (LLM stack book "The PagedAttention Kernel": GQA head mapping).  A context
    of length 0 gives zeros.  Returns float64 [B, H_q, d]; rows of sequences not
    in ``seqs`` (when given) are NaN.  ``counter['kv_bytes']`` accumulates the
    K and V bytes gathered (each KV row once per KV head).
    """
    nseq, hq, d = q.shape
    hkv = k_cache.shape[2]
    if hq % hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    grp = hq // hkv
    s64 = float(np.float32(scale))
    qf = to_f64(q, q_format)
    out = np.full((nseq, hq, d), np.nan)
    for b in (range(nseq) if seqs is None else seqs):
        n = int(context_lens[b])
        if n == 0:
            out[b] = 0.0
            continue
        for g in range(hkv):
            K = _gather(k_cache, block_tables[b], n, g, kv_format, k_scale, counter)
            V = _gather(v_cache, block_tables[b], n, g, kv_format, v_scale, counter)
            for h in range(g * grp, (g + 1) * grp):
                logits = s64 * (K @ qf[b, h])
                w = np.exp(logits - logits.max())
                out[b, h] = (w @ V) / w.sum()
    return out


def paged_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                    seq_lens: np.ndarray, query_start_loc: np.ndarray, scale: float, kv_format: str,
                    q_format: str, k_scale: float = 1.0, v_scale: float = 1.0, rows=None) -> np.ndarray:
    """Causal attention of several new tokens per sequence over the paged context.

    ai-infra-handbooks "Paged KV cache", section "Paged attention": sequence b's
    new tokens are q[qsl[b]:qsl[b+1]], the last n_b positions of a context of
    seq_lens[b] tokens; new token j sits at position seq_lens[b] - n_b + j and
    may see positions 0 .. that position (the lower-triangular mask offset by
    seq_len - n).  K/V are gathered through the block table in logical order,
    query head h reads KV head h // (H_q / H_kv), and each row is a plain
    two-pass softmax-weighted sum.  Returns float64 [N, H_q, d]; when ``rows`` (a set
    of row indices) is given, only those rows are computed and the others are NaN.
    """
    ntok, hq, d = q.shape
    hkv = k_cache.shape[2]
    grp = hq // hkv
    s64 = float(np.float32(scale))
    qf = to_f64(q, q_format)
    out = np.full((ntok, hq, d), np.nan)
    for b in range(len(seq_lens)):
        start, end = int(query_start_loc[b]), int(query_start_loc[b + 1])
        S, n = int(seq_lens[b]), end - start
        want = [j for j in range(n) if rows is None or start + j in rows]
        if not want:
            continue
        for g in range(hkv):
            K = _gather(k_cache, block_tables[b], S, g, kv_format, k_scale, None)
            V = _gather(v_cache, block_tables[b], S, g, kv_format, v_scale, None)
            for j in want:
                p = S - n + j                       # this token's position
                for h in range(g * grp, (g + 1) * grp):
                    logits = s64 * (K[:p + 1] @ qf[start + j, h])
                    w = np.exp(logits - logits.max())
                    out[start + j, h] = (w @ V[:p + 1]) / w.sum()
    return out


# ---------------------------------------------------------------------------
# split-K partials and their merge
# ---------------------------------------------------------------------------
def decode_partials(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                    context_lens: np.ndarray, scale: float, kv_format: str, q_format: str,
                    partition_tokens: int, k_scale: float = 1.0, v_scale: float = 1.0, seqs=None):
    """Per-partition softmax pieces of ``decode`` in base 2.

    Tokens [j*P, (j+1)*P) form partition j.  With x_t = scale * q.K_t * log2(e):
    m_j = max x_t, l_j = sum 2^(x_t - m_j), o_j = sum 2^(x_t - m_j) V_t.
    Returns (m, l, o) float64 of shapes [B, H_q, J], [B, H_q, J], [B, H_q, J, d]
    with J = ceil(max context / P); partitions past a sequence's end hold NaN.
    """
    nseq, hq, d = q.shape
    hkv = k_cache.shape[2]
    grp = hq // hkv
    P = int(partition_tokens)
    J = max(1, -(-int(np.max(context_lens)) // P))
    s64 = float(np.float32(scale))
    qf = to_f64(q, q_format)
    m = np.full((nseq, hq, J), np.nan)
    l = np.full((nseq, hq, J), np.nan)
    o = np.full((nseq, hq, J, d), np.nan)
    for b in (range(nseq) if seqs is None else seqs):
        n = int(context_lens[b])
        for g in range(hkv):
            K = _gather(k_cache, block_tables[b], n, g, kv_format, k_scale, None)
            V = _gather(v_cache, block_tables[b], n, g, kv_format, v_scale, None)
            for h in range(g * grp, (g + 1) * grp):
                x = s64 * (K @ qf[b, h]) * LOG2E
                for j in range(-(-n // P)):
                    sl = slice(j * P, min(n, (j + 1) * P))
                    mj = x[sl].max()
                    w = np.exp2(x[sl] - mj)
                    m[b, h, j], l[b, h, j], o[b, h, j] = mj, w.sum(), w @ V[sl]
    return m, l, o


def merge_partials(m: np.ndarray, l: np.ndarray, o: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """Combine partition pieces: out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j, M = max_j m_j.

    m, l: [B, H, J]; o: [B, H, J, d]; counts[b] = number of valid partitions of
    sequence b (the rest are ignored).  A sequence with 0 partitions gives zeros.
    """
    nseq, hq, J, d = o.shape
    out = np.zeros((nseq, hq, d))
    for b in range(nseq):
        c = int(counts[b])
        if c == 0:
            continue
        mb = m[b, :, :c]
        M = mb.max(axis=1, keepdims=True)
        w = np.exp2(mb - M)
        out[b] = np.einsum("hj,hjd->hd", w, o[b, :, :c]) / (w * l[b, :, :c]).sum(axis=1)[:, None]
    return out
