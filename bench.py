"""Benchmark of the paged-KV hot path on one MI355X.

Workload: one Llama-3-8B attention layer (32 query heads, 8 KV heads, head dim
128, bf16), batch 64, block size 16, context lengths = prompt U[100,2000] +
output U[20,1500] from the seeded generator, physical blocks shuffled over a
pool 10 % larger than needed.  One step is the whole hot path for one batch:
pa_write_kv of this step's 64 tokens, then pa_decode (the partition kernel, which
also merges the split-K pieces in its last workgroup of each sequence); with
--fused the decode launch writes the tokens itself (pa_decode_append).
Each step uses the next of L layer-pool copies, as a model's layers would, so
the 256 MB MALL cannot serve a pool read by an earlier step (the same effect as
flushing it before each step).

Prints one JSON line: value = algorithmic bytes of the step / step time (GB/s);
roofline = pa_decode (partition + merge, the dominant launch) against HBM peak,
timed live with HIP events on the stream it runs on; contiguous = the same decode
over identity-ordered block tables; cpu_baseline = the CPU oracle on all host cores
and on one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "llama3_8b_b64"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20          # MI355X memory-side cache (Infinity Cache)
LAYERS = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_mfma_llama3_8b_b64.traffic.json")
KERNEL_SOURCES = ["paged_kv_cache_112_amd/csrc/decode_mfma.hip", "paged_kv_cache_112_amd/csrc/common.hpp",
                  "paged_kv_cache_112_amd/csrc/mfma_tiles.hpp", "paged_kv_cache_112_amd/csrc/launch.hpp",
                  "paged_kv_cache_112_amd/csrc/merge_rows.hpp", "paged_kv_cache_112_amd/csrc/merge.hip"]


def algorithmic_bytes(w, kv_bytes=2, q_bytes=2, out_bytes=2, in_bytes=2):
    """Bytes the method itself must move (no partials, no re-reads).

    decode: every context token's K and V row for every KV head, the q rows
    in, the out rows out, one int32 table entry per block read and one int32
    context length per sequence.  write: each new row in and out, plus its slot.
    """
    ctx = w.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * w.num_kv_heads * w.head_dim * 2 * kv_bytes
    q = w.num_seqs * w.num_q_heads * w.head_dim * q_bytes
    out = w.num_seqs * w.num_q_heads * w.head_dim * out_bytes
    tables = 4 * int(((ctx + w.block_size - 1) // w.block_size).sum()) + 4 * w.num_seqs
    rows = w.num_seqs * w.num_kv_heads * w.head_dim * 2 * (in_bytes + kv_bytes)
    write = rows + 4 * w.num_seqs
    return {"partition": kv + q + tables, "partition_append": kv + q + tables + rows, "decode": kv + q + out + tables,
            "write": write, "step": kv + q + out + tables + write, "kv": kv}


def kernel_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per pa_decode launch from the committed rocprofv3 counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(w):
    """The oracle, as it stands, on the same decode workload (all 64 sequences): once with every
    host core its BLAS may use, once on one core; median of a few runs each (about 10-20 s)."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    from workloads import f32_to_bf16_bits

    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kc = np.full(shape, 0x7FC0, dtype=np.uint16)
    vc = np.full(shape, 0x7FC0, dtype=np.uint16)
    for b in range(w.num_seqs):
        pos = w.owned_positions(b)
        oracle.write_kv(kc, vc, f32_to_bf16_bits(w.seq_token_values("k", b)),
                        f32_to_bf16_bits(w.seq_token_values("v", b)), w.slots(b, pos), "bf16", "bf16")
    q = f32_to_bf16_bits(w.q_values())
    nbytes = algorithmic_bytes(w)["decode"]
    cores = _host_cores()

    def timed(limit):
        times = []
        with threadpool_limits(limits=limit):
            used = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
            deadline = time.perf_counter() + 10.0
            while len(times) < 3 or (time.perf_counter() < deadline and len(times) < 10):
                t0 = time.perf_counter()
                oracle.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale, "bf16", "bf16")
                times.append(time.perf_counter() - t0)
        t = statistics.median(times)
        return t, used, len(times)

    t_all, used_all, n_all = timed(cores)
    t_one, _, n_one = timed(1)
    return {"value": round(nbytes / t_all / 1e9, 4), "unit": "GB/s", "cores": used_all, "kind": "oracle",
            "tokens_per_s": round(w.num_seqs / t_all, 2), "seconds_per_decode": round(t_all, 4),
            "one_core": {"value": round(nbytes / t_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "tokens_per_s": round(w.num_seqs / t_one, 2), "seconds_per_decode": round(t_one, 4)},
            "nproc": cores, "cpu_model": _cpu_model(),
            "sample": f"full {WORKLOAD} decode (64 sequences, sum ctx {w.total_tokens}), fp64 numpy oracle; "
                      f"BLAS threads limited to the host's {cores} cores (median of {n_all} runs) and to one "
                      f"(median of {n_one})"}


def _time_launches(torch, fn, reps, warmup):
    """Average microseconds per call of fn() launched back to back, HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


# A plain streaming read, the practical ceiling the decode's HBM figure is set against:
# each thread reads 16 bytes per step of a grid-stride loop and XOR-folds them into one
# word it stores.  Built with hipcc when --op stream_read asks for it (not part of the
# library, not in the default run).
STREAM_READ_SRC = r"""
#include <hip/hip_runtime.h>
#include <stdint.h>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t x = 0;
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}
extern "C" int stream_read_launch(const void* p, size_t bytes, void* out, int grid, void* stream) {
  hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)p, bytes / 16,
                     (uint32_t*)out);
  return (int)hipGetLastError();
}
"""


def bench_stream_read(args, torch):
    """Best GB/s of a plain streaming read over the decode's byte count and over 2 GiB."""
    import ctypes
    import subprocess
    import tempfile
    from paged_kv_cache_112_amd.build import ARCH, hipcc
    tmp = tempfile.mkdtemp(prefix="pa_stream_read_")
    src, lib = os.path.join(tmp, "stream_read.hip"), os.path.join(tmp, "stream_read.so")
    with open(src, "w") as f:
        f.write(STREAM_READ_SRC)
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-O3", "-shared", "-fPIC", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-o", lib, src], check=True, capture_output=True)
    L = ctypes.CDLL(lib)
    L.stream_read_launch.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    from workloads import make_config
    w = make_config(WORKLOAD)
    decode_bytes = algorithmic_bytes(w)["partition"] // 16 * 16
    decode_bytes_1b = algorithmic_bytes(w, kv_bytes=1)["partition"] // 16 * 16     # one-byte pools
    buf = torch.ones((2 << 30) // 4, dtype=torch.int32, device=dev)
    grids = (512, 1024, 2048, 4096)
    out = torch.empty(max(grids) * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    results = []
    total = buf.numel() * 4
    for nbytes in (decode_bytes, decode_bytes_1b, 2 << 30):
        # successive launches read successive disjoint windows of the 2 GiB buffer, as the
        # decode bench reads a different layer's pools each step, so the MALL cannot serve them
        windows = total // nbytes
        turn = [0]

        def launch(grid):
            off = (turn[0] % windows) * nbytes
            turn[0] += 1
            L.stream_read_launch(buf.data_ptr() + off, nbytes, out.data_ptr(), grid, stream)

        best = None
        for grid in grids:
            us = _time_launches(torch, lambda: launch(grid), max(args.steps, 10), max(args.warmup, 3))
            gbs = nbytes / us / 1e3
            if best is None or gbs > best[1]:
                best = (grid, gbs, us)
        results.append({"bytes": nbytes, "windows": windows, "best_grid": best[0], "us": round(best[2], 2),
                        "GB/s": round(best[1], 1),
                        "frac_of_8TBps": round(best[1] / 8000.0, 4)})
    # a plain device-to-device copy of 1 GiB (read + write), the reference for the copy-shaped operations
    src = buf.view(torch.uint8)[: 1 << 30]
    dst = torch.empty_like(src)
    us = _time_launches(torch, lambda: dst.copy_(src), max(args.steps, 10), max(args.warmup, 3))
    copy = {"bytes_read_and_written": 2 << 30, "us": round(us, 2), "GB/s": round((2 << 30) / us / 1e3, 1),
            "frac_of_8TBps": round((2 << 30) / us / 1e3 / 8000.0, 4)}
    print(json.dumps({"metric": "plain streaming read (reference ceiling for the decode's HBM figure)",
                      "results": results, "torch_copy_1GiB": copy,
                      "timing": "HIP events around back-to-back launches, best of grids " + str(list(grids))}))


def side_op(args, w, torch, pa):
    """One JSON line for a measurement beside the headline step (not the default bench line)."""
    dev = torch.device("cuda:0")
    fp8 = w.kv_dtype == "e4m3"
    kv_dtype = torch.uint8 if fp8 else torch.bfloat16
    esz = 1 if fp8 else 2
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    block_bytes = w.block_size * w.num_kv_heads * w.head_dim * esz
    reps, warm = max(args.steps, 10), max(args.warmup, 3)
    if args.op == "copy_blocks":
        # LAYERS pool pairs, used in turn, so the 256 MB MALL cannot serve a block copied by
        # an earlier call
        pools = [(torch.randint(0, 255, shape, dtype=torch.uint8, device=dev).view(kv_dtype),
                  torch.randint(0, 255, shape, dtype=torch.uint8, device=dev).view(kv_dtype))
                 for _ in range(LAYERS)]
        rng = np.random.default_rng(5)
        perm = rng.permutation(w.num_blocks).astype(np.int32)
        half = w.num_blocks // 2
        lines = []
        turn = [0]

        def call(src, dst):
            kc, vc = pools[turn[0] % LAYERS]
            turn[0] += 1
            pa.copy_blocks(kc, vc, src, dst)

        # bulk: half the pool copied onto the other half; step-sized: one block per sequence
        for n in (half, w.num_seqs):
            src = torch.from_numpy(perm[:n].copy()).to(dev)
            dst = torch.from_numpy(perm[half:half + n].copy()).to(dev)
            us = _time_launches(torch, lambda: call(src, dst), reps, warm)
            nbytes = 2 * 2 * n * block_bytes                  # K and V, read and written
            gbs = nbytes / us / 1e3
            line = {"pairs": n, "us_per_call": round(us, 2), "bytes": nbytes, "GB/s": round(gbs, 1),
                    "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4)}
            if nbytes // 2 < 2 * MALL_BYTES:
                # the written blocks land in the memory-side cache and are drained to HBM while
                # later calls run: the time is mostly the reads'
                line["note"] = (f"writes {nbytes // 2 / 1e6:.0f} MB per call, which the 256 MB MALL absorbs "
                                "between back-to-back calls: not an HBM rate")
            lines.append(line)
        print(json.dumps({"metric": "pa_copy_blocks (copy-on-write block copies)", "workload": w.name,
                          "block_bytes": block_bytes, "dtype": w.kv_dtype, "results": lines,
                          "timing": "HIP events around back-to-back calls"}))
        return
    # write_prefill: every context token of the batch through pa_write_kv in one call
    kc = torch.zeros(shape, dtype=kv_dtype, device=dev)
    vc = torch.zeros(shape, dtype=kv_dtype, device=dev)
    slots = np.concatenate([w.slots(b, w.owned_positions(b)) for b in range(w.num_seqs)]).astype(np.int32)
    n = len(slots)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    k = torch.randn((n, w.num_kv_heads, w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((n, w.num_kv_heads, w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
    sl = torch.from_numpy(slots).to(dev)
    ks = float(np.float32(4.8 / 448)) if fp8 else 1.0
    us = _time_launches(torch, lambda: pa.write_kv(k, v, sl, kc, vc, ks, ks), reps, warm)
    nbytes = n * w.num_kv_heads * w.head_dim * 2 * (2 + esz) + 4 * n
    gbs = nbytes / us / 1e3
    print(json.dumps({"metric": "pa_write_kv, prefill-shaped (every context token in one call)",
                      "workload": w.name, "tokens": n, "us_per_call": round(us, 2), "bytes": nbytes,
                      "GB/s": round(gbs, 1), "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4),
                      "timing": "HIP events around back-to-back calls"}))


def bench_attention(args, torch, pa):
    """pa_paged_attention on llama3_8b_chunk512: the last 512-token chunk of 32 sequences."""
    from workloads import make_mq_config
    w = make_mq_config("llama3_8b_chunk512")
    dev = torch.device("cuda:0")
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    kvd = args.kv_dtype or "bf16"
    esz = 1 if kvd in ("e4m3", "i8") else 2
    k_scale = v_scale = 1.0

    def pool():
        x = torch.randn(shape, generator=gen, device=dev)
        if kvd == "bf16":
            return x.to(torch.bfloat16)
        # random codes of the one-byte format: e4m3 codes with the NaN patterns cleared, int8 in [-127, 127]
        if kvd == "e4m3":
            c = torch.randint(0, 256, shape, generator=gen, device=dev, dtype=torch.int32)
            c = torch.where((c & 0x7F) == 0x7F, c - 1, c)
            return c.to(torch.uint8)
        return torch.randint(-127, 128, shape, generator=gen, device=dev, dtype=torch.int32).to(torch.int8)

    if kvd in ("e4m3", "i8"):
        k_scale = v_scale = 0.01
    pools = [(pool(), pool()) for _ in range(LAYERS)]
    qsl = w.query_start_loc()
    n = int(qsl[-1])
    q = torch.randn((n, w.num_q_heads, w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(w.context_lens).to(dev)
    qs = torch.from_numpy(qsl).to(dev)
    maxq = int(w.query_lens.max())
    turn = [0]

    def call():
        kc, vc = pools[turn[0] % LAYERS]
        turn[0] += 1
        pa.paged_attention(q, kc, vc, bt, sl, qs, w.scale, maxq, out=out, k_scale=k_scale, v_scale=v_scale)

    us = _time_launches(torch, call, max(args.steps, 10), max(args.warmup, 3))
    # causal work actually needed: new token j of sequence b sees p + 1 keys, p = S - n + j
    keys = sum(int(S) * int(nq) - int(nq) * (int(nq) - 1) // 2 for S, nq in zip(w.context_lens, w.query_lens))
    flops = 4 * w.head_dim * w.num_q_heads * keys
    kv_bytes = int(w.context_lens.sum()) * w.num_kv_heads * w.head_dim * 2 * esz
    qo_bytes = 2 * n * w.num_q_heads * w.head_dim * 2
    tflops = flops / us / 1e6
    print(json.dumps({"metric": "pa_paged_attention (multi-query, causal), llama3_8b_chunk512",
                      "workload": w.name, "kv_dtype": kvd, "new_tokens": n, "us_per_call": round(us, 2),
                      "TFLOP/s": round(tflops, 1), "frac_of_bf16_mfma_2.5PF": round(tflops / 2500.0, 4),
                      "unique_kv_and_qo_bytes": kv_bytes + qo_bytes,
                      "GB/s_unique": round((kv_bytes + qo_bytes) / us / 1e3, 1),
                      "timing": "HIP events around back-to-back calls, 8 pool copies in turn"}))


def bench_graph_loop(args, torch, pa):
    """The batch-64 decode loop with no host work per step: pa_slot_mapping (advancing the
    lengths) -> pa_write_kv -> pa_decode, captured once per layer and replayed; each replay is
    one more token for every sequence, on the next of 8 layer pools."""
    from workloads import deal_tables, make_config
    w = make_config(WORKLOAD)
    dev = torch.device("cuda:0")
    steps = max(args.steps, 8) // LAYERS * LAYERS
    warm = max(args.warmup, 1)
    B, hq, hkv, d, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    reps = steps // LAYERS
    # every replay of the graph (warmup included) is one model step: one more token per sequence
    room = warm + reps + 2
    final = w.context_lens + room
    need = int(sum(-(-int(c) // bs) for c in final))
    nb = int(np.ceil(1.1 * need))
    bt, _ = deal_tables(final, bs, np.random.default_rng(12).permutation(nb).astype(np.int32))
    shape = (nb, bs, hkv, d)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    pools = [(torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16),
              torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)) for _ in range(LAYERS)]
    dbt = torch.from_numpy(bt).to(dev)
    ctx = torch.from_numpy((w.context_lens - 1).astype(np.int32)).to(dev)   # each replay of layer 0 advances
    slots = torch.zeros(B, dtype=torch.int32, device=dev)
    knew = torch.randn((B, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    vnew = torch.randn((B, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    q = torch.randn((B, hq, d), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
    max_ctx = int(final.max())
    ws = pa.new_workspace(B, hq, d, max_ctx, 0, dev)

    def model_step():
        # one token for the whole model: the lengths advance once, every layer writes and decodes
        # (--fused: the write done by the decode's partition launch)
        pa.slot_mapping(dbt, ctx, bs, slots, advance=True)
        for kc, vc in pools:
            if args.fused:
                pa.decode_append(q, knew, vnew, kc, vc, dbt, ctx, w.scale, out=out, max_context_len=max_ctx,
                                 workspace=ws)
            else:
                pa.write_kv(knew, vnew, slots, kc, vc)
                pa.decode(q, kc, vc, dbt, ctx, w.scale, out=out, max_context_len=max_ctx, workspace=ws)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        model_step()
    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        graph.replay()
    e1.record(s)
    torch.cuda.synchronize()
    us_layer = e0.elapsed_time(e1) * 1e3 / (reps * LAYERS)
    # the tables were sized for the growth: no length may have passed them
    grown = ctx.cpu().numpy()
    if not (grown == w.context_lens - 1 + warm + reps).all() or (grown > final).any():
        raise SystemExit("graph loop: context lengths outgrew the block tables")
    print(json.dumps({"metric": "device-side decode loop (slot mapping + write + decode per layer, graph replay)",
                      "workload": WORKLOAD, "fused_write": bool(args.fused), "layers_per_graph": LAYERS,
                      "model_steps": reps,
                      "us_per_layer_step": round(us_layer, 2),
                      "decode_tokens_per_s_per_layer": round(B / us_layer * 1e6, 1),
                      "note": "lengths grow by one token per replay; tables pre-filled for the growth"}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = library default)")
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 vector path, 2 matrix-core")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-contiguous", action="store_true", help="skip the identity-table comparator")
    ap.add_argument("--two-launch", action="store_true",
                    help="decode as pa_decode_partition + pa_merge (two launches) instead of pa_decode")
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=["llama3_8b_b64", "llama3_8b_long", "llama2_7b_mha", "llama3_8b_fp8_prefix"])
    ap.add_argument("--block-size", type=int, default=None, help="block size for llama2_7b_mha")
    ap.add_argument("--tp", type=int, default=1, metavar="N",
                    help="one rank's share of the layer under N-way tensor parallelism over KV heads "
                         "(H_q / N query and H_kv / N KV heads, the same sequences and tables)")
    ap.add_argument("--kv-dtype", default=None, choices=["bf16", "e4m3", "i8"],
                    help="pool format other than the workload's own (same lengths and tables)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB with torch (a plain copy of known size, for counter scaling)")
    ap.add_argument("--op", default="decode",
                    choices=["decode", "copy_blocks", "write_prefill", "attention", "graph_loop", "stream_read"],
                    help="decode: the hot-path step (the headline line); copy_blocks: copy-on-write block "
                         "copies over the workload's pools; write_prefill: pa_write_kv of every context token; "
                         "attention: multi-query paged attention on llama3_8b_chunk512; graph_loop: the decode "
                         "loop with device-side slot mapping, captured once and replayed; stream_read: a plain "
                         "streaming read of the same byte count, the practical HBM ceiling")
    ap.add_argument("--fused", action="store_true",
                    help="the step's write done by the decode launch itself (pa_decode_append) instead of "
                         "pa_write_kv + pa_decode")
    ap.add_argument("--contiguous", action="store_true",
                    help="identity-ordered block tables (each sequence's blocks adjacent): the contiguous comparator")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the paged-KV path here is "
              "single-GPU, see the design notes for how it would shard.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_112_amd as pa
    from workloads import f32_to_bf16_bits, make_config

    if args.copy_calibrate:
        n = args.copy_calibrate << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}))
        return

    if not os.path.exists(pa.LIB_PATH):
        from paged_kv_cache_112_amd.build import build
        build()
    if args.op == "attention":
        return bench_attention(args, torch, pa)
    if args.op == "stream_read":
        return bench_stream_read(args, torch)
    if args.op == "graph_loop":
        return bench_graph_loop(args, torch, pa)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = make_config(args.workload, args.block_size) if args.workload == "llama2_7b_mha" else make_config(args.workload)
    if args.kv_dtype and args.kv_dtype != w.kv_dtype:
        w = w.with_dtypes(args.kv_dtype, "bf16", name=f"{w.name}-{args.kv_dtype}")
    if args.tp > 1:
        if w.num_kv_heads % args.tp:
            raise SystemExit(f"--tp {args.tp} does not divide the {w.num_kv_heads} KV heads")
        from dataclasses import replace
        w = replace(w, num_q_heads=w.num_q_heads // args.tp, num_kv_heads=w.num_kv_heads // args.tp,
                    name=f"{w.name}-tp{args.tp}-rank")
    if args.contiguous:
        from workloads import deal_tables
        w.block_tables, _ = deal_tables(w.context_lens, w.block_size, np.arange(w.num_blocks, dtype=np.int32))
    B, hq, hkv, d, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    if args.op != "decode":
        return side_op(args, w, torch, pa)

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # ---- inputs resident in HBM: pools filled with every token but this step's ---------------
    # Values are seeded N(0,1) drawn on the device (bf16), written through pa_write_kv.
    fp8 = w.kv_dtype in ("e4m3", "i8")              # one-byte pools
    kv_dtype = {"e4m3": torch.uint8, "i8": torch.int8}.get(w.kv_dtype, torch.bfloat16)
    qmax = 448.0 if w.kv_dtype == "e4m3" else 127.0
    k_scale, v_scale = (float(np.float32(4.8 / qmax)), float(np.float32(4.8 / qmax))) if fp8 else (1.0, 1.0)
    shape = (w.num_blocks, bs, hkv, d)

    def fill_pools(tables):
        """LAYERS copies of the pools, [LAYERS, num_blocks, bs, H_kv, d] per K and V, holding every
        context token but this step's at the slots ``tables`` give; the same values for any tables."""
        k0 = torch.zeros(shape, dtype=kv_dtype, device=dev)
        v0 = torch.zeros(shape, dtype=kv_dtype, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed)
        for b in range(B):
            pos = w.owned_positions(b)[:-1]
            if len(pos) == 0:
                continue
            K = torch.randn((len(pos), hkv, d), generator=gen, device=dev).to(torch.bfloat16)
            V = torch.randn((len(pos), hkv, d), generator=gen, device=dev).to(torch.bfloat16)
            sl = (tables[b, pos // bs].astype(np.int64) * bs + pos % bs).astype(np.int32)
            pa.write_kv(K, V, to_dev(sl), k0, v0, k_scale, v_scale)
        k_all = k0.unsqueeze(0).repeat(LAYERS, 1, 1, 1, 1)
        v_all = v0.unsqueeze(0).repeat(LAYERS, 1, 1, 1, 1)
        del k0, v0
        return k_all, v_all

    k_all, v_all = fill_pools(w.block_tables)
    pools = [(k_all[l], v_all[l]) for l in range(LAYERS)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 1)
    k_new = torch.randn((B, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    v_new = torch.randn((B, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    slots = to_dev(w.append_slots())
    q = torch.randn((B, hq, d), generator=gen, device=dev).to(torch.bfloat16)
    bt = to_dev(w.block_tables)
    ctx = to_dev(w.context_lens)
    max_ctx = int(w.context_lens.max())
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
    # the partition size pa_decode takes by itself on the matrix cores (passed explicitly,
    # so that the two-launch and partition-only figures use the same one)
    P = args.partition or (pa.pa_default_partition_tokens() if args.kernel == pa.PA_KERNEL_VALU
                           else pa.pa_partition_tokens_for(max_ctx))
    ws = pa.new_workspace(B, hq, d, max_ctx, P, dev)
    if ws is None:
        ws = torch.empty(1, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    # --fused: the step's write is done by the decode launch itself (matrix-core grid kernel,
    # partitions of 256 tokens or more)
    fused = args.fused and args.kernel in (0, 2) and P >= 256 and w.kv_dtype != "f32"

    def decode(kc, vc, tables=bt):
        if fused:
            pa.decode_append(q, k_new, v_new, kc, vc, tables, ctx, w.scale, out=out, max_context_len=max_ctx,
                             workspace=ws, partition_tokens=P, k_scale=k_scale, v_scale=v_scale)
        elif args.two_launch:
            pa.decode_partition(q, kc, vc, tables, ctx, w.scale, out=out, max_context_len=max_ctx, workspace=ws,
                                partition_tokens=P, kernel=args.kernel, k_scale=k_scale, v_scale=v_scale)
            pa.merge(ws, ctx, out, max_ctx, P)
        else:
            pa.decode(q, kc, vc, tables, ctx, w.scale, out=out, max_context_len=max_ctx, workspace=ws,
                      partition_tokens=P, kernel=args.kernel, k_scale=k_scale, v_scale=v_scale)

    def step(i):
        kc, vc = pools[i % LAYERS]
        if not fused:
            pa.write_kv(k_new, v_new, slots, kc, vc, k_scale, v_scale)
        decode(kc, vc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    eager_out = out.clone()                      # result of step warmup-1 (every layer holds the same data)

    # ---- HIP graphs: one per layer's step, and one of all LAYERS steps in order (as a model's
    # forward pass would replay them); replays cost no per-kernel host work --------------------
    side = torch.cuda.Stream()
    side.wait_stream(stream)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                fn()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        return g

    graphs = [capture(lambda i=i: step(i)) for i in range(LAYERS)]
    all_layers = capture(lambda: [step(i) for i in range(LAYERS)])
    for i, g in enumerate(graphs + [all_layers]):   # every replay must reproduce the eager result exactly
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out.view(torch.int16), eager_out.view(torch.int16)):
            raise SystemExit(f"graph replay {i} differs from the eager step")

    # ---- timed region: exactly K steps ----------------------------------------------------------
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps // LAYERS):
        all_layers.replay()
    for i in range(args.steps % LAYERS):
        graphs[i].replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # ---- the step's distribution: each replay of the 8-layer graph between its own two events
    # (per step = replay / 8; a pair of events per single step would add its own overhead) ------
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(2, args.steps // LAYERS))]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        all_layers.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    per_step_us = sorted(e0.elapsed_time(e1) * 1e3 / LAYERS for e0, e1 in evs)

    def pct(xs, p):
        return round(float(np.percentile(np.asarray(xs), p)), 2)

    # ---- pa_decode alone (partition + merge, the dominant launch): back-to-back graph replays ---
    def time_decode(tables, layer_pools, fn=None):
        fn = fn or decode
        g = capture(lambda: [fn(*layer_pools[i], tables) for i in range(LAYERS)])
        g.replay()
        torch.cuda.synchronize()
        reps = max(2, args.steps // LAYERS)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        # per-replay spread: each replay of 8 launches between its own events
        spread = []
        for _ in range(reps):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            g.replay()
            a1.record(stream)
            spread.append((a0, a1))
        torch.cuda.synchronize()
        per = sorted(a0.elapsed_time(a1) * 1e3 / LAYERS for a0, a1 in spread)
        return e0.elapsed_time(e1) * 1e3 / (reps * LAYERS), per

    decode_us, decode_spread = time_decode(bt, pools)

    # the partition stage alone (pa_decode_partition), as earlier figures quoted it
    def partition_only(kc, vc, tables=bt):
        pa.decode_partition(q, kc, vc, tables, ctx, w.scale, out=out, max_context_len=max_ctx, workspace=ws,
                            partition_tokens=P, kernel=args.kernel, k_scale=k_scale, v_scale=v_scale)

    part_us, _ = time_decode(bt, pools, partition_only)

    nb = algorithmic_bytes(w, kv_bytes=1 if fp8 else 2)
    value = nb["step"] / (ms_per_step * 1e-3) / 1e9
    launch_bytes = nb["step"] if fused else nb["decode"]
    achieved = launch_bytes / (decode_us * 1e-6) / 1e9
    # the committed counter run covers the default launch of the headline workload only
    default_launch = (w.name == WORKLOAD and P == 256 and args.kernel in (0, 2) and not args.contiguous and not fused)
    traffic = measured_traffic() if default_launch else None

    # ---- the contiguous comparator: the same tokens and lengths, each sequence's blocks adjacent
    contiguous = None
    if not args.no_contiguous:
        from workloads import deal_tables
        ident, _ = deal_tables(w.context_lens, bs, np.arange(w.num_blocks, dtype=np.int32))
        del pools
        k_all = v_all = None
        torch.cuda.synchronize()
        ck_all, cv_all = fill_pools(ident)
        cpools = [(ck_all[l], cv_all[l]) for l in range(LAYERS)]
        bt_ident = to_dev(ident)
        c_us, c_spread = time_decode(bt_ident, cpools)
        contiguous = {"block_order": "identity (each sequence's blocks adjacent, in order)",
                      "decode_us": round(c_us, 2), "GB/s": round(launch_bytes / (c_us * 1e-6) / 1e9, 1),
                      "frac": round(launch_bytes / (c_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "decode_us_median": pct(c_spread, 50),
                      "paged_over_contiguous_time": round(decode_us / c_us, 4)}
        del cpools, ck_all, cv_all

    result = {
        "metric": "paged-attn decode achieved HBM GB/s + tokens/s, Llama-3-8B layer, batch 64",
        "value": round(value, 2),
        "unit": "GB/s",
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "kv_tokens_per_s": round(w.total_tokens / (ms_per_step * 1e-3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "step_us_median": pct(per_step_us, 50), "step_us_p10": pct(per_step_us, 10),
        "step_us_p90": pct(per_step_us, 90),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"bf16 q / {w.kv_dtype} kv" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
                   "block_size": bs, "sum_context": w.total_tokens, "max_context": max_ctx,
                   "partition_tokens": P, "kernel": ["auto", "valu", "mfma"][args.kernel],
                   "layer_pools_rotated": LAYERS,
                   "step": ("pa_decode_append (writes the 64 new tokens, decodes, merges)" if fused
                            else "pa_write_kv(64 tokens) + pa_decode_partition + pa_merge" if args.two_launch
                            else "pa_write_kv(64 tokens) + pa_decode"),
                   "block_order": "identity (contiguous comparator)" if args.contiguous else "seeded permutation"},
        "decode_partition": {"us": round(part_us, 2),
                             "GB/s": round(nb["partition"] / (part_us * 1e-6) / 1e9, 1),
                             "frac": round(nb["partition"] / (part_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "pa_decode": {"us": round(decode_us, 2), "us_median": pct(decode_spread, 50),
                      "us_p10": pct(decode_spread, 10), "us_p90": pct(decode_spread, 90),
                      "GB/s": round(achieved, 1), "tokens_per_s": round(B / (decode_us * 1e-6), 1),
                      "kv_tokens_per_s": round(w.total_tokens / (decode_us * 1e-6), 1)},
        "timing": "value/ms_per_step: K steps replayed from HIP graphs of the 8 layer steps between two events; "
                  "step_us_*: percentiles over replays of the 8-step graph, each between its own events, per "
                  "step; pa_decode: back-to-back replays of a graph of 8 pa_decode calls (one per layer pool), "
                  "HIP events on the launch stream, percentiles per replay",
        "bytes": nb,
        "roofline": {"bound": "hbm",
                     "kernel": ("pa_decode_append: decode_mfma_kernel (write + partition stage) + merge kernel"
                                if fused else "pa_decode: decode_mfma_kernel (partition stage) + merge kernel"),
                     "bytes_per_launch": launch_bytes,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "contiguous": contiguous,
    }
    if not args.no_cpu_baseline and args.workload == WORKLOAD and not args.kv_dtype:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
