"""pa_decode_noalloc (static scratch, no allocation) against pa_decode with a caller workspace.

Both run the same kernels on the same inputs, so the outputs must be identical bit for bit;
two calls in a row, the second on a smaller input, check that the shared static array keeps
nothing from one call that the next depends on.
The shape that needs more scratch than the array holds is refused before any launch.
"""
import ctypes

import numpy as np
import pytest

from pools import DeviceInputs, build_host_inputs, custom_workload, from_dev, out_to_f64
from workloads import make_config

pytestmark = pytest.mark.gpu


def _noalloc(dev, partition_tokens=0, kernel=0, out=None):
    """pa_decode_noalloc through the C ABI (ctypes), on the current stream."""
    import torch
    import paged_kv_cache_112_amd as pa
    h, w = dev.h, dev.h.w
    out = torch.empty_like(dev.q) if out is None else out
    desc = pa.cache_desc(dev.kc, h.k_scale, h.v_scale)
    st = pa.lib().pa_decode_noalloc(dev.q.data_ptr(), pa.dtype_code(dev.q), w.num_seqs, w.num_q_heads,
                                    dev.kc.data_ptr(), dev.vc.data_ptr(), ctypes.byref(desc), dev.bt.data_ptr(),
                                    w.max_blocks_per_seq, dev.ctx.data_ptr(), dev.max_ctx, ctypes.c_float(w.scale),
                                    out.data_ptr(), partition_tokens, kernel,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st, out


def _compare(dev, label, **kw):
    import paged_kv_cache_112_amd as pa
    print(f"no-alloc decode {label} {kw}", flush=True)
    st, got = _noalloc(dev, **kw)
    assert st == pa.PA_OK, pa.status_str(st)
    want = dev.decode(**kw)
    assert np.array_equal(from_dev(got), from_dev(want)), label
    err = float(np.abs(out_to_f64(got) - dev.h.oracle_decode()).max())
    tol = 1e-5 if dev.h.w.kv_dtype == "f32" else 2e-2
    print(f"  bitwise equal to pa_decode; max abs err vs oracle {err:.3e}", flush=True)
    assert err <= tol


def test_two_calls_second_smaller():
    """The batch-64 Llama-3-8B decode (the merge inside the partition launch), then a smaller
    batch with other lengths and partitions: each equals pa_decode with a workspace."""
    big = DeviceInputs(build_host_inputs(make_config("llama3_8b_b64")))
    _compare(big, "llama3_8b_b64")
    del big
    small = DeviceInputs(build_host_inputs(custom_workload([700, 1, 16, 300, 0, 257], 32, 8, 128, 16, "bf16",
                                                            "bf16", seed=61)))
    _compare(small, "6 sequences, P=64", partition_tokens=64)
    _compare(small, "6 sequences, P=512 (merge kernel)", partition_tokens=512)
    tiny = DeviceInputs(build_host_inputs(make_config("tiny_f32")))
    _compare(tiny, "tiny_f32 (vector path)", partition_tokens=32)


def test_too_large_is_refused_before_launch():
    """A shape whose pieces exceed the static array: PA_ERR_SCRATCH, output untouched."""
    import torch
    import paged_kv_cache_112_amd as pa
    w = custom_workload([16, 16], 32, 8, 128, 16, "bf16", "bf16", seed=63)
    dev = DeviceInputs(build_host_inputs(w))
    dev.max_ctx = 2 ** 20                      # only sizes the launch; the call is refused first
    bt = torch.zeros((2, 2 ** 20 // 16), dtype=torch.int32, device="cuda")
    dev.bt = bt
    w.block_tables = np.zeros((2, 2 ** 20 // 16), dtype=np.int32)
    out = torch.full_like(dev.q, 7.0)
    st, got = _noalloc(dev, partition_tokens=16, out=out)
    assert st == pa.PA_ERR_SCRATCH
    assert (got.float() == 7.0).all()
