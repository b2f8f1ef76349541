"""pa_decode at the workloads' full sizes, in the launch configuration the benchmark times.

Every sequence of every workload is compared with the oracle (it finishes the largest
in a few seconds).  With N(0, 1) data and contexts of thousands of tokens each token
weighs about 1/ctx, so a dropped 16-token tile can hide under the bf16 tolerance; the
peaky runs (scale 8/sqrt(d): a handful of tokens carry the softmax) and the f32
shadows (the same tables and values in f32 pools, compared at 1e-5) are the gates
that see such a slip at full size.  Each test prints its measured max-abs error.
"""
import numpy as np
import pytest

from pools import DeviceInputs, build_host_inputs, from_dev, out_to_f64
from workloads import make_config

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

PEAKY = 8 / np.sqrt(128)


def _parity(dev, tol, label="", scale=None, **kw):
    w = dev.h.w
    print(f"decode {w.name} kv={w.kv_dtype} B={w.num_seqs} sum(ctx)={w.total_tokens} scale={scale} {kw}", flush=True)
    out = out_to_f64(dev.decode(scale=scale, **kw))
    assert np.isfinite(out).all()
    ref = dev.h.oracle_decode(scale=scale)
    err = float(np.abs(out - ref).max())
    print(f"PARITY {w.name}{label} kv={w.kv_dtype} {kw} scale={'peaky' if scale else 'default'} "
          f"max_abs_err={err:.3e} max_abs_out={float(np.abs(ref).max()):.3e} tol={tol}", flush=True)
    assert err <= tol
    return out


@pytest.fixture(scope="module")
def llama3_b64():
    return DeviceInputs(build_host_inputs(make_config("llama3_8b_b64")))


def test_llama3_b64_default_launch(llama3_b64):
    _parity(llama3_b64, 2e-2)


def test_llama3_b64_peaky(llama3_b64):
    _parity(llama3_b64, 2e-2, scale=PEAKY)


def test_llama3_b64_vector_path_agrees(llama3_b64):
    a = _parity(llama3_b64, 2e-2, kernel=1)
    b = out_to_f64(llama3_b64.decode())
    assert np.abs(a - b).max() <= 2e-2


@pytest.mark.parametrize("P", [64, 128, 512, 1024])
def test_llama3_b64_other_partitions(llama3_b64, P):
    _parity(llama3_b64, 2e-2, partition_tokens=P)


def test_llama3_b64_f32_shadow():
    w = make_config("llama3_8b_b64").with_dtypes("f32", "f32")
    _parity(DeviceInputs(build_host_inputs(w)), 1e-5)


@pytest.fixture(scope="module")
def llama3_long():
    return DeviceInputs(build_host_inputs(make_config("llama3_8b_long")))


def test_llama3_long_context(llama3_long):
    _parity(llama3_long, 2e-2)


def test_llama3_long_context_peaky(llama3_long):
    _parity(llama3_long, 2e-2, scale=PEAKY)


def test_llama3_long_f32_shadow():
    w = make_config("llama3_8b_long").with_dtypes("f32", "f32")
    _parity(DeviceInputs(build_host_inputs(w)), 1e-5)


def test_llama2_mha_block_size_sweep():
    outs = []
    for bs in (1, 16, 64, 256):
        dev = DeviceInputs(build_host_inputs(make_config("llama2_7b_mha", bs)))
        _parity(dev, 2e-2, label=f"-bs{bs}")
        outs.append(from_dev(dev.decode()))
        del dev
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("bs", [1, 16, 64, 256])
def test_llama2_mha_f32_shadow(bs):
    w = make_config("llama2_7b_mha", bs).with_dtypes("f32", "f32")
    _parity(DeviceInputs(build_host_inputs(w)), 1e-5, label=f"-bs{bs}")


def test_llama2_mha_peaky():
    _parity(DeviceInputs(build_host_inputs(make_config("llama2_7b_mha", 16))), 2e-2, label="-bs16", scale=PEAKY)


def test_llama3_fp8_shared_prefix():
    w = make_config("llama3_8b_fp8_prefix")
    dev = DeviceInputs(build_host_inputs(w))
    out = _parity(dev, 2e-2)
    a = out_to_f64(dev.decode(kernel=1))
    assert np.abs(a - out).max() <= 2e-2


def test_llama3_b64_int8_pool():
    """The batch-64 workload with int8 pools (symmetric, per-pool scale amax / 127)."""
    w = make_config("llama3_8b_b64").with_dtypes("i8", "bf16")
    _parity(DeviceInputs(build_host_inputs(w)), 2e-2)


def test_llama3_b64_e4m3_pool():
    """The batch-64 workload with e4m3 pools (per-pool scale amax / 448)."""
    w = make_config("llama3_8b_b64").with_dtypes("e4m3", "bf16")
    _parity(DeviceInputs(build_host_inputs(w)), 2e-2)
