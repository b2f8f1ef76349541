"""pa_decode at the workloads' full sizes, in the launch configuration the benchmark times.

The oracle checks a sample of sequences one by one (shortest, longest and a
spread between; every query head); every output must be finite; the two GPU
paths must agree everywhere; the block-size sweep must be bitwise identical.
"""
import numpy as np
import pytest

from pools import DeviceInputs, build_host_inputs, from_dev, out_to_f64, sample_seqs
from workloads import make_config

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _parity(dev, tol, **kw):
    w = dev.h.w
    seqs = sample_seqs(w)
    print(f"decode {w.name} kv={w.kv_dtype} B={w.num_seqs} sum(ctx)={w.total_tokens} seqs={seqs} {kw}", flush=True)
    out = out_to_f64(dev.decode(**kw))
    assert np.isfinite(out).all()
    ref = dev.h.oracle_decode(seqs=seqs)
    err = float(np.abs(out[seqs] - ref[seqs]).max())
    print(f"  max abs err {err:.3e}", flush=True)
    assert err <= tol
    return out


@pytest.fixture(scope="module")
def llama3_b64():
    return DeviceInputs(build_host_inputs(make_config("llama3_8b_b64")))


def test_llama3_b64_default_launch(llama3_b64):
    _parity(llama3_b64, 2e-2)


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


def test_llama3_long_context():
    _parity(DeviceInputs(build_host_inputs(make_config("llama3_8b_long"))), 2e-2)


def test_llama2_mha_block_size_sweep():
    outs = []
    for bs in (1, 16, 64, 256):
        dev = DeviceInputs(build_host_inputs(make_config("llama2_7b_mha", bs)))
        _parity(dev, 2e-2)
        outs.append(from_dev(dev.decode()))
        del dev
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


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
