"""The binding shares torch's HIP runtime with the library, whatever is called first.

torch ships its own HIP runtime and asks for it by the file name libamdhip64.so; the library
asks for libamdhip64.so.7.  If the library were loaded before torch, the process would map two
runtimes, and kernels launched through one on memory and streams of the other fail.  Runs on
the CPU: it only inspects which runtime files a fresh process has mapped.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = """
import paged_kv_cache_112_amd as pa
pa.pa_partition_tokens_for(4096)          # host-only call: loads the library first
import torch
maps = set()
for line in open('/proc/self/maps'):
    path = line.split()[-1]
    if 'libamdhip64' in path:
        maps.add(os.path.realpath(path))
print(len(maps), sorted(maps))
"""


def test_one_hip_runtime_when_the_library_is_loaded_before_torch():
    r = subprocess.run([sys.executable, "-c", "import os\n" + SCRIPT], cwd=ROOT, capture_output=True, text=True,
                       timeout=300, env={**os.environ, "PYTHONPATH": ROOT})
    assert r.returncode == 0, r.stderr[-2000:]
    count = int(r.stdout.split()[0])
    assert count == 1, r.stdout


class _FakeDeviceTensor:
    """Stands in for a contiguous device tensor on another GPU (none exists on this host)."""

    is_cuda = True

    def __init__(self, index):
        import types
        self.device = types.SimpleNamespace(index=index)

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return 0x1000


def test_tensor_on_another_device_is_refused(monkeypatch):
    import pytest
    import torch
    from paged_kv_cache_112_amd import _binding
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    assert _binding._ptr(_FakeDeviceTensor(0)) == 0x1000
    with pytest.raises(ValueError, match="current device"):
        _binding._ptr(_FakeDeviceTensor(1))
