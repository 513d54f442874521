"""The Python binding on the GPU (needs an MI355X): the order in which a
process loads the library and torch."""
import pytest

pytestmark = pytest.mark.gpu


def test_library_loaded_before_torch_keeps_the_gpu_usable():
    """A process that loads the library before anything imported torch: torch
    still sees the GPU and a call matches the oracle (one process, run as a
    child so that this one's import order does not decide it)."""
    import os
    import subprocess
    import sys
    code = (
        "import split_kv_decode_amd as mx\n"
        "mx.lib()\n"
        "import torch, sys\n"
        "sys.path.insert(0, 'tests')\n"
        "assert torch.cuda.is_available(), 'torch sees no GPU'\n"
        "import workloads as wl, parity\n"
        "w = wl.Workload('order', B=2, qLen=1, Hq=8, Hkv=2, D=128, kv_cap=500, dtype='bf16',\n"
        "                causal=False, sigma=1.0, seed=5, len_range=(1, 500))\n"
        "inp = wl.make_inputs(w)\n"
        "out, lse, plan = parity.run_gpu(inp)\n"
        "ro, rl = parity.oracle_full(inp)\n"
        "print(parity.compare(out, lse, ro, rl, 'bf16'), flush=True)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=300)
    print(r.stdout, r.stderr[-2000:], flush=True)
    assert r.returncode == 0, r.stderr[-2000:]
