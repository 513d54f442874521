"""Build and drive the plain-C caller of the C ABI (``tests/c_consumer.c``).

The program is compiled with gcc in C99 mode against ``include/mxfa.h``,
the HIP runtime and ``libmxfa.so``; no Python or torch runs in its process.
``write_problem`` and ``read_result`` speak its file formats (documented at
the top of the C source).  Test infrastructure: the library does not use it.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_consumer.c")
BIN_PATH = os.path.join(HERE, "_build", "c_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
MAGIC = 0x4146584D
PLAN_FIELDS = ("path", "layout", "schedule", "rows", "row_block", "head_block", "num_splits",
               "chunk", "grid_x", "grid_y", "grid_z", "combine", "num_cus")


def compile_command(out_path: str):
    lib_dir = os.path.join(ROOT, "split_kv_decode_amd")
    rel = os.path.relpath(lib_dir, os.path.dirname(out_path))
    return ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-pedantic", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
            SRC, "-o", out_path,
            "-L", lib_dir, "-lmxfa", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]


def build(out_path: str = BIN_PATH) -> str:
    """Compile the program (the library must be built first); the binary is
    written under a temporary name and moved into place."""
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = f"{out_path}.{os.getpid()}.tmp"
    try:
        r = subprocess.run(compile_command(tmp), capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"gcc failed for {SRC}:\n{r.stderr}")
        if r.stderr.strip():
            raise RuntimeError(f"gcc warnings for {SRC}:\n{r.stderr}")
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return out_path


def _u16(t) -> bytes:
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().tobytes()


def write_problem(path, inp, num_splits=0, paged=None):
    """Write the inputs of ``inp`` (a workloads.Inputs), contiguous or, with
    ``paged`` (a workloads.PagedCache), as pages."""
    w = inp.workload
    has_sl = paged is not None or inp.cache_seqlens is not None
    hdr = np.zeros(16, dtype=np.int32)
    hdr[:14] = [MAGIC, w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, int(w.causal),
                1 if w.dtype == "bf16" else 0, int(has_sl), num_splits,
                paged.page_size if paged is not None else 0,
                paged.block_table.shape[1] if paged is not None else 0,
                paged.k_pages.shape[0] if paged is not None else 0]
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        f.write(_u16(inp.q))
        if paged is None:
            f.write(_u16(inp.k_cache))
            f.write(_u16(inp.v_cache))
            if has_sl:
                f.write(inp.cache_seqlens.numpy().astype(np.int32).tobytes())
        else:
            f.write(_u16(paged.k_pages))
            f.write(_u16(paged.v_pages))
            f.write(paged.cache_seqlens.numpy().astype(np.int32).tobytes())
            f.write(paged.block_table.numpy().astype(np.int32).tobytes())


def read_result(path, inp):
    """(status, plan dict, workspace bytes, out float64 [B, qLen, Hq, D],
    lse float64 [B, Hq, qLen])."""
    import torch
    w = inp.workload
    raw = open(path, "rb").read()
    status = int(np.frombuffer(raw, np.int32, 1, 0)[0])
    plan = dict(zip(PLAN_FIELDS, np.frombuffer(raw, np.int32, 13, 4).tolist()))
    ws = int(np.frombuffer(raw, np.int64, 1, 56)[0])
    n_out = w.B * w.qLen * w.Hq * w.D
    bits = np.frombuffer(raw, np.int16, n_out, 64).copy()
    out = torch.from_numpy(bits).view(w.torch_dtype).float().double().numpy()
    lse = np.frombuffer(raw, np.float32, w.B * w.Hq * w.qLen, 64 + 2 * n_out).astype(np.float64)
    return (status, plan, ws, out.reshape(w.B, w.qLen, w.Hq, w.D),
            lse.reshape(w.B, w.Hq, w.qLen))


def run(problem_path, result_path, timeout=120):
    return subprocess.run([BIN_PATH, problem_path, result_path], capture_output=True, text=True,
                          timeout=timeout)
