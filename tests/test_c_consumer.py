"""The C ABI from plain C, on the CPU: include/mxfa.h is a strict C99 header
and the tests' plain-C caller builds against it and the library without a
warning.  The program's argument and file checks run before any HIP call,
so they are exercised here too."""
import os
import subprocess

import pytest

import c_consumer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_is_strict_c99(tmp_path):
    """mxfa.h alone (no HIP header), in C99 with every pedantic warning as an
    error: the boundary needs nothing but a C compiler."""
    src = tmp_path / "h.c"
    src.write_text('#include "mxfa.h"\n'
                   "int main(void) { mxfa_plan_t p; (void)p; return mxfa_version() < 0; }\n")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.join(ROOT, "include"), "-c", str(src),
                        "-o", str(tmp_path / "h.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_consumer_builds_without_warnings(tmp_path):
    import split_kv_decode_amd.mxfa as mxfa
    if not os.path.exists(mxfa.LIB_PATH):
        pytest.fail("libmxfa.so is not built: run __graft_entry__.build()")
    out = c_consumer.build(str(tmp_path / "c_consumer"))
    assert os.access(out, os.X_OK)


def _env():
    # no GPU may be touched by these runs: they must stop at the argument checks
    return dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")


def test_consumer_rejects_bad_usage_and_files(tmp_path):
    exe = c_consumer.build(str(tmp_path / "c_consumer"))
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(), timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr
    bad = tmp_path / "bad.bin"
    bad.write_bytes(b"\0" * 64)
    r = subprocess.run([exe, str(bad), str(tmp_path / "o.bin")], capture_output=True, text=True,
                       env=_env(), timeout=60)
    assert r.returncode == 2 and "header" in r.stderr
