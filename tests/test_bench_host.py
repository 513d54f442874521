"""Host logic of bench.py that needs no GPU: the source digest that keeps the
recorded counter traffic tied to the code it was measured on, the profile
summary's counter arithmetic, and the one-GPU guard."""
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


SRC = """// a line comment
#include "x.h"   /* trailing */
int f(int a) {
    const char *s = "// not a comment /* either */";
    char q = '"';   // a quote in a char literal
    return a  +  1;  /* multi
                        line */
}
"""


def test_code_text_drops_comments_and_layout_only():
    t = bench.code_text(SRC)
    assert "comment" not in t.replace('"// not a comment /* either */"', "")
    assert '"// not a comment /* either */"' in t       # literals kept whole
    assert "char q = '\"';" in t
    assert "return a + 1;" in t
    assert "\n\n" not in t


def test_comment_edits_keep_the_digest_and_code_edits_change_it():
    base = bench.code_text(SRC)
    reworded = SRC.replace("// a line comment", "// another comment\n\n// and one more")
    relaid = SRC.replace("return a  +  1;", "return a + 1;")
    assert bench.code_text(reworded) == base
    assert bench.code_text(relaid) == base
    for edit in (SRC.replace("a  +  1", "a  +  2"), SRC.replace('"x.h"', '"y.h"'),
                 SRC.replace("// not a comment", "// not a commend")):
        assert bench.code_text(edit) != base


def test_every_kernel_has_a_digest():
    for kernel in bench.KERNEL_SOURCES:
        d = bench.kernel_digest(kernel)
        assert len(d) == 16 and int(d, 16) >= 0


def test_library_binds_to_the_hip_runtime_torch_brings():
    """Loading the library first (before anything imported torch) must still
    leave torch's own HIP runtime as the process's one copy."""
    import os
    import subprocess
    import sys
    code = ("import split_kv_decode_amd as mx; mx.lib(); import torch, os; "
            "maps = open('/proc/self/maps').read().split('\\n'); "
            "paths = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}); "
            "print('\\n'.join(paths))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True,
                         text=True, timeout=600)
    assert out.returncode == 0, out.stderr
    paths = [p for p in out.stdout.split("\n") if p]
    import torch
    torch_lib = os.path.join(os.path.dirname(torch.__file__), "lib")
    assert len(paths) == 1 and paths[0].startswith(torch_lib), paths


def _csv(path, header, rows):
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summary_scales_the_counters_by_the_copy_calibration(tmp_path):
    """The traffic record is the split kernel's median FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) times what a 1 GiB device copy reads as,
    and the achieved rate is the algorithmic bytes over the trace average."""
    import json
    import bench
    import workloads as wl
    split = "void mxfa::split_kv_valu_kernel<0, 128, 4, 4, 1, 1, false>(mxfa::KernelArgs)"
    merge = "void mxfa::combine_kernel<0, 128, 4, false>(mxfa::KernelArgs)"
    copy = "__amd_rocclr_copyBuffer"
    _csv(tmp_path / "t" / "run_kernel_stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
         [[split, 65, 10000.0, 9000, 12000], [merge, 65, 4000.0, 3500, 5000]])
    gib_kib = (1 << 30) // 1024
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    fetch = [[copy, "FETCH_SIZE", gib_kib // 2]] * 3 + \
        [[split, "FETCH_SIZE", v] for v in (30000, 31000, 32000, 33000, 34000)] + \
        [[merge, "FETCH_SIZE", 300]] * 5
    write = [[copy, "WRITE_SIZE", gib_kib]] * 3 + \
        [[split, "WRITE_SIZE", v] for v in (500, 510, 520, 530, 540)] + [[merge, "WRITE_SIZE", 8]] * 5
    _csv(tmp_path / "f" / "run_counter_collection.csv", hdr, fetch)
    _csv(tmp_path / "w" / "run_counter_collection.csv", hdr, write)
    traffic = tmp_path / "traffic.json"
    rec = bench.summarize_profiles(str(tmp_path / "t"), str(tmp_path / "f"), str(tmp_path / "w"),
                                   "smallq_mha_q1_kv1023", ["cmd"], out_dir=str(tmp_path / "p"),
                                   traffic_file=str(traffic))
    # fetch reads half a copy's bytes (scale 2), write all of them (scale 1)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_raw_kib"] == 32000 and rec["write_raw_kib"] == 520
    assert rec["fetch_bytes"] == 32000 * 1024 * 2 and rec["write_bytes"] == 520 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["kernel"] == "split_kv_valu_kernel"
    assert rec["kernel_digest"] == bench.kernel_digest("split_kv_valu_kernel")
    assert json.load(open(traffic))["smallq_mha_q1_kv1023"] == rec
    text = (tmp_path / "p" / "split_kv_valu_kernel_smallq_mha_q1_kv1023.md").read_text()
    w = wl.WORKLOADS["smallq_mha_q1_kv1023"]
    alg = wl.kv_bytes(w, [w.kv_cap] * w.B) + w.B * w.qLen * w.Hq * w.D * w.elt
    assert f"{alg / 10e-6 / 1e9:.1f} GB/s" in text          # over the 10 us trace average
    assert "| 65 | 10.0 |" in text and "| 65 | 4.0 |" in text


def test_profile_summary_of_a_packed_batch(tmp_path):
    """The packed chunked-prefill batch: the same counter arithmetic, its
    distinct K/V + Q bytes and its attention flops."""
    import bench
    import workloads as wl
    split = "void mxfa::mfma::split_kv_mfma_kernel<1, 128, 128, 1, 0, false, 0, false, true, false, 0>(mxfa::KernelArgs)"
    copy = "__amd_rocclr_copyBuffer"
    _csv(tmp_path / "t" / "run_kernel_stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
         [[split, 25, 900000.0, 880000, 950000]])
    gib_kib = (1 << 30) // 1024
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _csv(tmp_path / "f" / "run_counter_collection.csv", hdr,
         [[copy, "FETCH_SIZE", gib_kib // 2]] * 3 + [[split, "FETCH_SIZE", 1000000]] * 3)
    _csv(tmp_path / "w" / "run_counter_collection.csv", hdr,
         [[copy, "WRITE_SIZE", gib_kib]] * 3 + [[split, "WRITE_SIZE", 20000]] * 3)
    rec = bench.summarize_profiles(str(tmp_path / "t"), str(tmp_path / "f"), str(tmp_path / "w"),
                                   "llama70b_chunked_prefill", ["cmd"],
                                   out_dir=str(tmp_path / "p"),
                                   traffic_file=str(tmp_path / "traffic.json"))
    assert rec["kernel"] == "split_kv_mfma_kernel" and rec["fetch_bytes"] == 1000000 * 2048
    w = wl.VARLEN_WORKLOADS["llama70b_chunked_prefill"]
    text = (tmp_path / "p" / "split_kv_mfma_kernel_llama70b_chunked_prefill.md").read_text()
    fl = wl.varlen_flops(w)
    assert f"{fl / 900e-6 / 1e12:.1f} TFLOP/s from the trace average" in text
    alg = 2 * sum(w.klens) * w.Hkv * w.D * 2 + sum(w.qlens) * w.Hq * w.D * 2
    assert f"{1000000 * 2048 / alg:.2f}x the distinct" in text


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout
