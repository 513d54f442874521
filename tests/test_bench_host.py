"""Host logic of bench.py that needs no GPU: the source digest that keeps the
recorded counter traffic tied to the code it was measured on."""
import bench


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
