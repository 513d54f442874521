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
