"""The source hash under which committed counter summaries stay valid
(bench.kernel_source_digest): it covers the code of the kernel and host
sources, not their comments or layout."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench


def test_comments_and_layout_do_not_count():
    a = "int f(int x) {\n  return x + 1;   // one more\n}\n"
    b = "/* a function */\nint f(int x)\n{\n    return x + 1;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)


def test_code_changes_count():
    a = "int f(int x) { return x + 1; }"
    b = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) != bench._code_only(b)


def test_literals_are_kept_as_written():
    # a comment marker inside a string literal is part of the code
    a = 'const char* s = "a // b"; int y;'
    b = 'const char* s = "a "; int y;'
    assert bench._code_only(a) != bench._code_only(b)
    assert "// b" in bench._code_only(a)
    # an escaped quote does not end the literal
    c = 'const char* s = "x\\" // y"; int z;'
    assert "// y" in bench._code_only(c)


def test_digest_of_the_sources_is_stable():
    d = bench.kernel_source_digest()
    assert len(d) == 64 and d == bench.kernel_source_digest()
