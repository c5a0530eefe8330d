"""Host-side pieces of bench.py (no GPU): the source digest that ties a
committed counter summary to the code it was taken on."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_code_tokens_drop_comments_and_layout_only():
    src = 'int a = 1; // note\n/* block\n   comment */ const char* s = "a//b /*c*/";\n  char q = \'"\';  int  b;\n'
    assert bench._code_tokens(src) == 'int a = 1; const char* s = "a//b /*c*/"; char q = \'"\'; int b;'
    # a comment or re-indented line changes nothing; a changed token does
    assert bench._code_tokens(src.replace("// note", "// other words")) == bench._code_tokens(src)
    assert bench._code_tokens(src.replace("  int  b;", "\n\tint b;")) == bench._code_tokens(src)
    assert bench._code_tokens(src.replace("int a = 1", "int a = 2")) != bench._code_tokens(src)
    assert bench._code_tokens(src.replace('"a//b', '"a/b')) != bench._code_tokens(src)


def test_source_digest_is_stable():
    assert bench.source_digest() == bench.source_digest()
    assert len(bench.source_digest()) == 64
