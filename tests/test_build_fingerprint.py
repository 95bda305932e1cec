"""CPU tests of the kernel fingerprint that ties a recorded profile to the
code it measured: comments and white space do not change it, code does."""

from fp4_block_scaled_amax_amd.build import _code_only


def test_comments_and_spacing_ignored():
    a = "int f(int x) {  // doubles x\n    return 2 * x; /* fast */ }\n"
    b = "int f(int x)\n{\n  /* no comment */ return 2 * x;\n}"
    assert _code_only(a) == _code_only(b)


def test_code_and_literals_count():
    assert _code_only("return 2 * x;") != _code_only("return 3 * x;")
    # comment markers inside literals are code, not comments
    s = 'asm("v_add // not a comment"); char c = \'/\'; const char* t = "/* kept */";'
    assert _code_only(s) == s
    assert _code_only('x = "a\\"//b"; // gone') == 'x = "a\\"//b";'
