"""Host-side logic of bench.py that needs no GPU: the code-only hash that
keys the committed counter summaries to the kernel sources."""
import os

import bench


def test_code_only_drops_comments_and_layout():
    a = "int f(int x)\n{\n    return x + 1;  // one more\n}\n"
    b = "/* header */\nint f(int x)\n{\n\n      return x + 1;\n}   \n"
    assert bench._code_only(a) == bench._code_only(b) == "int f(int x)\n{\nreturn x + 1;\n}"


def test_code_only_keeps_literals_and_code_changes():
    s = 'const char *u = "http://x/*y*/"; char c = \'/\'; // tail\n'
    assert bench._code_only(s) == 'const char *u = "http://x/*y*/"; char c = \'/\';'
    esc = 'const char *q = "a\\"//b"; int k;\n'
    assert bench._code_only(esc) == 'const char *q = "a\\"//b"; int k;'
    assert bench._code_only("x = a + b;") != bench._code_only("x = a - b;")


def test_kernel_source_sha_follows_code_only(tmp_path, monkeypatch):
    src = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "causal_attention_attn_amd", "csrc")
    for n in os.listdir(src):
        (tmp_path / n).write_text(open(os.path.join(src, n), encoding="utf-8").read(), encoding="utf-8")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    base = bench.kernel_source_sha()
    f = tmp_path / "gemm.hip"
    f.write_text("// a new comment line\n" + f.read_text(encoding="utf-8"), encoding="utf-8")
    assert bench.kernel_source_sha() == base
    f.write_text(f.read_text(encoding="utf-8") + "\nnamespace attn { int kernel_source_probe_symbol; }\n",
                 encoding="utf-8")
    assert bench.kernel_source_sha() != base
