"""Host logic of bench.py (no GPU): the digest that ties stored counter
readings to the kernel sources sees code changes and ignores comments."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_strip_comments_keeps_code_and_literals():
    b = _bench()
    src = ('#define N 8 // eight\n'
           'int f(int x) { /* block\n comment */ return x + N; }  \n\n'
           'const char* s = "a // not a comment /* nor this */";\n'
           "char q = '\\'';  // quote\n")
    assert b.strip_comments(src) == ('#define N 8\n'
                                     'int f(int x) { return x + N; }\n'
                                     'const char* s = "a // not a comment /* nor this */";\n'
                                     "char q = '\\'';")


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "CSRC", str(tmp_path))
    f = tmp_path / "k.hip"
    f.write_text("__global__ void k(float* p) { p[0] = 1.f; }\n")
    d0 = b.kernel_source_digest(["k.hip"])
    f.write_text("// a kernel\n\n__global__  void k(float* p) { p[0] = 1.f;  /* one */ }  // store\n")
    assert b.kernel_source_digest(["k.hip"]) == d0
    f.write_text("__global__ void k(float* p) { p[0] = 2.f; }\n")
    assert b.kernel_source_digest(["k.hip"]) != d0

