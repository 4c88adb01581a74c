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



def test_graded_bound_follows_arithmetic_intensity():
    """Decode and the two HBM-bound prefill layers are graded on HBM bandwidth,
    the 24B share (intensity near the ridge) on the matrix cores."""
    b = _bench()
    from mixture_experts_transformer_moe_amd import workloads as W
    S = W.WORKLOADS
    assert b.graded_bound(S["decode_350m_moe128"], 7.8, 7.8) == "hbm"
    assert b.graded_bound(S["prefill_1p3b_moe128"], 32, 483) == "hbm"
    assert b.graded_bound(S["prmoe_residual"], 64, 2048) == "hbm"
    assert b.graded_bound(S["share_24b_moe128"], 16, 4628) == "mfma"


def test_cpu_baseline_on_a_prefill_shaped_batch():
    """The sampled oracle baseline of a large batch (routing of every token, some
    experts timed, the rest scaled by rows) runs on host tensors and says what it
    sampled."""
    b = _bench()
    from mixture_experts_transformer_moe_amd import workloads as W
    for shape in (W.REDUCED["prefill_reduced"].with_(T=256, H=128, F=256),
                  W.REDUCED["residual_reduced"].with_(T=128, H=64, F=128)):
        w = W.make_weights(shape, 0)
        xs = [W.make_x(shape, 1000)]
        r = b.cpu_baseline(shape, w, xs, 0.05)
        assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
        assert "active experts" in r["sample"] and "rows" in r["sample"]
