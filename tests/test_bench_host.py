"""Host-side logic of bench.py (CPU only): the one-GPU guard and the rule that
counter summaries under profiles/ are used only while they match the kernel
source they were taken on."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def fake_tree(tmp_path, code):
    (tmp_path / "sparse_moe_ffn_softmax_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "sparse_moe_ffn_softmax_amd" / "csrc" / "k.hip").write_text(code)


def test_source_digest_ignores_comments_not_code(tmp_path):
    b = load_bench()
    b.ROOT = str(tmp_path)
    fake_tree(tmp_path, "int f(int a) {\n  return a + 1;\n}\n")
    d0 = b.source_digest("k.hip")
    (tmp_path / "sparse_moe_ffn_softmax_amd" / "csrc" / "k.hip").write_text(
        "// header\n\nint f(int a) {  // trailing note\n  return a + 1;\n\n}\n")
    assert b.source_digest("k.hip") == d0
    (tmp_path / "sparse_moe_ffn_softmax_amd" / "csrc" / "k.hip").write_text("int f(int a) {\n  return a + 2;\n}\n")
    assert b.source_digest("k.hip") != d0


def test_measured_traffic_only_for_the_same_source_and_layout(tmp_path):
    b = load_bench()
    b.ROOT = str(tmp_path)
    fake_tree(tmp_path, "int f() { return 0; }\n")
    rec = {"code_sha256_16": b.source_digest("k.hip"), "weight_layout": "panels", "hbm_bytes_per_launch": 12345}
    (tmp_path / "profiles" / "kern_wl_pmc.json").write_text(json.dumps(rec))
    assert b.measured_traffic("kern", "wl", "k.hip", "panels") == 12345
    assert b.measured_traffic("kern", "wl", "k.hip", "rows") is None        # other layout
    assert b.measured_traffic("kern", "other", "k.hip", "panels") is None   # no summary
    (tmp_path / "sparse_moe_ffn_softmax_amd" / "csrc" / "k.hip").write_text("int f() { return 1; }\n")
    assert b.measured_traffic("kern", "wl", "k.hip", "panels") is None      # kernel changed since
