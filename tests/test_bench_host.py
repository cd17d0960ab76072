"""Host-side checks of bench.py: the single-GPU guard and the kernel code digest that decides
whether the committed counter summary still applies."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


def test_code_digest_ignores_comments_only(tmp_path):
    code = "int f(int x) {\n  return x + 1;\n}\n"
    a = tmp_path / "a.hip"
    a.write_text(code)
    b = tmp_path / "b.hip"
    b.write_text("// header\n/* block\n comment */\nint f(int x) {  // trailing\n\n  return x + 1;\n}\n")
    c = tmp_path / "c.hip"
    c.write_text(code.replace("+ 1", "+ 2"))
    assert bench.src_sha(str(a)) == bench.src_sha(str(b))
    assert bench.src_sha(str(a)) != bench.src_sha(str(c))
