"""CPU checks of the measurement tooling: bench.py's one-GPU contract and the
source hash that ties a committed counter record to the kernel code."""
import os
import subprocess
import sys

from verify_gemm_amd import profile_summary

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    """--gpus above 1 ends with a message and exit status 2, before any GPU
    work (there is no multi-GPU path)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {\n  // a comment\n  return x + 1;  /* inline */\n}\n"
    b = "int f(int x) {\n\n    return x + 1;\n}  // changed comment\n"
    assert profile_summary.code_only(a) == profile_summary.code_only(b)


def test_code_only_sees_code_changes():
    a = "int f(int x) { return x + 1; }\n"
    b = "int f(int x) { return x + 2; }\n"
    assert profile_summary.code_only(a) != profile_summary.code_only(b)


def test_code_only_keeps_comment_markers_inside_literals():
    """A '//' inside a string literal is code, not a comment."""
    a = 'const char* s = "a // b";\n'
    assert "// b" in profile_summary.code_only(a)
    assert profile_summary.code_only(a) != profile_summary.code_only('const char* s = "a ";\n')
