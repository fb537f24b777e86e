"""CPU tests of bench.py's host logic (no GPU, no library calls): the source
digest that ties stored counter figures to kernel code, the traffic lookup
that honours it, and the refusal of more than one GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_blank_lines_but_not_strings():
    src = (
        "// header comment\n"
        "int a = 1;   // trailing\n"
        "\n"
        "/* block\n   comment */ int b = 2;\n"
        'const char *s = "// not a comment";  /* x */\n'
        "char c = '/';\n"
    )
    want = "int a = 1;\n int b = 2;\nconst char *s = \"// not a comment\";\nchar c = '/';"
    assert bench._code_only(src) == want


def test_code_only_keeps_every_token_of_code():
    src = "x = y / z;  // divide\nw = *p;\n"
    assert bench._code_only(src) == "x = y / z;\nw = *p;"


def _digest_of(tmp_path, files, only=None):
    csrc = tmp_path / "sparse_attention_block_qsa_amd" / "csrc"
    csrc.mkdir(parents=True, exist_ok=True)
    for name in os.listdir(csrc):
        (csrc / name).unlink()
    for name, text in files.items():
        (csrc / name).write_text(text)
    old = bench.ROOT
    try:
        bench.ROOT = str(tmp_path)
        return bench.source_digest(only)
    finally:
        bench.ROOT = old


def test_source_digest_ignores_comments_and_follows_code(tmp_path):
    base = _digest_of(tmp_path, {"k.hip": "int f() { return 1; }\n"})
    assert _digest_of(tmp_path, {"k.hip": "// why\nint f() { return 1; }  // one\n\n"}) == base
    assert _digest_of(tmp_path, {"k.hip": "int f() { return 2; }\n"}) != base
    assert _digest_of(tmp_path, {"k2.hip": "int f() { return 1; }\n"}) != base


def test_kernel_digest_follows_only_its_own_files(tmp_path):
    a = {"a.hip": "int f() { return 1; }\n", "b.hip": "int g() { return 1; }\n"}
    base = _digest_of(tmp_path, a, only=("a.hip",))
    assert _digest_of(tmp_path, {**a, "b.hip": "int g() { return 2; }\n"}, only=("a.hip",)) == base
    assert _digest_of(tmp_path, {**a, "a.hip": "int f() { return 2; }\n"}, only=("a.hip",)) != base
    for files in bench.KERNEL_FILES.values():   # every listed file exists
        for name in files:
            assert os.path.exists(os.path.join(ROOT, "sparse_attention_block_qsa_amd", "csrc", name))


def test_read_traffic_needs_the_current_digest(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    (prof / "traffic_k_w.txt").write_text(
        "# comment\nsource_digest=%s\nbytes_per_launch=1234\n" % bench.source_digest())
    assert bench.read_traffic("k", "w") == 1234.0
    (prof / "traffic_k_w.txt").write_text("source_digest=0000000000000000\nbytes_per_launch=1234\n")
    assert bench.read_traffic("k", "w") is None
    assert bench.read_traffic("missing", "w") is None


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
