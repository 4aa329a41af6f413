"""Host-side pieces of bench.py that need no GPU: the digest that decides whether the
committed HBM-traffic counters still describe the kernel sources, and the refusal of
more than one GPU."""
import subprocess
import sys

import bench


def test_digest_ignores_comments_and_whitespace():
    a = "int f(int x) {  // scale\n  return 2 * x; /* twice */\n}\n"
    b = "// a comment line\nint f(int x) {\n    return 2 * x;\n}   /* trailing\n block */\n"
    assert bench._code_text(a) == bench._code_text(b)


def test_digest_sees_code_changes():
    a = "int f(int x) { return 2 * x; }"
    assert bench._code_text(a) != bench._code_text("int f(int x) { return 3 * x; }")
    assert bench._code_text(a) != bench._code_text("int f(int y) { return 2 * y; }")


def test_digest_of_the_sources_is_stable():
    d = bench._source_digest()
    assert len(d) == 16 and d == bench._source_digest()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
