"""Host-side pieces of bench.py (CPU only): the digest that ties the committed
traffic counters to the decode sources ignores comments and whitespace but
not code."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _digest(monkeypatch, tmp_path, texts):
    paths = []
    for i, t in enumerate(texts):
        p = tmp_path / f"src{i}.hip"
        p.write_text(t)
        paths.append(str(p))
    monkeypatch.setattr(bench, "DECODE_SRCS", paths)
    return bench.source_digest()


def test_digest_ignores_comments_and_whitespace(monkeypatch, tmp_path):
    base = _digest(monkeypatch, tmp_path, ["int f(int x) { return x + 1; }\n", "// a\nint g;\n"])
    same = _digest(monkeypatch, tmp_path, ["/* note */ int f(int x) {\n  return x + 1;  // add one\n}\n",
                                           "int   g;\n"])
    assert same == base


def test_digest_follows_code(monkeypatch, tmp_path):
    base = _digest(monkeypatch, tmp_path, ["int f(int x) { return x + 1; }\n", "int g;\n"])
    changed = _digest(monkeypatch, tmp_path, ["int f(int x) { return x + 2; }\n", "int g;\n"])
    assert changed != base

