"""Host-side pieces of bench.py (no GPU): the digest that ties the committed
counter summary to the GEMV sources, and the summary's parse."""
import os
import shutil
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _copy_sources(dst):
    for f in bench.GEMV_SOURCES:
        os.makedirs(os.path.join(dst, os.path.dirname(f)), exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), os.path.join(dst, f))


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.sources_digest()
    src = os.path.join(tmp_path, bench.GEMV_SOURCES[0])
    text = open(src).read()
    open(src, "w").write("// a new comment line\n" + text.replace("\n", "\n  ", 3) + "\n/* trailing */\n")
    assert bench.sources_digest() == d0
    open(src, "w").write(text.replace("kLookahead = 3", "kLookahead = 4"))
    assert bench.sources_digest() != d0


def test_committed_traffic_summary_parses():
    # The committed summary carries a byte count and a digest; whether it
    # matches the current sources is checked where the counters are taken.
    text = open(bench.TRAFFIC_FILE).read()
    assert "hbm_bytes_per_launch:" in text and "sources_digest:" in text
