"""bench.py's host logic (CPU): the committed profile figures it reads are
taken on the current prefill sources, its source digest ignores comments and
whitespace but not code, and a request for several GPUs ends with a message
before anything touches a device."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_profile_figures_match_the_sources():
    """The traffic and counted-MFMA lines of profiles/ carry the digest of
    the sources as they stand, so the bench line reports both (a kernel
    change without a re-taken profile makes them null and fails here)."""
    traffic = bench.measured_traffic()
    flops = bench.counted_mfma_flops()
    assert traffic is not None and flops is not None
    # 9.69 GB of algorithmic bytes per K3 call: the counted traffic is above
    # it, and the counted 16-bit MFMA FLOPs above the 8.85e11 useful ones
    assert 9.69e9 < traffic < 5e10
    assert 8.85e11 < flops < 5e12


def test_digest_ignores_comments_not_code(tmp_path, monkeypatch):
    csrc = os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc")
    copy = tmp_path / "gated_delta_rule_21_amd" / "csrc"
    copy.mkdir(parents=True)
    for f in bench.PREFILL_SOURCES:
        shutil.copy(os.path.join(csrc, f), copy / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_sources_digest()
    target = copy / "kda_chunk.h"
    text = target.read_text()
    target.write_text("// a new comment line\n/* and a block\n   comment */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_sources_digest() == base
    target.write_text(text + "\nstatic const int kda_digest_probe = 1;\n")
    assert bench.kernel_sources_digest() != base


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
