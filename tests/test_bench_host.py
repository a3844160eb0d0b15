"""Host-side checks of bench.py and of the committed measurement records (no
GPU): the benchmark refuses more than one GPU before touching any; the HBM
traffic figure it reports is read from the committed counter record only
while the kernel sources it was taken on are unchanged; and every summary
under profiles/ names the digest of the kernel sources it was taken on,
which is that of the sources as they stand."""

import glob
import hashlib
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _csrc_digest():
    """sha256 over sparse_moe_expert_amd/csrc/*.hip and *.h, contents
    concatenated in sorted path order (the digest the summaries quote)."""
    csrc = os.path.join(ROOT, "sparse_moe_expert_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h")))
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_is_current():
    import bench
    t = bench.measured_traffic("decode_t4", "select_gate_up_kernel")
    assert t is not None and t > 0


def test_traffic_record_ignored_when_sources_change(monkeypatch):
    import bench
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "0" * 64)
    assert bench.measured_traffic("decode_t4", "select_gate_up_kernel") is None
    assert bench.measured_traffic("decode_t4", "no_such_kernel") is None


def test_profiles_name_the_current_sources():
    digest = _csrc_digest()[:16]
    mds = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert mds
    for p in mds:
        with open(p) as f:
            text = f.read()
        m = re.search(r"sha256 prefix:? `([0-9a-f]{16})`", text)
        assert m, f"{os.path.basename(p)} names no source digest"
        assert m.group(1) == digest, f"{os.path.basename(p)} was taken on other sources"
