"""bench.py on the CPU: its one-GPU contract and the freshness of the counter
records it reports.

* ``--gpus`` above 1 exits with status 2 and a message that says there is no
  multi-GPU path (nothing is launched).
* The committed rocprofv3 records (prefill HBM traffic, prefill MFMA
  utilisation, decode HBM bytes) were taken on the kernel code now in the
  tree.  Each record carries a hash of its kernel's sources, comments and
  blank space removed.  A stale record makes the bench report its traffic as
  null, so a kernel change must come with new counter runs.
* A record whose hash does not match is refused."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_committed_counter_records_are_current():
    assert bench._current_record(bench.TRAFFIC_FILE) is not None, "prefill traffic record is stale"
    assert bench._current_record(bench.MFMA_FILE) is not None, "prefill MFMA record is stale"
    assert bench._current_record(bench.DECODE_TRAFFIC_FILE, bench.DECODE_SOURCES) is not None, \
        "decode traffic record is stale"
    assert bench.traffic_per_launch() is not None


def test_stale_record_is_refused(tmp_path):
    rec = json.load(open(bench.TRAFFIC_FILE))
    rec["kernel_source_sha"] = "0" * 16
    p = tmp_path / "stale.json"
    p.write_text(json.dumps(rec))
    assert bench._current_record(str(p)) is None
    assert bench._current_record(str(tmp_path / "missing.json")) is None


def test_mfma_record_covers_both_launches():
    """The non-causal launch's busy cycles per SIMD equal its algorithmic
    MFMA count (1.0995e12 FLOP / 32,768 FLOP per 32x32x16 MFMA / 1024 SIMDs,
    32 cycles each); the causal launch needs at least half of that (its
    visible pairs) and, with whole tiles on the diagonal, a little more."""
    rec = json.load(open(bench.MFMA_FILE))
    assert rec["kernel"] == bench.PREFILL_KERNEL
    assert set(rec["mfma_busy_cycles_per_simd"]) == {1048576}
    c = rec["causal"]
    assert c["kernel"] == bench.PREFILL_KERNEL_CAUSAL
    assert all(524288 <= b <= 1.1 * 524288 for b in c["mfma_busy_cycles_per_simd"])
    assert len(c["mfma_util_pct"]) == c["dispatches"] == len(c["clock_ghz"])
