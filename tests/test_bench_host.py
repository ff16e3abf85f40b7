"""Host-side contract of bench.py (no GPU): one GPU only, and the stored HBM
traffic figure is used only for the GEMM source it was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_committed_traffic_record_is_well_formed():
    # the counter record under profiles/ names the source it was taken on; the
    # bench uses its figure only while that source is unchanged (else null)
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    assert len(rec["source_sha256"]) == 64
    assert rec["bytes_per_launch"] > 0
    t = bench.stored_traffic()
    assert t is None or t == rec["bytes_per_launch"]


def test_traffic_is_null_once_the_source_changes(tmp_path):
    src = tmp_path / "gemm.hip"
    src.write_text("// a different kernel\n")
    rec = {"source_sha256": bench.source_hash(bench.GEMM_SOURCE), "bytes_per_launch": 1.0}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    assert bench.stored_traffic(str(f), bench.GEMM_SOURCE) == 1.0
    assert bench.stored_traffic(str(f), str(src)) is None
    assert bench.stored_traffic(str(tmp_path / "missing.json")) is None
