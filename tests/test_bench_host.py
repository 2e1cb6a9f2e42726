"""Host-side logic of bench.py that needs no GPU: the key under which HBM
traffic counters are recorded (profiles/traffic.json)."""
import json
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


def test_code_hash_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) {  /* twice */ return 2 * x; }\n")
    h0 = bench.sources_code_sha256([str(a)])
    a.write_text("// a different header\n\nint f(int x) {\n  // doubled\n  return 2 * x;\n}\n")
    assert bench.sources_code_sha256([str(a)]) == h0
    a.write_text("int f(int x) { return 3 * x; }\n")
    assert bench.sources_code_sha256([str(a)]) != h0


def test_code_hash_separates_files(tmp_path):
    a, b = tmp_path / "a.h", tmp_path / "b.h"
    a.write_text("int x;")
    b.write_text("int y;")
    assert bench.sources_code_sha256([str(a), str(b)]) != bench.sources_code_sha256([str(b), str(a)])


def test_traffic_records_are_well_formed():
    """Each record names its kernel, existing source files, a code hash, the
    counter means and their scale factors, and byte counts that follow from
    them; a record is only reported for its own workload and kernel."""
    recs = json.loads((ROOT / "profiles" / "traffic.json").read_text())["workloads"]
    assert {"decode_llama3_8b", "decode_70b_ragged", "decode_long_131k"} <= set(recs)
    for workload, rec in recs.items():
        assert all((ROOT / s).is_file() for s in rec["sources"])
        assert len(rec["sources_code_sha256"]) == 64
        assert rec["read_bytes"] > 0 and rec["write_bytes"] > 0
        assert abs(rec["read_bytes"] - rec["fetch_kib_mean"] * rec["fetch_scale"] * 1024) < 1024
        assert abs(rec["write_bytes"] - rec["write_kib_mean"] * rec["write_scale"] * 1024) < 1024
        assert bench.recorded_traffic(rec["kernel"], "no_such_workload") is None
        assert bench.recorded_traffic("no_such_kernel", workload) is None
