"""Host-side pieces of the benchmark (no GPU needed)."""
import json
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parents[1]


def test_source_hash_ignores_comments_and_blank_lines(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) {  // doubles x\n    return 2 * x;\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("// a file comment\nint f(int x) {  // another comment\n\n    return 2 * x;   \n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) {\n    return 3 * x;\n}\n")
    assert bench.source_hash(a) == bench.source_hash(b)
    assert bench.source_hash(a) != bench.source_hash(c)


def test_counters_file_names_the_hashed_source():
    js = json.loads((ROOT / "profiles" / "diffusion_march_counters.json").read_text())
    assert (ROOT / js["source"]).exists()
    assert len(js["source_sha"]) == 16
    assert set(js["per_launch_bytes"]) >= {"f32_16384_T10"}


def test_more_than_one_gpu_is_refused_with_a_message():
    out = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    line = json.loads(out.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
