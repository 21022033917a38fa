"""bench.py on the CPU: the one-GPU guard and the traffic-summary reader (no GPU needed)."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_cli_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""


def test_traffic_summaries_parse(tmp_path):
    b = load_bench()
    # a summary whose hashes match nothing yields no figures; a matching one yields bytes
    k = "extend_kernel"
    good = tmp_path / "good.txt"
    good.write_text(f"# header\nkernel={k} dispatches=4 hbm_bytes=1234 source_sha={b.source_sha(k)}\n")
    stale = tmp_path / "stale.txt"
    stale.write_text(f"kernel={k} dispatches=4 hbm_bytes=1234 source_sha=0000000000000000\n")
    assert b.read_traffic(str(good)) == {k: 1234}
    assert b.read_traffic(str(stale)) == {}
