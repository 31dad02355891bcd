"""bench.py's contract that needs no GPU: more than one GPU is refused with a
message, and the recorded traffic of a kernel is dropped once its source
changes."""
import hashlib
import importlib.util
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


def test_traffic_is_dropped_when_the_source_changes(tmp_path):
    b = _bench()
    tab = json.load(open(b.TRAFFIC_TABLE))
    src_name = tab["workloads"]["mixtral"]["ffn_up"]["source"]
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    shutil.copy(os.path.join(b.CSRC, src_name), csrc / src_name)
    b.CSRC = str(csrc)
    now = hashlib.sha256((csrc / src_name).read_bytes()).hexdigest()
    expected = tab["workloads"]["mixtral"]["ffn_up"]["hbm_bytes"] if tab["sources"][src_name] == now else None
    assert b.kernel_traffic("mixtral", "ffn_up") == expected
    with open(csrc / src_name, "a") as f:
        f.write("\n// changed\n")
    assert b.kernel_traffic("mixtral", "ffn_up") is None
    assert b.kernel_traffic("mixtral", "no_such_kernel") is None
