"""bench.py's command-line contract on the host: more than one GPU is refused with a message and
exit status 2, before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_oracle_row_subset():
    """The CPU baseline's subset: the first 256 rows, the last 256 (the 94-row tail tile at S = 37726
    lies inside them) and every 64th row, each once."""
    import importlib.util

    import numpy as np
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    S = 37726
    r = bench.subset_rows(S)
    assert np.all(np.diff(r) > 0) and r[0] == 0 and r[-1] == S - 1
    assert set(range(256)) <= set(r.tolist()) and set(range(S - 256, S)) <= set(r.tolist())
    assert set(range(0, S, 64)) <= set(r.tolist())
    assert len(r) == 256 + 256 + len(range(256, S - 256, 64))
    assert list(bench.subset_rows(100)) == list(range(100))
