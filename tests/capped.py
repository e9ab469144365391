"""Helper of the workgroup-cap tests: runs tests.cap_child in a child
process with one cap variable set, and returns what it computed."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_capped(tmp_path, scenario, arrays, var, cap):
    src, dst = tmp_path / f"{scenario}_in.npz", tmp_path / f"{scenario}_{cap}_out.npz"
    np.savez(src, **arrays)
    env = dict(os.environ, **{var: str(cap)})
    print(f"child process: {scenario} with {var}={cap}", flush=True)
    r = subprocess.run([sys.executable, "-m", "tests.cap_child", scenario, str(src), str(dst)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"child failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    with np.load(dst) as d:
        return [d[f"arr_{k}"] for k in range(len(d.files))]
