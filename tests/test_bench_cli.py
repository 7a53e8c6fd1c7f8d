"""bench.py contract checks that need no GPU."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_defines_every_run_it_uses():
    tree = ast.parse(open(BENCH).read())
    defined = {n.name for n in tree.body if isinstance(n, (ast.FunctionDef, ast.ClassDef))}
    used = {n.func.id for n in ast.walk(tree) if isinstance(n, ast.Call) and isinstance(n.func, ast.Name)}
    for name in ("VarlenRun", "PagedRun", "DecodeRun", "DecodeStepsRun", "BwdRun", "time_launches", "cpu_baseline",
                 "load_traffic"):
        assert name in defined and name in used, name
