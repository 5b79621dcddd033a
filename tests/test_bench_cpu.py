"""CPU checks of bench.py's contract that need no GPU: every function its main
path calls is defined, and more than one GPU is refused with a message."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_main_calls_defined_functions():
    tree = ast.parse(open(BENCH).read())
    defined = {n.name for n in tree.body if isinstance(n, ast.FunctionDef)}
    called = set()
    for fn in tree.body:
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, ast.Call) and isinstance(node.func, ast.Name):
                    called.add(node.func.id)
    local = {c for c in called if c.startswith(("bench_", "time_", "cpu_", "prefill_", "segment_", "merge_",
                                                 "direct_", "kernel_"))}
    assert local <= defined, sorted(local - defined)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr
