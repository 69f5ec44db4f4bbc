"""bench.py's command line on the CPU: more than one GPU is refused with a
message before any device work, and the JSON keys the benchmark promises
are the ones main() assembles."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert not any(line.lstrip().startswith("{") for line in r.stdout.splitlines())


def test_json_line_carries_the_contract_keys():
    # the keys are read from the dict literal in bench.main(), so the check
    # needs no GPU
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    keys, roof_keys = set(), set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Dict):
            ks = {k.value for k in node.keys if isinstance(k, ast.Constant)}
            if "metric" in ks and "roofline" in ks:
                keys = ks
                roof = [v for k, v in zip(node.keys, node.values)
                        if isinstance(k, ast.Constant) and k.value == "roofline"][0]
                roof_keys = {k.value for k in roof.keys if isinstance(k, ast.Constant)}
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline", "prediction_interval"):
        assert k in keys, k
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof_keys, k
