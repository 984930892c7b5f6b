"""Contract checks that need no GPU: the product path never reaches the oracle, and the benchmark
refuses more than one GPU with a message."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_product_package_does_not_import_the_oracle():
    """No module of the package (binding, device helpers, build) imports `oracle`, and importing the
    package leaves it unloaded."""
    pkg = os.path.join(ROOT, "world_action_video_amd")
    for name in os.listdir(pkg):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(pkg, name)).read())
        for node in ast.walk(tree):
            mods = []
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)
    code = "import sys; import world_action_video_amd, world_action_video_amd.device; print('oracle' in sys.modules)"
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == "False", out.stderr


def test_oracle_does_not_import_the_product_path():
    odir = os.path.join(ROOT, "oracle")
    for name in os.listdir(odir):
        if name.endswith(".py"):
            src = open(os.path.join(odir, name)).read()
            assert "world_action_video_amd" not in src, name


def test_bench_refuses_more_than_one_gpu():
    out = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode != 0 and "one GPU" in out.stderr
