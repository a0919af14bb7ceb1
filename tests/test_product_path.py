"""The product path has no fallback: the binding refuses to import without
its HIP library, and no product source imports the CPU oracle (only tests,
the smoke check and the benchmark's CPU-baseline leg may)."""
import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mla_latent_kv_17_amd")


def test_binding_fails_loudly_without_library(tmp_path):
    copy = tmp_path / "mla_latent_kv_17_amd"
    copy.mkdir()
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            shutil.copy(os.path.join(PKG, f), copy / f)
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    r = subprocess.run([sys.executable, "-c", "import mla_latent_kv_17_amd"], cwd=tmp_path, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "is not built" in r.stderr, r.stderr[-2000:]


def test_binding_refuses_a_stale_library(tmp_path):
    """A library built from other sources than the ones beside it (here: one
    kernel source changed after the build) is refused at import."""
    copy = tmp_path / "mla_latent_kv_17_amd"
    shutil.copytree(PKG, copy, ignore=shutil.ignore_patterns("_build", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    with open(copy / "csrc" / "combine.hip", "a") as fh:
        fh.write("\n// changed after the build\n")
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    r = subprocess.run([sys.executable, "-c", "import mla_latent_kv_17_amd"], cwd=tmp_path, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "built from other sources" in r.stderr, r.stderr[-2000:]


def test_product_sources_never_import_the_oracle():
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle[\s.])", re.M)
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), errors="replace").read()
                assert not pat.search(text), os.path.join(dirpath, f)
                assert "mla_oracle" not in text, os.path.join(dirpath, f)
