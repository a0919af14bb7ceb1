import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


import pytest


@pytest.fixture(params=["64", "32"], ids=lambda r: f"rows{r}")
def decode_rows(request, monkeypatch):
    """Runs a test with the bf16 decode fixed at 64, then at 32 query rows
    per workgroup (the library otherwise picks by launch size)."""
    monkeypatch.setenv("MLA_DECODE_ROWS", request.param)
    yield request.param


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def _ensure_built():
    """Build the HIP library in-tree when nothing is built yet, or when the
    built one carries the hash of other sources than the ones checked out (so
    the tests never run a stale binary)."""
    import importlib.util  # by path: importing the package needs the library
    spec = importlib.util.spec_from_file_location("_mla_build", os.path.join(ROOT, "mla_latent_kv_17_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    if mod.built_hash() != mod.source_hash():
        print(f"conftest: building {mod.LIB} (built {mod.built_hash()}, sources {mod.source_hash()})", flush=True)
        mod.build()


_ensure_built()
