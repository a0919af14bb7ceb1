import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def _ensure_built():
    """Build the HIP library in-tree when nothing is built yet."""
    lib = os.path.join(ROOT, "mla_latent_kv_17_amd", "libmla.so")
    if not os.path.exists(lib):
        import importlib.util  # by path: importing the package needs the library
        spec = importlib.util.spec_from_file_location("_mla_build", os.path.join(ROOT, "mla_latent_kv_17_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


_ensure_built()
