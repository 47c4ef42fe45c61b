import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _ensure_built():
    lib = os.path.join(ROOT, "mixture_experts_layer_30_amd", "libmok.so")
    if not os.path.exists(lib):
        from mixture_experts_layer_30_amd.build import build
        build()


_ensure_built()
