import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_report_header(config):
    """Name the library the session loads and whether it was built from the
    sources in the tree (the loader refuses it otherwise)."""
    from mixture_experts_layer_amd import build as B
    from mixture_experts_layer_amd._abi import lib_path
    path = lib_path()
    want = B.source_sha256()
    try:
        import mixture_experts_layer_amd as M
        got = M.moe_source_sha256()
        state = "matches the sources" if got == want else f"STALE (built from {got[:12]})"
    except ImportError as e:
        state = f"not loadable: {e}"
    return f"HIP library {path}: sources {want[:12]}, {state}"


def golden(name):
    import json
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return json.load(f)
