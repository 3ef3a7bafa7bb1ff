import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_addoption(parser):
    parser.addoption("--tq-lib", default=None,
                     help="load this build of the library in the CPU ABI tests (the host-sanitizer build)")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle work that takes more than a few seconds")


def load_golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session", autouse=True)
def _oracle_forkserver(request):
    """Start the server that oracle worker pools fork from before any test
    touches the GPU, so the workers are copies of a process that never
    initialised the device (only when GPU tests are selected)."""
    if any(item.get_closest_marker("gpu") for item in request.session.items):
        import multiprocessing as mp
        from multiprocessing import forkserver
        # one BLAS thread per worker process (the pool has one per core)
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
        os.environ.update(OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
        mp.get_context("forkserver").set_forkserver_preload(
            ["numpy", "oracle.store", "oracle.decode", "oracle.soa", "fullsize_oracle"])
        forkserver.ensure_running()
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    yield
