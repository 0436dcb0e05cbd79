import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def _gpu_tests_deselected(config):
    expr = " ".join((config.getoption("markexpr", default="") or "").split())
    return expr == "not gpu"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # Worker processes for the fp64 oracle over whole full-size workloads.  They are forked here,
    # before any test touches the GPU (a process that has initialised HIP must not fork).
    # A second, smaller pool runs the autograd oracle of the backward: torch's autograd engine asks the
    # GPU runtime for its device count on its first backward pass, which opens the GPU in that worker,
    # and a GPU machine admits at most 16 processes with the GPU open (this one and the workers).
    config._oracle_pool = config._oracle_grad_pool = None
    if not _gpu_tests_deselected(config):
        from oracle.parallel import grad_workers, make_pool

        config._oracle_pool = make_pool()
        config._oracle_grad_pool = make_pool(grad_workers())


def pytest_unconfigure(config):
    for name in ("_oracle_pool", "_oracle_grad_pool"):
        pool = getattr(config, name, None)
        if pool is not None:
            pool.terminate()
            pool.join()


@pytest.fixture(scope="session")
def oracle_pool(request):
    pool = request.config._oracle_pool
    if pool is None:
        from oracle.parallel import make_pool

        # only reached when the marker expression deselected the GPU tests: no GPU in this process
        pool = request.config._oracle_pool = make_pool(2)
    return pool


@pytest.fixture(scope="session")
def oracle_grad_pool(request):
    pool = request.config._oracle_grad_pool
    if pool is None:
        from oracle.parallel import make_pool

        # only reached when the marker expression deselected the GPU tests: no GPU in this process
        pool = request.config._oracle_grad_pool = make_pool(2)
    return pool
