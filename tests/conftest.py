import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for _p in (TESTS, ROOT):  # worker processes forked at configure time import from both
    if _p not in sys.path:
        sys.path.insert(0, _p)


def _may_run_gpu_tests(config) -> bool:
    expr = " ".join((config.option.markexpr or "").split())
    return "not gpu" not in expr and os.path.exists("/dev/kfd")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")
    # Worker processes for the host side of the stack tests (drawing,
    # expanding and checking 252 matrices).  They are forked here, before any
    # test module initialises the GPU runtime in this process, and never use
    # the GPU themselves.
    config._lvq_pool = None
    if _may_run_gpu_tests(config):
        import multiprocessing as mp
        try:
            n = len(os.sched_getaffinity(0))
        except AttributeError:
            n = os.cpu_count() or 1
        config._lvq_pool = mp.get_context("fork").Pool(max(1, min(16, n)))


def pytest_unconfigure(config):
    pool = getattr(config, "_lvq_pool", None)
    if pool is not None:
        pool.terminate()
        pool.join()


@pytest.fixture(scope="session")
def host_pool(request):
    """The worker pool forked before the GPU runtime started, or None."""
    return request.config._lvq_pool


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The HIP library binding; GPU tests need it built and loadable."""
    import dequant_gemv_lvq_amd as lvq
    return lvq
