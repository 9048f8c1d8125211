"""bench.py's command-line contract, on the host: it measures one GPU only
(asked for more it exits with status 2 and says so) and needs a GPU (without
one it exits with status 2 instead of falling back to anything); the source
hash that keys the measured HBM traffic is stable and covers the listed
kernel sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_no_gpu_means_no_number():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_kernel_sources_hash_is_stable():
    sys.path.insert(0, ROOT)
    import bench
    for files in (bench.BF16_SOURCES, bench.FP8_SOURCES, bench.MXFP4_SOURCES, bench.RESIDUAL_SOURCES):
        for f in files:
            assert os.path.isfile(os.path.join(ROOT, f)), f
        h = bench.kernel_sources_hash(files)
        assert h == bench.kernel_sources_hash(list(files)) and len(h) == 16
        int(h, 16)
    assert len({bench.kernel_sources_hash(f) for f in (bench.BF16_SOURCES, bench.FP8_SOURCES,
                                                       bench.MXFP4_SOURCES, bench.RESIDUAL_SOURCES)}) == 4
