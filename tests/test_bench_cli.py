"""bench.py's host-side contract (no GPU needed): more than one GPU is
refused with a message, and without a GPU it fails loudly instead of
falling back to anything."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("launches", ["fused", "clipped"])
def test_one_call_steps_and_8bit_together_are_refused_or_need_a_gpu(launches):
    r = run("--launches", launches, "--state8")
    assert r.returncode != 0 and r.stdout.strip() == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_no_gpu_fails_loudly():
    r = run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_slices_cover_every_element_once_at_the_alignment():
    sys.path.insert(0, ROOT)
    import bench

    for n in (0, 1, 5, 31, 32, 100, 1000, 4097):
        for parts in (1, 3, 8, 16):
            for align in (1, 32):
                s = bench._slices(n, parts, align)
                assert len(s) <= parts
                assert [e for lo, hi in s for e in range(lo, hi)] == list(range(n))
                assert all(lo % align == 0 and hi > lo for lo, hi in s)


def test_cpu_baseline_reports_one_thread_and_all_threads():
    """The oracle leg of the bench on host tensors: one-thread and threaded
    timings of the same sample, each with its core count."""
    sys.path.insert(0, ROOT)
    import bench
    from mixed_precision_sharded_amd import synth
    from mixed_precision_sharded_amd.configs import Workload

    w = Workload(cfg=1, name="tiny_two_tensors", tensors=(("a", 3000), ("b", 70)),
                 grad_bf16=True, copy_bf16=True, step=1)
    cols = synth.workload_inputs(w, torch.device("cpu"))
    r = bench.cpu_baseline(w, cols, 0.05, 3)
    assert r["cores"] == 1 and r["kind"] == "oracle" and r["value"] > 0
    assert r["all_cores"]["cores"] == 3 and r["all_cores"]["value"] > 0


def test_same_stream_ceiling_library_rejects_bad_arguments():
    """bench_ceiling.so (the benchmark's same-stream ceiling kernels) exports
    its two functions, and both refuse bad sizes before any HIP call."""
    import ctypes
    path = os.path.join(ROOT, "bench_ceiling.so")
    if not os.path.exists(path):
        import __graft_entry__
        __graft_entry__.build_bench_ceiling()
    fn = ctypes.CDLL(path).stream_ceiling_us
    fn.restype = ctypes.c_double
    P = ctypes.c_void_p
    fn.argtypes = [ctypes.c_int, P, P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, P]
    fake = 0x7f0000000000
    assert fn(1, fake, fake, fake, fake, None, 0, 256, 1, 10, None) < 0       # no elements
    assert fn(1, fake, fake, fake, fake, None, 6, 256, 1, 10, None) < 0       # not a multiple of 4
    assert fn(1, fake, fake, fake, fake, None, 1024, 256, 3, 10, None) < 0    # unroll 3
    assert fn(1, None, fake, fake, fake, None, 1024, 256, 1, 10, None) < 0    # NULL buffer
    fn8 = ctypes.CDLL(path).stream_ceiling8_us
    fn8.restype = ctypes.c_double
    fn8.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P]
    assert fn8(1, fake, fake, None, fake, fake, fake, fake, 0, 256, 10, None) < 0        # no elements
    assert fn8(1, fake, fake, None, fake, fake, fake, fake, 16384 + 32, 256, 10, None) < 0  # not whole chunks
    assert fn8(1, fake, fake, None, None, fake, fake, fake, 16384, 256, 10, None) < 0    # NULL codes
    assert fn8(1, fake, fake, None, fake, fake, fake, fake, 16384, 0, 10, None) < 0      # no blocks
    # Without a GPU, valid arguments pass the checks and fail at the first HIP
    # call (-2 or -3, not the -1 of a refused argument).  Never run with a GPU:
    # the pointers here are not device memory.
    import torch
    if not torch.cuda.is_available():
        assert fn(1, fake, fake, fake, fake, None, 1 << 20, 256, 1, 10, None) <= -2
        assert fn8(0, fake, fake, None, fake, fake, fake, fake, 1 << 20, 256, 10, None) <= -2
