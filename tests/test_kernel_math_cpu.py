"""The FFT gray block's arithmetic (csrc/fi_fft.h), compiled for the CPU with a
small shim and run thread by thread: every transform size the kernels use must
reproduce the direct sum of the gray block.  This checks the HIP path's own
code (pairing of real bins, radix-16 groups, twiddles, pruning), not the oracle."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fft_tile_arithmetic_matches_direct_sums(tmp_path):
    exe = str(tmp_path / "fft_tile_check")
    src = os.path.join(HERE, "kernel_math", "fft_tile_check.cpp")
    inc = os.path.join(HERE, "kernel_math")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-I", inc, src, "-o", exe], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("compile failed:\n" + r.stderr[-3000:])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert r.stdout.count("rel err") == 24
    assert r.stdout.count(" ok") == 15 + 9
    assert r.stdout.count("pair base") == 9
    assert r.stdout.count("two halves") == 11


def test_chain_tanh_accuracy(tmp_path):
    exe = str(tmp_path / "tanh_check")
    src = os.path.join(HERE, "kernel_math", "tanh_check.cpp")
    inc = os.path.join(HERE, "kernel_math")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-I", inc, src, "-o", exe], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("compile failed:\n" + r.stderr[-3000:])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
