"""CPU oracle for exact autoregressive causal long convolution.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, loads or calls this package; only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg do.  It shares
no code, constants, tables or helpers with the GPU path.

What it computes (Flash Inference, arXiv 2410.12982; the summary page's
"Aufgabendefinition", "LCSM-spezifische Definition" and Algorithm 2 in
"LCSM-Inferenz-Algorithmus"):

* ``conv_rows`` / ``conv_points`` -- the causal convolution
  ``y_t = sum_{s<=t} h_{t-s} x_s`` per channel, summed in fp64 in C
  (``naive.c``).  This is the definition itself; the method is exact, so the
  GPU's tiled result must equal it up to rounding.
* ``stack`` -- the autoregressive mixer stack: per position, layers in order,
  ``x^{l+1}_t = tanh(y^l_t)`` between layers, and the next layer-0 input either
  given (teacher forcing) or ``tanh(y^{M-1}_t)`` (feedback), fp64 throughout.
* ``stack_f32`` -- the same loop in fp32, used only to measure the divergence
  horizon of feedback runs (how far two correct evaluations that round
  differently stay within tolerance).
* ``schedule`` -- the relaxed tiling enumerated from Algorithm 1 ("Kachelung-
  Strategie"), for coverage and counting pins.
* ``relaxed`` -- Algorithm 1 evaluated tile by tile in fp64 numpy (direct and
  circular-FFT tiles); a pin aid showing the tiling reproduces the definition.
* ``block`` -- the Hyena-style block of the 18-layer B=4 D=768 workload in fp64
  numpy (projection, gate, GELU MLP, RMSNorm).

Every function states the passage it follows.  See ``tests/test_oracle_*.py``
for the pins that tie each function to something other than itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "naive.c")
_LIB_PATH = os.path.join(_HERE, "_liborc.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``naive.c`` into ``_liborc.so`` with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.orc_num_threads.restype = ci
        lib.orc_conv_rows.argtypes = [P, i64, P, i64, i64, i64, P]
        lib.orc_conv_points.argtypes = [P, P, P, i64, P]
        lib.orc_stack.argtypes = [ci, ci, i64, P, ci, P, P, P, ci, ci, i64, P, P]
        lib.orc_stack_f32.argtypes = [ci, ci, i64, P, ci, P, P, ci, ci, i64, P, P]
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the C oracle runs with."""
    return int(_load().orc_num_threads())


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def conv_rows(h, x) -> np.ndarray:
    """Causal convolution of matching rows: ``out[r, t] = sum_{s<=t} h[r, t-s] x[r, s]``.

    ``h`` and ``x`` are fp32 ``[rows, L]`` (or 1-D); result fp64 ``[rows, L]``.
    Definition from "Aufgabendefinition" (0-based storage of the 1-based sum).
    """
    h = _f32(h)
    x = _f32(x)
    one = h.ndim == 1
    if one:
        h, x = h[None], x[None]
    assert h.shape == x.shape and h.ndim == 2
    rows, L = h.shape
    out = np.empty((rows, L), dtype=np.float64)
    _load().orc_conv_rows(_ptr(h), L, _ptr(x), L, rows, L, _ptr(out))
    return out[0] if one else out


def conv_points(h, x, ts) -> np.ndarray:
    """``out[k] = sum_{s<=ts[k]} h[ts[k]-s] x[s]`` for one row, fp64 (same definition)."""
    h = _f32(h)
    x = _f32(x)
    ts = np.ascontiguousarray(ts, dtype=np.int64)
    assert h.ndim == 1 and x.ndim == 1 and h.shape == x.shape
    if ts.size:
        assert ts.min() >= 0 and ts.max() < h.shape[0]
    out = np.empty(ts.shape[0], dtype=np.float64)
    _load().orc_conv_points(_ptr(h), _ptr(x), _ptr(ts), ts.shape[0], _ptr(out))
    return out


def stack(filters, chans, x_first, steps, x_given=None, map_tanh=True, fb_tanh=True):
    """Autoregressive mixer stack for independent chains (Algorithm 2 with
    elementwise tanh block and tanh sampler), fp64.

    filters : fp32 ``[M, D, L]``; chans : channel of each chain ``[nch]``;
    x_first : layer-0 input at the first position ``[nch]``;
    x_given : ``[nch, steps]`` teacher-forced layer-0 inputs, or None (feedback).
    Returns ``(y, x)`` fp64 ``[nch, M, steps]``: mixer output and layer input.
    """
    filters = _f32(filters)
    M, D, L = filters.shape
    chans = np.ascontiguousarray(chans, dtype=np.int32)
    nch = chans.shape[0]
    assert steps <= L and chans.min() >= 0 and chans.max() < D
    x_first = _f32(x_first).reshape(nch)
    xg = None
    if x_given is not None:
        xg = _f32(x_given).reshape(nch, steps)
    ys = np.empty((nch, M, steps), dtype=np.float64)
    xs = np.empty((nch, M, steps), dtype=np.float64)
    _load().orc_stack(M, D, L, _ptr(filters), nch, _ptr(chans), _ptr(x_first),
                      _ptr(xg) if xg is not None else None, int(map_tanh), int(fb_tanh),
                      steps, _ptr(ys), _ptr(xs))
    return ys, xs


def stack_f32(filters, chans, x_first, steps, map_tanh=True, fb_tanh=True):
    """Feedback stack evaluated in fp32 with the same loop order (divergence
    horizon measurement only).  Returns ``(y, x)`` fp32 ``[nch, M, steps]``."""
    filters = _f32(filters)
    M, D, L = filters.shape
    chans = np.ascontiguousarray(chans, dtype=np.int32)
    nch = chans.shape[0]
    x_first = _f32(x_first).reshape(nch)
    ys = np.empty((nch, M, steps), dtype=np.float32)
    xs = np.empty((nch, M, steps), dtype=np.float32)
    _load().orc_stack_f32(M, D, L, _ptr(filters), nch, _ptr(chans), _ptr(x_first),
                          int(map_tanh), int(fb_tanh), steps, _ptr(ys), _ptr(xs))
    return ys, xs
