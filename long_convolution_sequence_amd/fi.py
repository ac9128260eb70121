"""Thin Python binding of the C-ABI in ``include/fi.h`` (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
library ``libfi.so``.  torch is used for device memory (workspace, inputs,
outputs) and for the current HIP stream.  There is no fallback: if the
library is missing or no GPU is present, construction raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfi.so")

FI_OK, FI_EINVAL, FI_ENOMEM, FI_EDEVICE, FI_ERANGE, FI_ESTATE = 0, -1, -2, -3, -4, -5
MAP_TANH, MAP_IDENTITY, MAP_EXTERNAL, MAP_HYENA = 0, 1, 2, 3
FEEDBACK_TANH, FEEDBACK_IDENTITY = 0, 1
TAU_AUTO, TAU_DIRECT, TAU_FFT = 0, 1, 2
PATH_NONE, PATH_DIRECT, PATH_FFT = 0, 1, 2
BASE_LAZY, BASE_EAGER, BASE_LAZY_NP, BASE_EAGER_NP = 0, 1, 2, 3
_STATUS = {0: "FI_OK", -1: "FI_EINVAL", -2: "FI_ENOMEM", -3: "FI_EDEVICE", -4: "FI_ERANGE",
           -5: "FI_ESTATE"}


class FiError(RuntimeError):
    def __init__(self, status, msg=""):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")


class Options(ctypes.Structure):
    _fields_ = [("map", ctypes.c_int), ("feedback", ctypes.c_int), ("tau_mode", ctypes.c_int),
                ("tau_split", ctypes.c_int), ("record", ctypes.c_int), ("use_graphs", ctypes.c_int),
                ("block_graph_log2", ctypes.c_int), ("filters_on_device", ctypes.c_int),
                ("fft_max_log2", ctypes.c_int), ("time_blocks", ctypes.c_int),
                ("defer_wide", ctypes.c_int), ("chunk_direct", ctypes.c_int), ("eager_prefill", ctypes.c_int),
                ("reserved", ctypes.c_int * 3)]


_lib = None


def load_library():
    """Load libfi.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FiError(FI_ESTATE, f"{LIB_PATH} is not built; run __graft_entry__.build()")
    try:
        import torch  # noqa: F401  (loads the HIP runtime the library binds to)
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    OP = ctypes.POINTER(Options)
    sig = {
        "fi_default_options": (None, [OP]),
        "fi_version": (ctypes.c_char_p, []),
        "fi_workspace_bytes": (S, [I, I, I, I64, OP]),
        "fi_init": (I, [ctypes.POINTER(P), I, I, I, I64, P, OP, P, P]),
        "fi_destroy": (I, [P]),
        "fi_reset": (I, [P]),
        "fi_set_defer_wide": (I, [P, I]),
        "fi_step": (I, [P, P, P]),
        "fi_set_input": (I, [P, P]),
        "fi_prefill": (I, [P, P, I64, P]),
        "fi_generate": (I, [P, I64, P]),
        "fi_position": (I64, [P]),
        "fi_last_error": (ctypes.c_char_p, [P]),
        "fi_debug_schedule": (I, [P, I64, ctypes.POINTER(I), ctypes.POINTER(I)]),
        "fi_tau_table": (I, [P, P, P, P]),
        "fi_history": (I, [P, I, I, I64, I64, P]),
        "fi_chunk_table": (I, [P, P, P]),
        "fi_stamps": (I, [P, I64, I64, P]),
        "fi_layer_red": (I, [P, I, P, P]),
        "fi_tiles": (I, [P]),
        "fi_lazy_step": (I, [P, P, P]),
        "fi_lazy_generate": (I, [P, I64, P]),
        "fi_block_times": (I, [P, I, P, P]),
        "fi_chunk_times": (I, [P, I, P, P]),
        "fi_baseline_step": (I, [P, I, P, P]),
        "fi_baseline_generate": (I, [P, I, I64, P]),
        "fi_baseline_time": (I, [P, I, I64, I, ctypes.POINTER(ctypes.c_double)]),
        "fi_set_block_weights": (I, [P, P, P, P, I]),
        "fi_set_block_weights_static": (I, [P, P, P, P, I]),
        "fi_lazy_time": (I, [P, I64, I, ctypes.POINTER(ctypes.c_double)]),
        "fi_time_block": (I, [P, I, I, I, ctypes.POINTER(ctypes.c_double)]),
        "fi_time_hyena_block": (I, [P, I, ctypes.POINTER(ctypes.c_double)]),
        "fi_dd_workspace_bytes": (S, [I, I, I64, I]),
        "fi_dd_init": (I, [ctypes.POINTER(P), I, I, I64, I, P, P]),
        "fi_dd_stack_workspace_bytes": (S, [I, I, I, I64, I]),
        "fi_dd_stack_init": (I, [ctypes.POINTER(P), I, I, I, I64, I, P, P]),
        "fi_dd_step": (I, [P, P, P, P]),
        "fi_dd_run": (I, [P, P, P, I64, P]),
        "fi_dd_reset": (I, [P]),
        "fi_dd_position": (I64, [P]),
        "fi_dd_last_error": (ctypes.c_char_p, [P]),
        "fi_dd_destroy": (I, [P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def default_options() -> Options:
    o = Options()
    load_library().fi_default_options(ctypes.byref(o))
    return o


def workspace_bytes(M, B, D, L, opt: Options | None = None) -> int:
    return int(load_library().fi_workspace_bytes(M, B, D, L, ctypes.byref(opt) if opt else None))


def _dptr(t, shape=None, device=None, name="tensor", dtypes=None):
    """Device pointer of a tensor (None passes through), after checking that it
    is a contiguous tensor on ``device`` with the dtype and exact shape the C
    call will read or write.  A mismatch raises FiError(FI_EINVAL) instead of
    letting a kernel run past the buffer."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise FiError(FI_EINVAL, f"{name}: expected a torch tensor, got {type(t).__name__}")
    ok = dtypes or (torch.float32,)
    if t.dtype not in ok:
        raise FiError(FI_EINVAL, f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in ok)}")
    if not t.is_cuda:
        raise FiError(FI_EINVAL, f"{name}: not a device tensor")
    if device is not None and t.device != device:
        raise FiError(FI_EINVAL, f"{name}: on {t.device}, the context is on {device}")
    if not t.is_contiguous():
        raise FiError(FI_EINVAL, f"{name}: not contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise FiError(FI_EINVAL, f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


class Context:
    """One fi_ctx bound to the current torch stream.

    filters: fp32 [M][D][L], a CUDA tensor (copied device to device) or a
    numpy array (copied from host).  Keyword options map to ``fi_options``.
    """

    def __init__(self, filters, batch, *, map=MAP_TANH, feedback=FEEDBACK_TANH, tau_mode=TAU_AUTO,
                 tau_split=-1, record=False, use_graphs=True, block_graph_log2=6, fft_max_log2=14,
                 time_blocks=False, defer_wide=False, chunk_direct=True, eager_prefill=True, device=None):
        import torch
        if not torch.cuda.is_available():
            raise FiError(FI_EDEVICE, "no GPU visible; the library has no CPU path")
        lib = load_library()
        self._torch = torch
        self.device = torch.device(device or "cuda")
        opt = default_options()
        opt.map, opt.feedback, opt.tau_mode, opt.tau_split = map, feedback, tau_mode, tau_split
        opt.record, opt.use_graphs, opt.block_graph_log2 = int(record), int(use_graphs), block_graph_log2
        opt.fft_max_log2 = fft_max_log2
        opt.time_blocks = int(time_blocks)
        opt.defer_wide = int(defer_wide)
        opt.chunk_direct = int(chunk_direct)
        opt.eager_prefill = int(eager_prefill)
        if getattr(filters, "ndim", 0) != 3:
            raise FiError(FI_EINVAL, "filters: expected an fp32 [M][D][L] array or tensor")
        if isinstance(filters, np.ndarray):
            f = np.ascontiguousarray(filters, dtype=np.float32)
            fptr = f.ctypes.data_as(ctypes.c_void_p)
            opt.filters_on_device = 0
            keep = f
        else:
            keep = filters.to(self.device, torch.float32).contiguous()
            fptr = ctypes.c_void_p(keep.data_ptr())
            opt.filters_on_device = 1
        M, D, L = (int(s) for s in filters.shape)
        self.M, self.B, self.D, self.L = M, int(batch), D, L
        self.P = L.bit_length() - 1
        nbytes = lib.fi_workspace_bytes(M, self.B, D, L, ctypes.byref(opt))
        if nbytes == 0:
            raise FiError(FI_EINVAL, f"unsupported shape M={M} B={batch} D={D} L={L}")
        self.workspace = torch.empty(int(nbytes), dtype=torch.uint8, device=self.device)
        self.stream = torch.cuda.current_stream(self.device)
        h = ctypes.c_void_p()
        st = lib.fi_init(ctypes.byref(h), M, self.B, D, L, fptr, ctypes.byref(opt),
                         ctypes.c_void_p(self.workspace.data_ptr()),
                         ctypes.c_void_p(self.stream.cuda_stream))
        del keep
        if st != FI_OK:
            raise FiError(st, "fi_init failed")
        self._h = h
        self._lib = lib
        self.options = opt

    # -- helpers ------------------------------------------------------------
    def _check(self, st):
        if st != FI_OK:
            msg = self._lib.fi_last_error(self._h)
            raise FiError(st, msg.decode() if msg else "")

    def _bd(self, lead=()):
        return self._torch.empty(tuple(lead) + (self.B, self.D), dtype=self._torch.float32,
                                 device=self.device)

    def _p(self, t, lead=(), name="tensor"):
        """Checked device pointer of an fp32 [*lead][B][D] tensor (or None)."""
        dev = self.device if self.device.index is not None else None
        p = _dptr(t, tuple(lead) + (self.B, self.D), dev, name)
        if t is not None and dev is None and t.device.index != self._torch.cuda.current_device():
            raise FiError(FI_EINVAL, f"{name}: on {t.device}, the context is on the current device")
        return p

    # -- API ----------------------------------------------------------------
    @property
    def position(self) -> int:
        return int(self._lib.fi_position(self._h))

    def set_input(self, x0):
        if x0 is None:
            raise FiError(FI_EINVAL, "x0: required")
        self._check(self._lib.fi_set_input(self._h, self._p(x0, name="x0")))

    def set_defer_wide(self, level):
        """Defer the later sub-blocks of wide gray blocks to a second stream: 0 off,
        1 (or True) the split classes, 2 the two-half class too (the context must
        have been made with defer_wide=2)."""
        self._check(self._lib.fi_set_defer_wide(self._h, int(level)))

    def step(self, x=None, y=None):
        """One position; x: [B][D] device tensor or None (feedback). Returns y [B][D]."""
        y = self._bd() if y is None else y
        self._check(self._lib.fi_step(self._h, self._p(x, name="x"), self._p(y, name="y")))
        return y

    def prefill(self, x, y=None, want_y=True):
        if x is None or getattr(x, "ndim", 0) != 3:
            raise FiError(FI_EINVAL, "x: expected a [P][B][D] device tensor")
        P = int(x.shape[0])
        if want_y and y is None:
            y = self._bd((P,))
        self._check(self._lib.fi_prefill(self._h, self._p(x, (P,), "x"), P, self._p(y, (P,), "y")))
        return y

    def generate(self, steps, y=None, want_y=True):
        steps = int(steps)
        if want_y and y is None:
            y = self._bd((steps,))
        self._check(self._lib.fi_generate(self._h, steps, self._p(y, (steps,), "y")))
        return y

    def lazy_step(self, x=None, y=None):
        y = self._bd() if y is None else y
        self._check(self._lib.fi_lazy_step(self._h, self._p(x, name="x"), self._p(y, name="y")))
        return y

    def lazy_generate(self, steps, y=None, want_y=True):
        steps = int(steps)
        if want_y and y is None:
            y = self._bd((steps,))
        self._check(self._lib.fi_lazy_generate(self._h, steps, self._p(y, (steps,), "y")))
        return y

    def baseline_step(self, kind, x=None, y=None):
        y = self._bd() if y is None else y
        self._check(self._lib.fi_baseline_step(self._h, int(kind), self._p(x, name="x"), self._p(y, name="y")))
        return y

    def baseline_generate(self, kind, steps, y=None, want_y=True):
        steps = int(steps)
        if want_y and y is None:
            y = self._bd((steps,))
        self._check(self._lib.fi_baseline_generate(self._h, int(kind), steps, self._p(y, (steps,), "y")))
        return y

    def layer_red(self, layer, q, y=None):
        y = self._bd() if y is None else y
        if q is None:
            raise FiError(FI_EINVAL, "q: required")
        self._check(self._lib.fi_layer_red(self._h, int(layer), self._p(q, name="q"), self._p(y, name="y")))
        return y

    def tiles(self):
        self._check(self._lib.fi_tiles(self._h))

    def set_block_weights_static(self, W, W1, W2):
        """set_block_weights staged through the library's fixed device array (fi_set_block_weights_static:
        no device allocation; D <= 1024)."""
        self.set_block_weights(W, W1, W2, _fn="fi_set_block_weights_static")

    def set_block_weights(self, W, W1, W2, _fn="fi_set_block_weights"):
        """Hyena-style block weights as bf16 bit patterns (uint16 numpy arrays or int16/uint16
        device tensors): W [M][D][3D], W1 [M][D][4D], W2 [M][4D][D] (row-major x*W)."""
        if isinstance(W, np.ndarray):
            arrs = [np.ascontiguousarray(a, dtype=np.uint16) for a in (W, W1, W2)]
            M, D = self.M, self.D
            for a, shp, nm in zip(arrs, ((M, D, 3 * D), (M, D, 4 * D), (M, 4 * D, D)), ("W", "W1", "W2")):
                if a.shape != shp:
                    raise FiError(FI_EINVAL, f"{nm}: shape {a.shape}, expected {shp}")
            ptrs = [a.ctypes.data_as(ctypes.c_void_p) for a in arrs]
            on_dev = 0
        else:
            import torch
            M, D = self.M, self.D
            shapes = ((M, D, 3 * D), (M, D, 4 * D), (M, 4 * D, D))
            arrs = [a.contiguous() for a in (W, W1, W2)]
            ptrs = [_dptr(a, shp, None, nm, (torch.int16, torch.uint16, torch.bfloat16))
                    for a, shp, nm in zip(arrs, shapes, ("W", "W1", "W2"))]
            on_dev = 1
        self._check(getattr(self._lib, _fn)(self._h, *ptrs, on_dev))

    def history(self, layer, what, count=None, first=1):
        """[count][B][D] device tensor of positions first.. : what=0 layer (convolution) inputs,
        1 mixer outputs, 2 block outputs (Hyena-style block mode)."""
        count = self.position - first + 1 if count is None else count
        dst = self._torch.empty((max(count, 1), self.B, self.D), dtype=self._torch.float32,
                                device=self.device)[:count]
        self._check(self._lib.fi_history(self._h, int(layer), int(what), int(first), int(count),
                                         ctypes.c_void_p(dst.data_ptr())))
        return dst

    def stamps(self, first, count):
        out = np.zeros(count, dtype=np.int64)
        self._check(self._lib.fi_stamps(self._h, int(first), int(count),
                                        out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def tau_table(self):
        P = max(self.P, 1)
        path = (ctypes.c_int * P)()
        ud = (ctypes.c_double * P)()
        uf = (ctypes.c_double * P)()
        self._check(self._lib.fi_tau_table(self._h, path, ud, uf))
        return [(q, path[q], ud[q], uf[q]) for q in range(self.P)]

    def chunk_table(self):
        """Chunk-path calibration per candidate first FFT class g: (g, us of one chunk + its FFT block,
        modeled us of a run); -1 where not timed."""
        n = self.P + 1
        uc = (ctypes.c_double * n)()
        ur = (ctypes.c_double * n)()
        self._check(self._lib.fi_chunk_table(self._h, uc, ur))
        return [(g, uc[g], ur[g]) for g in range(n)]

    def block_times(self, clear=False):
        """Per class q: (summed FFT gray-block ms, launches) measured with HIP events."""
        P = max(self.P, 1)
        ms = (ctypes.c_double * P)()
        cnt = (ctypes.c_int64 * P)()
        self._check(self._lib.fi_block_times(self._h, int(clear), ms, cnt))
        return [(q, ms[q], cnt[q]) for q in range(self.P)]

    def chunk_times(self, clear=False):
        """(summed chunk-kernel ms, launches) measured with HIP events (time_blocks contexts)."""
        ms = ctypes.c_double()
        cnt = ctypes.c_int64()
        self._check(self._lib.fi_chunk_times(self._h, int(clear), ctypes.byref(ms), ctypes.byref(cnt)))
        return ms.value, cnt.value

    def time_block(self, q, path, reps=10):
        """Mean microseconds of class q's gray-block kernels on one path (needs reset after)."""
        us = ctypes.c_double()
        self._check(self._lib.fi_time_block(self._h, int(q), int(path), int(reps), ctypes.byref(us)))
        return us.value

    def time_hyena_block(self, reps=10):
        """Mean microseconds of one position's block kernels (Hyena-style block mode; needs reset after)."""
        us = ctypes.c_double()
        self._check(self._lib.fi_time_hyena_block(self._h, int(reps), ctypes.byref(us)))
        return us.value

    def lazy_time(self, n, reps=3):
        """Mean microseconds of the Lazy baseline's work at position n (needs reset after)."""
        us = ctypes.c_double()
        self._check(self._lib.fi_lazy_time(self._h, int(n), int(reps), ctypes.byref(us)))
        return us.value

    def baseline_time(self, kind, n, reps=3):
        """Mean microseconds of one baseline position n of the given kind (needs reset after)."""
        us = ctypes.c_double()
        self._check(self._lib.fi_baseline_time(self._h, int(kind), int(n), int(reps), ctypes.byref(us)))
        return us.value

    def schedule(self, n):
        q, pth = ctypes.c_int(), ctypes.c_int()
        self._check(self._lib.fi_debug_schedule(self._h, int(n), ctypes.byref(q), ctypes.byref(pth)))
        return q.value, pth.value

    def reset(self):
        self._check(self._lib.fi_reset(self._h))

    def close(self):
        if getattr(self, "_h", None):
            self._lib.fi_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()


class DDContext:
    """Data-dependent filters: per position both the input x_t and the filter tap h_t arrive
    ([B][D] each, one layer, taps per (b, c)) and y_t = sum_{i+j=t} x_i h_j is produced.
    layers=M makes a stack (fi_dd_stack_*): x_t [B][D] is layer 0's input, h_t and y_t are
    [M][B][D], and layer l+1's input is tanh(y^l_t).  Wraps the fi_dd_* calls (see
    include/fi.h); no CPU path."""

    def __init__(self, batch, channels, L, *, fft_min_log2=-1, layers=None, device=None):
        import torch
        if not torch.cuda.is_available():
            raise FiError(FI_EDEVICE, "no GPU visible; the library has no CPU path")
        lib = load_library()
        self._torch = torch
        self.device = torch.device(device or "cuda")
        self.B, self.D, self.L = int(batch), int(channels), int(L)
        self.M = None if layers is None else int(layers)
        if self.M is None:
            nbytes = lib.fi_dd_workspace_bytes(self.B, self.D, self.L, int(fft_min_log2))
        else:
            nbytes = lib.fi_dd_stack_workspace_bytes(self.M, self.B, self.D, self.L, int(fft_min_log2))
        if nbytes == 0:
            raise FiError(FI_EINVAL, f"unsupported shape M={layers} B={batch} D={channels} L={L}")
        self.workspace = torch.empty(int(nbytes), dtype=torch.uint8, device=self.device)
        self.stream = torch.cuda.current_stream(self.device)
        h = ctypes.c_void_p()
        ws, strm = ctypes.c_void_p(self.workspace.data_ptr()), ctypes.c_void_p(self.stream.cuda_stream)
        if self.M is None:
            st = lib.fi_dd_init(ctypes.byref(h), self.B, self.D, self.L, int(fft_min_log2), ws, strm)
        else:
            st = lib.fi_dd_stack_init(ctypes.byref(h), self.M, self.B, self.D, self.L, int(fft_min_log2), ws, strm)
        if st != FI_OK:
            raise FiError(st, "fi_dd_init failed")
        self._h = h
        self._lib = lib

    def _check(self, st):
        if st != FI_OK:
            msg = self._lib.fi_dd_last_error(self._h)
            raise FiError(st, msg.decode() if msg else "")

    def _p(self, t, shape, name):
        dev = self.device if self.device.index is not None else None
        p = _dptr(t, shape, dev, name)
        if t is not None and dev is None and t.device.index != self._torch.cuda.current_device():
            raise FiError(FI_EINVAL, f"{name}: on {t.device}, the context is on the current device")
        return p

    @property
    def position(self) -> int:
        return int(self._lib.fi_dd_position(self._h))

    def _layer_shape(self):
        return (self.B, self.D) if self.M is None else (self.M, self.B, self.D)

    def step(self, x, h, y=None):
        """One position: x [B][D], h [B][D] (a stack: [M][B][D]) device tensors; returns y
        shaped like h."""
        ls = self._layer_shape()
        y = self._torch.empty(ls, dtype=self._torch.float32, device=self.device) if y is None else y
        if x is None or h is None:
            raise FiError(FI_EINVAL, "x and h are required")
        self._check(self._lib.fi_dd_step(self._h, self._p(x, (self.B, self.D), "x"), self._p(h, ls, "h"),
                                         self._p(y, ls, "y")))
        return y

    def run(self, x, h, y=None):
        """len(x) positions: x [T][B][D], h [T][B][D] (a stack: [T][M][B][D]) device tensors;
        returns y shaped like h."""
        if x is None or h is None or getattr(x, "ndim", 0) != 3:
            raise FiError(FI_EINVAL, "x and h: expected [T][B][D] (h of a stack [T][M][B][D]) device tensors")
        T = int(x.shape[0])
        hs = (T,) + self._layer_shape()
        y = self._torch.empty(hs, dtype=self._torch.float32, device=self.device) if y is None else y
        self._check(self._lib.fi_dd_run(self._h, self._p(x, (T, self.B, self.D), "x"), self._p(h, hs, "h"), T,
                                        self._p(y, hs, "y")))
        return y

    def reset(self):
        self._check(self._lib.fi_dd_reset(self._h))

    def close(self):
        if getattr(self, "_h", None):
            self._lib.fi_dd_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()
