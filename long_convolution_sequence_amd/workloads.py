"""Seeded synthetic inputs for the mixer workloads.

This module only draws random numbers and shapes them; it holds none of the
convolution's arithmetic.  Both the GPU path's tests and the CPU oracle's
checks take their inputs from here, so every comparison runs on identical fp32
arrays.

The pages (Flash Inference, arXiv 2410.12982, summary page, "Experimentelle
Einrichtung" and "Schwaechen") use randomly initialised weights only; there is
no dataset or checkpoint to stand in for.  Shapes follow the pages' sweep
(B in {1,2,4,8}, M in {18,36}, D in {256,768,864}, L = 2^15..2^18) and its
largest mixer shape (B=1, M=18, D=864, L=2^17, "Hauptergebnisse").

Recipe (stated once, used everywhere):
* every random row has its own ``numpy.random.SeedSequence([seed, tag, ...])``
  so any subset of rows can be regenerated without drawing the others;
* filters: ``h^l[c][k] = g * exp(-k / decay) * scale`` with g ~ N(0,1), the
  product formed in fp64 and rounded once to fp32;
* first input x^0_1 ~ N(0,1) per (b, c); teacher-forced inputs ~ N(0,1);
* block weights ~ N(0, 0.02) rounded to bfloat16 (round to nearest even).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TAG_FILTER, TAG_X0, TAG_XTF, TAG_W = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    B: int
    D: int
    L: int
    decay: float
    scale: float = 1.0
    block: str = "tanh"          # "tanh": elementwise tanh map; "hyena": projection/MLP block
    teacher_forced: bool = False  # also run with given inputs
    seed: int = 1000
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def P(self) -> int:
        return int(math.log2(self.L))


WORKLOADS = {
    1: Workload("stack M=1 B=1 D=4 L=2^10", 1, 1, 4, 1024, 256.0, seed=1001),
    2: Workload("stack M=1 B=1 D=256 L=2^14", 1, 1, 256, 16384, 2048.0, teacher_forced=True,
                seed=1002),
    3: Workload("stack M=18 B=4 D=768 L=2^15", 18, 4, 768, 32768, 32768 / 8.0, seed=1003),
    4: Workload("stack M=18 B=1 D=864 L=2^17", 18, 1, 864, 131072, 16384.0,
                scale=1.0 / math.sqrt(131072.0), seed=1004),
    5: Workload("hyena M=18 B=4 D=768 L=2^15", 18, 4, 768, 32768, 32768 / 8.0, block="hyena",
                seed=1005),
}


def custom(M, B, D, L, decay, scale=1.0, seed=7, block="tanh", name=None) -> Workload:
    """A workload of arbitrary (small) shape with the same recipe, for tests."""
    return Workload(name or f"custom M={M} B={B} D={D} L={L}", M, B, D, L, float(decay),
                    float(scale), block=block, seed=seed)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def filter_row(w: Workload, layer: int, chan: int) -> np.ndarray:
    """One filter row h^layer[chan][0..L-1] as fp32."""
    g = _rng(w.seed, TAG_FILTER, layer, chan).standard_normal(w.L)
    k = np.arange(w.L, dtype=np.float64)
    return (g * np.exp(-k / w.decay) * w.scale).astype(np.float32)


def filters(w: Workload, layers=None, chans=None, threads: int = 8) -> np.ndarray:
    """Filters ``[len(layers)][len(chans)][L]`` fp32 (all rows by default)."""
    layers = list(range(w.M)) if layers is None else list(layers)
    chans = list(range(w.D)) if chans is None else list(chans)
    out = np.empty((len(layers), len(chans), w.L), dtype=np.float32)
    k = np.arange(w.L, dtype=np.float64)
    env = np.exp(-k / w.decay) * w.scale

    def fill(i):
        for j, c in enumerate(chans):
            g = _rng(w.seed, TAG_FILTER, layers[i], c).standard_normal(w.L)
            out[i, j] = (g * env).astype(np.float32)

    if len(layers) * len(chans) > 64 and threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(len(layers))))
    else:
        for i in range(len(layers)):
            fill(i)
    return out


def x_first(w: Workload) -> np.ndarray:
    """Layer-0 input at the first position, ``[B][D]`` fp32, N(0,1)."""
    return _rng(w.seed, TAG_X0).standard_normal((w.B, w.D)).astype(np.float32)


def x_teacher(w: Workload, steps=None, batch=None, chans=None) -> np.ndarray:
    """Teacher-forced layer-0 inputs ``[steps][len(batch)][len(chans)]`` fp32, N(0,1).

    Each (b, c) sequence has its own seed, so sampled channels can be rebuilt alone.
    """
    steps = w.L if steps is None else steps
    batch = list(range(w.B)) if batch is None else list(batch)
    chans = list(range(w.D)) if chans is None else list(chans)
    out = np.empty((steps, len(batch), len(chans)), dtype=np.float32)
    for i, b in enumerate(batch):
        for j, c in enumerate(chans):
            out[:, i, j] = _rng(w.seed, TAG_XTF, b, c).standard_normal(w.L)[:steps]
    return out


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest even); return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def hyena_weights(w: Workload) -> dict:
    """Per-layer block weights as bf16 bit patterns (``uint16``):
    ``W [M][D][3D]``, ``W1 [M][D][4D]``, ``W2 [M][4D][D]``, all N(0, 0.02)."""
    D = w.D
    shapes = {"W": (D, 3 * D), "W1": (D, 4 * D), "W2": (4 * D, D)}
    out = {}
    for idx, (key, shp) in enumerate(shapes.items()):
        arr = np.empty((w.M,) + shp, dtype=np.uint16)
        for l in range(w.M):
            g = _rng(w.seed, TAG_W, l, idx).standard_normal(shp) * 0.02
            arr[l] = to_bf16_bits(g.astype(np.float32))
        out[key] = arr
    return out
