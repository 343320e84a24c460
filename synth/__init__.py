"""Seeded synthetic input images (shared by the tests, the benchmark and the smoke
check).  The pictures are drawn by ``synth.c`` (C + OpenMP, built with gcc);
this module builds it and returns numpy arrays.  Nothing here labels anything.

The five workloads (shapes, dtypes and seeds) are those the labeller is measured
and parity-checked on; ``generate(k)`` returns workload k at its full size and
the ``*_image`` functions take explicit sizes for smaller cases with the same
recipe.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libccl_synth.so")
_lib = None

# workload id -> (description, shape [B, H, W], numpy dtype, seed)
CONFIGS = {
    1: ("drawing-256: 40 anti-aliased lines + 10 palette rectangles, u32", (1, 256, 256), np.uint32, 1),
    2: ("bernoulli-64x512: p from 0.05 to 0.95 across the batch, u8", (64, 512, 512), np.uint8, 2),
    3: ("spiral-4096: two interleaved 1-px spirals on a fringed background, u32", (1, 4096, 4096), np.uint32, 3),
    4: ("tissue-20000: blurred noise (sigma 6) thresholded at the 60th percentile, u8", (1, 20000, 20000), np.uint8, 7),
    5: ("sheet-33600x24000: synthetic construction drawing at 800 dpi, u32", (1, 24000, 33600), np.uint32, 5),
}


def build() -> str:
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    # no -march: the built library also runs on other hosts; no fast-math: the
    # float blur must round identically everywhere
    subprocess.run(["gcc", "-O3", "-std=gnu11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
                   check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, u64, vp, d = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double
        lib.synth_lines.argtypes = [vp, i64, i64, u64, ctypes.c_int, ctypes.c_int]
        lib.synth_bernoulli.argtypes = [vp, i64, i64, i64, u64, d, d]
        lib.synth_spiral.argtypes = [vp, i64, i64, u64]
        lib.synth_tissue.argtypes = [vp, i64, i64, u64, d, d]
        lib.synth_sheet.argtypes = [vp, i64, i64, u64, d]
        for f in (lib.synth_lines, lib.synth_bernoulli, lib.synth_spiral, lib.synth_tissue,
                  lib.synth_sheet):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} failed with status {rc}")


def _vp(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def lines_image(H=256, W=256, seed=1, nlines=40, nrects=10) -> np.ndarray:
    out = np.empty((H, W), np.uint32)
    _check(_load().synth_lines(_vp(out), H, W, seed, nlines, nrects), "synth_lines")
    return out


def bernoulli_batch(B=64, H=512, W=512, seed=2, p_lo=0.05, p_hi=0.95) -> np.ndarray:
    out = np.empty((B, H, W), np.uint8)
    _check(_load().synth_bernoulli(_vp(out), B, H, W, seed, p_lo, p_hi), "synth_bernoulli")
    return out


def spiral_image(H=4096, W=4096, seed=3) -> np.ndarray:
    out = np.empty((H, W), np.uint32)
    _check(_load().synth_spiral(_vp(out), H, W, seed), "synth_spiral")
    return out


def tissue_image(H=20000, W=20000, seed=7, sigma=6.0, quantile=0.6) -> np.ndarray:
    out = np.empty((H, W), np.uint8)
    _check(_load().synth_tissue(_vp(out), H, W, seed, sigma, quantile), "synth_tissue")
    return out


# The sheet's primitive counts (per 806.4 Mpx: 400 walls, 80 hatching fields,
# 300 bubbles, 200k glyphs) are scaled by this factor so that exact-white paper
# covers about 95% of the sheet, the share the every-colour page gives for a
# drawing (ch.08 "Making it fast").
SHEET_DENSITY = 0.45


def sheet_image(H=24000, W=33600, seed=5, density=SHEET_DENSITY) -> np.ndarray:
    out = np.empty((H, W), np.uint32)
    _check(_load().synth_sheet(_vp(out), H, W, seed, density), "synth_sheet")
    return out


def generate(config: int) -> np.ndarray:
    """Workload ``config`` (1..5) at full size, always as [B, H, W]."""
    _, (B, H, W), _, seed = CONFIGS[config]
    if config == 1:
        img = lines_image(H, W, seed)
    elif config == 2:
        return bernoulli_batch(B, H, W, seed)
    elif config == 3:
        img = spiral_image(H, W, seed)
    elif config == 4:
        img = tissue_image(H, W, seed)
    elif config == 5:
        img = sheet_image(H, W, seed)
    else:
        raise KeyError(config)
    return img[None]


def rgb24(img: np.ndarray) -> np.ndarray:
    """An 0x00RRGGBB picture (u32 [.., H, W]) stored as RGB bytes, uint8
    [.., H, W, 3] in the order R, G, B: the same picture, three bytes a pixel."""
    img = np.asarray(img, dtype=np.uint32)
    out = np.empty(img.shape + (3,), dtype=np.uint8)
    out[..., 0] = (img >> 16) & 0xFF
    out[..., 1] = (img >> 8) & 0xFF
    out[..., 2] = img & 0xFF
    return out


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()
