"""CPU oracle for connected-component labelling -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, loads or calls it.

The arithmetic lives in ``ccl_oracle.c`` (plain sequential C, built with gcc);
this module only builds that file and marshals numpy arrays to it.  See the C
file's header for what each function computes and which passages of the pages
it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ccl_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libccl_oracle.so")

_lib = None


def build(mutant: int = 0, out_path: str | None = None) -> str:
    """Compile the oracle with gcc; ``mutant`` > 0 plants a known mistake
    (used only by the tests that show the pins catch it)."""
    if out_path is None:
        if mutant:
            out_path = os.path.join(tempfile.mkdtemp(prefix="ccl_oracle_m"),
                                    f"libccl_oracle_m{mutant}.so")
        else:
            out_path = _LIB_PATH
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = out_path + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", f"-DORACLE_MUTANT={int(mutant)}",
           "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def _bind(lib):
    i64, i32p, vp = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p
    for name in ("oracle_label", "oracle_connect", "oracle_bfs_label"):
        f = getattr(lib, name)
        f.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, i32p]
        f.restype = ctypes.c_int
    lib.oracle_label_ignore.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int,
                                        ctypes.c_uint32, i32p]
    lib.oracle_label_ignore.restype = ctypes.c_int
    lib.oracle_number.argtypes = [i32p, i64, i64, i64, i32p, i32p]
    lib.oracle_number.restype = ctypes.c_int
    lib.oracle_count.argtypes = [i32p, i64, i64, i64, i32p]
    lib.oracle_count.restype = ctypes.c_int
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_label64.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_uint32, i64p]
    lib.oracle_label64.restype = ctypes.c_int
    lib.oracle_number64.argtypes = [i64p, i64, i64, i64, i64p, i64p]
    lib.oracle_number64.restype = ctypes.c_int
    lib.oracle_region_stats.argtypes = [i32p, i64, i64, i64, i32p, i32p, i32p, i64p, i64p]
    lib.oracle_region_stats.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the built oracle (building it first if nothing is built)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _as_batch(img: np.ndarray, rgb: bool = False):
    """(contiguous [B, H, W] or [B, H, W, 3] array, dtype code, squeezed?)."""
    img = np.asarray(img)
    if rgb:
        if img.dtype != np.uint8 or img.shape[-1:] != (3,):
            raise TypeError("an RGB picture is uint8 with a last dimension of 3")
        squeeze = img.ndim == 3
        if squeeze:
            img = img[None]
        if img.ndim != 4:
            raise ValueError("RGB picture must be [H, W, 3] or [B, H, W, 3]")
        return np.ascontiguousarray(img), 3, squeeze
    squeeze = img.ndim == 2
    if squeeze:
        img = img[None]
    if img.ndim != 3:
        raise ValueError("image must be [H, W] or [B, H, W]")
    if img.dtype == np.uint8:
        dtype = 1
    elif img.dtype in (np.uint32, np.int32):
        dtype = 4
    else:
        raise TypeError(f"unsupported dtype {img.dtype}")
    return np.ascontiguousarray(img), dtype, squeeze


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _run_labeller(fname: str, img, connectivity: int, lib, *extra, rgb: bool = False):
    img, dtype, squeeze = _as_batch(img, rgb)
    B, H, W = img.shape[:3]
    out = np.empty((B, H, W), dtype=np.int32)
    rc = getattr(lib, fname)(img.ctypes.data_as(ctypes.c_void_p), dtype, B, H, W,
                             int(connectivity), *extra, _ptr(out))
    if rc != 0:
        raise ValueError(f"{fname} failed with status {rc}")
    return out[0] if squeeze else out


def label(img, connectivity: int = 8, lib=None, ignore=None, rgb: bool = False) -> np.ndarray:
    """Leader image: each pixel's region minimum reading-order index (per image).
    With ``ignore`` set, pixels of that colour get -1 and join nothing.  With
    ``rgb``, ``img`` is uint8 [.., H, W, 3] and all three bytes are compared."""
    if ignore is None:
        return _run_labeller("oracle_label", img, connectivity, lib or load(), rgb=rgb)
    return _run_labeller("oracle_label_ignore", img, connectivity, lib or load(),
                         ctypes.c_uint32(int(ignore) & 0xFFFFFFFF), rgb=rgb)


def label64(img, connectivity: int = 8, lib=None, ignore=None, rgb: bool = False) -> np.ndarray:
    """As ``label``, with int64 leaders: for images of any size, also beyond
    2^31 pixels."""
    lib = lib or load()
    img, dtype, squeeze = _as_batch(img, rgb)
    B, H, W = img.shape[:3]
    out = np.empty((B, H, W), dtype=np.int64)
    ign = ignore is not None
    rc = lib.oracle_label64(img.ctypes.data_as(ctypes.c_void_p), dtype, B, H, W,
                            int(connectivity), int(ign),
                            ctypes.c_uint32(int(ignore) & 0xFFFFFFFF if ign else 0),
                            out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    if rc != 0:
        raise ValueError(f"oracle_label64 failed with status {rc}")
    return out[0] if squeeze else out


def number64(leaders, lib=None):
    """As ``number``, on int64 leaders: (int64 labels, int64 counts)."""
    lib = lib or load()
    L = np.ascontiguousarray(np.asarray(leaders, dtype=np.int64))
    squeeze = L.ndim == 2
    if squeeze:
        L = L[None]
    B, H, W = L.shape
    out = np.empty_like(L)
    counts = np.empty(B, dtype=np.int64)
    i64p = ctypes.POINTER(ctypes.c_int64)
    rc = lib.oracle_number64(L.ctypes.data_as(i64p), B, H, W, out.ctypes.data_as(i64p),
                             counts.ctypes.data_as(i64p))
    if rc != 0:
        raise ValueError(f"oracle_number64 failed with status {rc}")
    return (out[0], counts) if squeeze else (out, counts)


def connect(img, connectivity: int = 8, lib=None, rgb: bool = False) -> np.ndarray:
    """Parent array after the Start and Connect stages (before Collapse)."""
    return _run_labeller("oracle_connect", img, connectivity, lib or load(), rgb=rgb)


def bfs_label(img, connectivity: int = 8, lib=None, rgb: bool = False) -> np.ndarray:
    """Independent breadth-first flood-fill labeller (leader = seed index)."""
    return _run_labeller("oracle_bfs_label", img, connectivity, lib or load(), rgb=rgb)


def number(leaders, lib=None):
    """(labels 1..n in reading order, counts per image) from a leader image;
    pixels with a negative leader (ignored) get 0 and are not counted."""
    lib = lib or load()
    L = np.ascontiguousarray(np.asarray(leaders, dtype=np.int32))
    squeeze = L.ndim == 2
    if squeeze:
        L = L[None]
    B, H, W = L.shape
    out = np.empty_like(L)
    counts = np.empty(B, dtype=np.int32)
    rc = lib.oracle_number(_ptr(L), B, H, W, _ptr(out), _ptr(counts))
    if rc != 0:
        raise ValueError(f"oracle_number failed with status {rc}")
    return (out[0], counts) if squeeze else (out, counts)


def count(leaders, lib=None) -> np.ndarray:
    """Number of leaders per image."""
    lib = lib or load()
    L = np.ascontiguousarray(np.asarray(leaders, dtype=np.int32))
    if L.ndim == 2:
        L = L[None]
    B, H, W = L.shape
    counts = np.empty(B, dtype=np.int32)
    rc = lib.oracle_count(_ptr(L), B, H, W, _ptr(counts))
    if rc != 0:
        raise ValueError(f"oracle_count failed with status {rc}")
    return counts


def label_and_number(img, connectivity: int = 8, lib=None, ignore=None, rgb: bool = False):
    """(leaders, labels, counts): the whole path as the oracle computes it."""
    lib = lib or load()
    leaders = label(img, connectivity, lib, ignore=ignore, rgb=rgb)
    labels, counts = number(leaders, lib)
    return leaders, labels, counts


def region_stats(labels, counts, lib=None) -> dict:
    """Per-region area, bounding box (min row, min col, max row, max col) and
    sums of row / column indices of a numbered label image, regions of all
    images concatenated (image b's region k at sum(counts[:b]) + k - 1)."""
    lib = lib or load()
    L = np.ascontiguousarray(np.asarray(labels, dtype=np.int32))
    if L.ndim == 2:
        L = L[None]
    B, H, W = L.shape
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.int32).reshape(-1))
    if c.size != B:
        raise ValueError("one count per image")
    n = int(c.sum())
    area = np.empty(n, np.int32)
    bbox = np.empty((n, 4), np.int32)
    sy = np.empty(n, np.int64)
    sx = np.empty(n, np.int64)
    i64p = ctypes.POINTER(ctypes.c_int64)
    rc = lib.oracle_region_stats(_ptr(L), B, H, W, _ptr(c), _ptr(area), _ptr(bbox),
                                 sy.ctypes.data_as(i64p), sx.ctypes.data_as(i64p))
    if rc != 0:
        raise ValueError(f"oracle_region_stats failed with status {rc}")
    return {"area": area, "bbox": bbox, "sum_y": sy, "sum_x": sx}
