"""MI355X (gfx950) connected-component labeller: a thin Python binding over the
C ABI of ``include/ccl.h`` (``libccl.so``, built from ``csrc/``).

This module only marshals arguments: PyTorch supplies device memory and the
stream, every step of the labelling runs in the HIP kernels of ``libccl.so``.
If the library is missing or cannot be loaded, importing the binding's
functions raises -- there is no CPU fallback.

    out, counts = label(img, connectivity=8, number=True)   # 1..n per image
    leaders, _  = label(img)                                # region minima
    out, counts = label(img, number=True, ignore=0xFFFFFF)  # white ignored: 0
    labels, counts = number(leaders)
    counts = count(leaders)
    out, counts = label_large(img, number=True)             # int64, any size
    out, counts = label_noalloc(img, number=True)           # no device allocation
    out, counts = label_host(pinned_img, number=True)       # host in, host out, copies overlapped

``img`` is a CUDA (HIP) tensor of shape [H, W] or [B, H, W], dtype uint8, or
uint32 / int32 (the 32 bits are compared as they are), or with ``rgb=True`` an
RGB picture as stored, uint8 [H, W, 3] or [B, H, W, 3] (all three bytes are
compared; an ignored RGB colour is named b0 | b1 << 8 | b2 << 16, b0 the
pixel's first byte); results are int32.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

__all__ = ["label", "number", "count", "region_stats", "workspace_bytes", "Labeller",
           "error_word", "CclError", "library_path", "label_large", "large_workspace_bytes",
           "label_noalloc", "SCRATCH_BYTES", "label_host", "HostLabeller", "label_stats"]

CCL_U8, CCL_RGB24, CCL_U32 = 1, 3, 4
CCL_NUMBER, CCL_IGNORE = 1, 2
CCL_WS_ERR_LOOP = 1
SCRATCH_BYTES = 64 << 20   # CCL_SCRATCH_BYTES: the static workspace of ccl_label_noalloc

_lib = None


class CclError(RuntimeError):
    pass


def library_path() -> str:
    return _build.LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB_PATH
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.ccl_workspace_bytes.argtypes = [i64, i64, i64]
    lib.ccl_workspace_bytes.restype = sz
    lib.ccl_label.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                              ctypes.c_uint32, vp, vp, vp, sz, vp]
    lib.ccl_label.restype = ctypes.c_int
    lib.ccl_label_profiled.argtypes = lib.ccl_label.argtypes + [ctypes.POINTER(vp), ctypes.c_int]
    lib.ccl_label_profiled.restype = ctypes.c_int
    lib.ccl_number.argtypes = [vp, i64, i64, i64, vp, vp, vp, sz, vp]
    lib.ccl_number.restype = ctypes.c_int
    lib.ccl_count.argtypes = [vp, i64, i64, i64, vp, vp, sz, vp]
    lib.ccl_count.restype = ctypes.c_int
    lib.ccl_region_stats.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, sz, vp]
    lib.ccl_region_stats.restype = ctypes.c_int
    lib.ccl_label_stats.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_uint32, vp, vp, vp, i64, vp, sz, vp]
    lib.ccl_label_stats.restype = ctypes.c_int
    lib.ccl_large_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.ccl_large_workspace_bytes.restype = sz
    lib.ccl_label_large.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_uint32, i64, vp, vp, vp, sz, vp]
    lib.ccl_label_large.restype = ctypes.c_int
    lib.ccl_label_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_uint32, vp, vp, vp]
    lib.ccl_label_noalloc.restype = ctypes.c_int
    lib.ccl_label_host.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_uint32, vp, vp, vp, vp, vp, sz, i64, vp, vp, vp]
    lib.ccl_label_host.restype = ctypes.c_int
    lib.ccl_status_string.argtypes = [ctypes.c_int]
    lib.ccl_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise CclError(f"ccl status {rc}: {_load().ccl_status_string(rc).decode()}")


def workspace_bytes(batch: int, height: int, width: int) -> int:
    return int(_load().ccl_workspace_bytes(batch, height, width))


def _batch_view(t: torch.Tensor, rgb: bool = False):
    if rgb:
        if t.dtype != torch.uint8 or t.shape[-1:] != (3,):
            raise TypeError("an RGB picture is a uint8 tensor with a last dimension of 3")
        if t.dim() == 3:
            return t.unsqueeze(0), True
        if t.dim() != 4:
            raise ValueError("expected an [H, W, 3] or [B, H, W, 3] RGB tensor")
        return t, False
    if t.dim() == 2:
        return t.unsqueeze(0), True
    if t.dim() != 3:
        raise ValueError("expected a [H, W] or [B, H, W] tensor")
    return t, False


def _dtype_code(t: torch.Tensor, rgb: bool = False) -> int:
    if rgb:
        return CCL_RGB24
    if t.dtype == torch.uint8:
        return CCL_U8
    if t.dtype in (torch.int32, torch.uint32):
        return CCL_U32
    raise TypeError(f"colour dtype must be uint8, uint32 or int32, not {t.dtype}")


def _require_device(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


def _output(out, B, H, W, dtype, device, squeeze):
    """(tensor the kernels write, tensor returned): a new [B, H, W] tensor
    (returned as [H, W] for a single image), or the caller's ``out`` as given,
    which must be contiguous, of ``dtype`` and hold B*H*W values."""
    if out is None:
        out = torch.empty((B, H, W), dtype=dtype, device=device)
        return out, (out[0] if squeeze else out)
    _require_device(out, "out")
    if out.dtype != dtype or out.numel() != B * H * W:
        raise ValueError(f"out must be a {dtype} tensor of {B * H * W} values")
    return out, out


def _new_workspace(B, H, W, device):
    n = workspace_bytes(B, H, W)
    if n == 2**64 - 1:
        raise CclError("image or batch too large to index" if min(B, H, W) >= 0
                       else "batch, height or width is negative")
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def error_word(workspace: torch.Tensor) -> int:
    """The workspace's error word as the last call left it (each call clears it
    first; nonzero only if a bounded loop of that call gave up).  Reading it
    waits for the device."""
    return int(workspace[:4].view(torch.int32).item())


def _check_word(workspace: torch.Tensor, stream):
    """Wait for the call on ``stream`` and raise if it set the error word."""
    (stream if stream is not None else torch.cuda.current_stream()).synchronize()
    err = error_word(workspace)
    if err != 0:
        raise CclError(f"a bounded loop gave up (workspace error word 0x{err:x}): the labels "
                       f"of this call are not valid")


def _flags(number: bool, ignore) -> tuple[int, int]:
    """(flags, ignore value) for ccl_label; ``ignore`` None ignores nothing."""
    flags = CCL_NUMBER if number else 0
    if ignore is None:
        return flags, 0
    return flags | CCL_IGNORE, int(ignore) & 0xFFFFFFFF


def label(img: torch.Tensor, connectivity: int = 8, number: bool = False, stream=None,
          workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
          with_counts: bool = True, ignore: int | None = None, rgb: bool = False,
          check: bool = False):
    """Label ``img``: leaders (per-image reading-order index of each region's first
    pixel) or, with ``number=True``, numbers 1..n per image.  With ``ignore`` set,
    pixels of that colour belong to no region: -1 as leaders, 0 as numbers, never
    counted.  With ``rgb``, ``img`` is an RGB picture of three bytes per pixel.
    ``out``, if given, is a contiguous int32 tensor of B*H*W values (any
    shape), returned as it is.  With ``check``, waits for the call and raises
    CclError if one of its bounded loops gave up (the default does not wait).
    Returns (out, counts)."""
    _require_device(img, "img")
    x, squeeze = _batch_view(img, rgb)
    B, H, W = x.shape[:3]
    out, ret = _output(out, B, H, W, torch.int32, img.device, squeeze)
    counts = torch.empty(B, dtype=torch.int32, device=img.device) if with_counts else None
    if workspace is None:
        workspace = _new_workspace(B, H, W, img.device)
    flags, ign = _flags(number, ignore)
    _check(_load().ccl_label(_ptr(x), _dtype_code(x, rgb), B, H, W, int(connectivity), flags, ign,
                             _ptr(out), _ptr(counts), _ptr(workspace), workspace.numel(),
                             ctypes.c_void_p(_stream_handle(stream))))
    if check and B * H * W > 0:
        _check_word(workspace, stream)
    return ret, counts


def label_noalloc(img: torch.Tensor, connectivity: int = 8, number: bool = False, stream=None,
                  out: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                  ignore: int | None = None, rgb: bool = False):
    """``label`` through ccl_label_noalloc: no workspace, the library's static
    per-GPU scratch array instead (batches up to SCRATCH_BYTES of workspace;
    calls that overlap on one GPU race).  With ``out`` and ``counts`` given
    (contiguous device int32 tensors of B*H*W and B values) nothing is
    allocated.  Returns (out, counts)."""
    _require_device(img, "img")
    x, squeeze = _batch_view(img, rgb)
    B, H, W = x.shape[:3]
    out, ret = _output(out, B, H, W, torch.int32, img.device, squeeze)
    if counts is None:
        counts = torch.empty(B, dtype=torch.int32, device=img.device)
    else:
        _require_device(counts, "counts")
        if counts.dtype != torch.int32 or counts.numel() != B:
            raise ValueError(f"counts must be an int32 tensor of {B} values")
    flags, ign = _flags(number, ignore)
    _check(_load().ccl_label_noalloc(_ptr(x), _dtype_code(x, rgb), B, H, W, int(connectivity),
                                     flags, ign, _ptr(out), _ptr(counts),
                                     ctypes.c_void_p(_stream_handle(stream))))
    return ret, counts


def number(leaders: torch.Tensor, stream=None, inplace: bool = False,
           workspace: torch.Tensor | None = None):
    """Numbers 1..n per image from a leader image.  Returns (labels, counts)."""
    _require_device(leaders, "leaders")
    if leaders.dtype != torch.int32:
        raise TypeError("leaders must be int32")
    x, squeeze = _batch_view(leaders)
    B, H, W = x.shape
    labels = x if inplace else torch.empty_like(x)
    counts = torch.empty(B, dtype=torch.int32, device=leaders.device)
    if workspace is None:
        workspace = _new_workspace(B, H, W, leaders.device)
    _check(_load().ccl_number(_ptr(x), B, H, W, _ptr(labels), _ptr(counts), _ptr(workspace),
                              workspace.numel(), ctypes.c_void_p(_stream_handle(stream))))
    return (labels[0] if squeeze else labels), counts


def count(leaders: torch.Tensor, stream=None, workspace: torch.Tensor | None = None):
    """Regions per image of a leader image (pixels with leaders[p] == p)."""
    _require_device(leaders, "leaders")
    if leaders.dtype != torch.int32:
        raise TypeError("leaders must be int32")
    x, _ = _batch_view(leaders)
    B, H, W = x.shape
    counts = torch.empty(B, dtype=torch.int32, device=leaders.device)
    if workspace is None:
        workspace = _new_workspace(B, H, W, leaders.device)
    _check(_load().ccl_count(_ptr(x), B, H, W, _ptr(counts), _ptr(workspace), workspace.numel(),
                             ctypes.c_void_p(_stream_handle(stream))))
    return counts


def region_stats(labels: torch.Tensor, counts: torch.Tensor, n_total: int | None = None,
                 stream=None, workspace: torch.Tensor | None = None) -> dict:
    """Per-region area, bounding box (min row, min col, max row, max col) and sums
    of row / column indices of a numbered labelling (label(..., number=True)),
    regions of all images concatenated: image b's region k is record
    sum(counts[:b]) + k - 1.  ``n_total`` (the sum of ``counts``) is read from
    the device when not given.  Returns views of one int64 [n, 5] tensor of
    ccl_region records ("records"): "area", "bbox", "sum_y", "sum_x"."""
    _require_device(labels, "labels")
    if labels.dtype != torch.int32 or counts.dtype != torch.int32:
        raise TypeError("labels and counts must be int32")
    x, _ = _batch_view(labels)
    B, H, W = x.shape
    if counts.numel() != B or not counts.is_cuda:
        raise ValueError("counts must be a device tensor with one entry per image")
    if n_total is None:
        n_total = int(counts.to(torch.int64).sum().item())
    dev = labels.device
    rec = torch.empty((n_total, 5), dtype=torch.int64, device=dev)  # 40-byte ccl_region records
    if workspace is None:
        workspace = _new_workspace(B, H, W, dev)
    _check(_load().ccl_region_stats(_ptr(x), B, H, W, _ptr(counts.contiguous()), n_total,
                                    _ptr(rec), _ptr(workspace), workspace.numel(),
                                    ctypes.c_void_p(_stream_handle(stream))))
    return _stats_views(rec)


def _stats_views(rec: torch.Tensor) -> dict:
    r32 = rec.view(torch.int32)
    return {"records": rec, "area": r32[:, 4], "bbox": r32[:, 5:9], "sum_y": rec[:, 0],
            "sum_x": rec[:, 1]}


def label_stats(img: torch.Tensor, max_regions: int, connectivity: int = 8, stream=None,
                workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                records: torch.Tensor | None = None, ignore: int | None = None,
                rgb: bool = False, trim: bool = True, check: bool = False):
    """``label(img, number=True)`` and ``region_stats`` in one call
    (ccl_label_stats): the statistics come from the run records of the call,
    not from a pass over the labels.  ``max_regions`` is the capacity of the
    records (regions past it are not recorded; ``records``, if given, is a
    contiguous int64 [>= max_regions, 5] tensor).  Returns (labels, counts,
    stats) with ``stats`` as ``region_stats`` gives it; with ``trim`` (waits
    for the device) its views are cut to the number of regions recorded.
    ``check`` as for ``label``."""
    _require_device(img, "img")
    x, squeeze = _batch_view(img, rgb)
    B, H, W = x.shape[:3]
    out, ret = _output(out, B, H, W, torch.int32, img.device, squeeze)
    counts = torch.empty(B, dtype=torch.int32, device=img.device)
    cap = int(max_regions)
    if records is None:
        records = torch.empty((max(cap, 1), 5), dtype=torch.int64, device=img.device)
    elif records.dtype != torch.int64 or records.dim() != 2 or records.shape[1] != 5 or \
            records.shape[0] < cap or not records.is_contiguous():
        raise ValueError("records must be a contiguous int64 [max_regions, 5] tensor")
    if workspace is None:
        workspace = _new_workspace(B, H, W, img.device)
    flags, ign = _flags(True, ignore)
    _check(_load().ccl_label_stats(_ptr(x), _dtype_code(x, rgb), B, H, W, int(connectivity), flags,
                                   ign, _ptr(out), _ptr(counts), _ptr(records), cap,
                                   _ptr(workspace), workspace.numel(),
                                   ctypes.c_void_p(_stream_handle(stream))))
    if check and B * H * W > 0:
        _check_word(workspace, stream)
    rec = records
    if trim:
        n = min(cap, int(counts.to(torch.int64).sum().item()))
        rec = records[:n]
    return ret, counts, _stats_views(rec)


def large_workspace_bytes(batch: int, height: int, width: int, band_rows: int = 0) -> int:
    return int(_load().ccl_large_workspace_bytes(batch, height, width, band_rows))


def label_large(img: torch.Tensor, connectivity: int = 8, number: bool = False, stream=None,
                workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                with_counts: bool = True, ignore: int | None = None, rgb: bool = False,
                band_rows: int = 0, check: bool = False):
    """As ``label``, for images of any size (also beyond 2^31 pixels): int64
    leaders or numbers and int64 counts.  The image is labelled in bands of
    ``band_rows`` rows (0: automatic, about 2^30 pixels each; else a multiple
    of 64), joined across the band seams; results do not depend on it.
    ``check`` as for ``label``.  Returns (out, counts)."""
    _require_device(img, "img")
    x, squeeze = _batch_view(img, rgb)
    B, H, W = x.shape[:3]
    out, ret = _output(out, B, H, W, torch.int64, img.device, squeeze)
    counts = torch.empty(B, dtype=torch.int64, device=img.device) if with_counts else None
    flags, ign = _flags(number, ignore)
    lib = _load()

    def call(ws, nbytes):
        return lib.ccl_label_large(_ptr(x), _dtype_code(x, rgb), B, H, W, int(connectivity), flags,
                                   ign, int(band_rows), _ptr(out), _ptr(counts), ws, nbytes,
                                   ctypes.c_void_p(_stream_handle(stream)))

    if workspace is None:
        n = large_workspace_bytes(B, H, W, band_rows)
        if n == 2**64 - 1:
            # the shape or band height is rejected: the call names why (its
            # checks all run on the host before anything is enqueued)
            _check(call(ctypes.c_void_p(256), 0))
            _check(-3)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=img.device)
    _check(call(_ptr(workspace), workspace.numel()))
    if check and B * H * W > 0:
        _check_word(workspace, stream)
    return ret, counts


class Labeller:
    """Holds output, counts and workspace for one batch shape, so repeated calls
    allocate nothing (as a benchmark or a serving loop wants)."""

    def __init__(self, shape, device="cuda", connectivity: int = 8):
        """``shape`` is the label shape, [H, W] or [B, H, W] (for an RGB picture,
        its shape without the last dimension)."""
        if len(shape) == 2:
            shape = (1, *shape)
        self.B, self.H, self.W = (int(v) for v in shape)
        self.connectivity = connectivity
        self.out = torch.empty((self.B, self.H, self.W), dtype=torch.int32, device=device)
        self.counts = torch.empty(self.B, dtype=torch.int32, device=device)
        self.workspace = _new_workspace(self.B, self.H, self.W, device)

    def __call__(self, img: torch.Tensor, number: bool = True, stream=None, events=None,
                 ignore: int | None = None, rgb: bool = False):
        x, _ = _batch_view(img, rgb)
        if tuple(x.shape[:3]) != (self.B, self.H, self.W):
            raise ValueError("image shape does not match the Labeller")
        lib = _load()
        flags, ign = _flags(number, ignore)
        args = [_ptr(x), _dtype_code(x, rgb), self.B, self.H, self.W, self.connectivity,
                flags, ign, _ptr(self.out), _ptr(self.counts),
                _ptr(self.workspace), self.workspace.numel(),
                ctypes.c_void_p(_stream_handle(stream))]
        if events is None:
            _check(lib.ccl_label(*args))
        else:
            arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e) for e in events])
            _check(lib.ccl_label_profiled(*args, arr, len(events)))
        return self.out, self.counts


_copy_streams = {}


def _copy_streams_for(device):
    """Two streams (default priority) for the copies of label_host, made once
    per device."""
    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    if idx not in _copy_streams:
        _copy_streams[idx] = (torch.cuda.Stream(device=idx), torch.cuda.Stream(device=idx))
    return _copy_streams[idx]


class HostLabeller:
    """Labels pictures in page-locked host memory through ccl_label_host: the
    picture goes in and the labels come out on two copy streams, band by band,
    beside the kernels.  Holds the device copy of the picture, the device
    labels, the page-locked host labels, the counts and the workspace for one
    batch shape, so repeated calls allocate nothing."""

    def __init__(self, shape, dtype=torch.uint8, rgb: bool = False, device="cuda",
                 connectivity: int = 8, band_rows: int = 0):
        """``shape`` is the label shape, [H, W] or [B, H, W]; ``dtype`` the colour
        dtype (uint8, or uint32 / int32; with ``rgb``, three uint8 per pixel)."""
        if len(shape) == 2:
            shape = (1, *shape)
        self.B, self.H, self.W = (int(v) for v in shape)
        self.rgb = rgb
        self.connectivity = connectivity
        self.band_rows = int(band_rows)
        pix = (self.B, self.H, self.W, 3) if rgb else (self.B, self.H, self.W)
        self.dev_img = torch.empty(pix, dtype=torch.uint8 if rgb else dtype, device=device)
        self.dev_out = torch.empty((self.B, self.H, self.W), dtype=torch.int32, device=device)
        self.out = torch.empty((self.B, self.H, self.W), dtype=torch.int32, pin_memory=True)
        self.counts = torch.empty(self.B, dtype=torch.int32, device=device)
        self.workspace = _new_workspace(self.B, self.H, self.W, device)
        self.copy_streams = _copy_streams_for(device)

    def __call__(self, img: torch.Tensor, number: bool = True, stream=None,
                 ignore: int | None = None, wait: bool = True):
        """Label ``img`` (a page-locked CPU tensor of this labeller's shape and
        dtype).  Returns (host labels, device counts); with ``wait`` the call
        is complete on return, else once ``stream`` reaches its end."""
        if img.is_cuda or not img.is_contiguous():
            raise ValueError("img must be a contiguous host tensor")
        if not img.is_pinned():
            raise ValueError("img must be page-locked (pin_memory()) for the copies to overlap")
        x, _ = _batch_view(img, self.rgb)
        if tuple(x.shape) != tuple(self.dev_img.shape) or x.dtype != self.dev_img.dtype:
            raise ValueError("image shape or dtype does not match the HostLabeller")
        flags, ign = _flags(number, ignore)
        s = stream if stream is not None else torch.cuda.current_stream()
        h2d, d2h = self.copy_streams
        _check(_load().ccl_label_host(
            _ptr(x), _dtype_code(x, self.rgb), self.B, self.H, self.W, self.connectivity, flags,
            ign, _ptr(self.out), _ptr(self.counts), _ptr(self.dev_img), _ptr(self.dev_out),
            _ptr(self.workspace), self.workspace.numel(), self.band_rows,
            ctypes.c_void_p(s.cuda_stream), ctypes.c_void_p(h2d.cuda_stream),
            ctypes.c_void_p(d2h.cuda_stream)))
        if wait:
            s.synchronize()
        return self.out, self.counts


def label_host(img: torch.Tensor, connectivity: int = 8, number: bool = False,
               ignore: int | None = None, rgb: bool = False, band_rows: int = 0,
               device="cuda"):
    """``label`` for a page-locked host picture, with the copies in and out
    overlapped with the labelling band by band (ccl_label_host).  Returns
    (host labels [B, H, W] or [H, W], device counts) once complete."""
    x, squeeze = _batch_view(img, rgb)
    lab = HostLabeller(tuple(x.shape[:3]), dtype=x.dtype, rgb=rgb, device=device,
                       connectivity=connectivity, band_rows=band_rows)
    out, counts = lab(img, number=number, ignore=ignore)
    return (out[0] if squeeze else out), counts
