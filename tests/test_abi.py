"""The C-ABI library: it loads, exports every function include/ccl.h declares,
and rejects bad arguments on the host before touching HIP (so these run
without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ccl.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ccl_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from connected_component_labelling_amd import _load
    return _load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("ccl_label", "ccl_number", "ccl_count", "ccl_workspace_bytes",
                     "ccl_status_string", "ccl_label_large", "ccl_large_workspace_bytes",
                     "ccl_label_noalloc", "ccl_label_host", "ccl_label_stats"):
        assert required in names


def test_library_exports_every_declared_function(lib):
    from connected_component_labelling_amd import library_path
    out = subprocess.run(["nm", "-D", "--defined-only", library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ccl_\w+)", out))
    for name in declared_functions():
        assert name in exported, f"{name} declared in ccl.h but not exported"
        assert getattr(lib, name) is not None


def test_library_is_built_for_gfx950():
    from connected_component_labelling_amd import library_path
    blob = open(library_path(), "rb").read()
    assert b"gfx950" in blob


def test_workspace_bytes(lib):
    assert lib.ccl_workspace_bytes(0, 10, 10) == 0
    assert lib.ccl_workspace_bytes(1, 0, 10) == 0
    assert lib.ccl_workspace_bytes(-1, 10, 10) == 2**64 - 1
    a = lib.ccl_workspace_bytes(1, 256, 256)
    b = lib.ccl_workspace_bytes(2, 256, 256)
    assert 0 < a < b
    assert a % 256 == 0
    # 806-Mpx sheet: a few bytes per pixel of workspace
    big = lib.ccl_workspace_bytes(1, 24000, 33600)
    assert 0 < big < 8 * 24000 * 33600
    # per-image indices must fit in int32
    assert lib.ccl_workspace_bytes(1, 65536, 65536) == 2**64 - 1
    # fewer than 2^24 tiles of 64 x 32 in one image (a one-row image of 2^30
    # pixels has 2^24 tiles; the largest square image is far below that)
    assert lib.ccl_workspace_bytes(1, 1, 2**30) == 2**64 - 1
    assert lib.ccl_workspace_bytes(1, 1, 2**30 - 64) < 2**64 - 1
    # a batch of more tiles runs in passes of whole images: one pass's workspace
    one = lib.ccl_workspace_bytes(2**24 - 1, 2, 2)
    assert lib.ccl_workspace_bytes(2**24, 2, 2) == one
    assert lib.ccl_workspace_bytes(3 * 2**24, 2, 2) == one
    assert lib.ccl_workspace_bytes(2**23, 64, 128) == lib.ccl_workspace_bytes(2**23 - 1, 64, 128)
    assert lib.ccl_workspace_bytes(1, 46340, 46340) < 2**64 - 1


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


@pytest.mark.parametrize("args,status", [
    # (dtype, B, H, W, conn, flags, ignore, workspace_bytes), expected status
    ((4, 1, 8, 8, 6, 0, 0, 1 << 30), -4),          # connectivity
    ((2, 1, 8, 8, 8, 0, 0, 1 << 30), -5),          # dtype
    ((4, -1, 8, 8, 8, 0, 0, 1 << 30), -2),         # shape
    ((4, 1, 8, -3, 8, 0, 0, 1 << 30), -2),
    ((4, 1, 65536, 65536, 8, 0, 0, 1 << 30), -3),  # H*W > 2^31-1
    ((4, 1, 8, 8, 8, 4, 0, 1 << 30), -8),          # flags
    ((4, 1, 8, 8, 8, 0, 0, 16), -6),               # workspace too small
    ((4, 1, 8, 8, 8, 3, 0, 16), -6),               # ... with an ignored colour too
    ((1, 1, 8, 8, 8, 2, 256, 1 << 30), -9),        # ignored colour wider than a byte
    ((1, 1, 8, 8, 8, 3, 0xFFFFFFFF, 1 << 30), -9),
    ((3, 1, 8, 8, 8, 2, 0x1000000, 1 << 30), -9),  # ... wider than three bytes
    ((3, 1, 8, 8, 5, 2, 0xFFFFFF, 1 << 30), -4),
    ((3, 1, 8, 8, 8, 2, 0xFFFFFF, 16), -6),        # an RGB picture passes the dtype check
])
def test_label_validation(lib, args, status):
    dtype, B, H, W, conn, flags, ign, wsb = args
    rc = lib.ccl_label(FAKE, dtype, B, H, W, conn, flags, ign, FAKE, None, FAKE, wsb, None)
    assert rc == status
    assert lib.ccl_status_string(rc)


def test_null_pointers(lib):
    assert lib.ccl_label(None, 4, 1, 8, 8, 8, 0, 0, FAKE, None, FAKE, 1 << 30, None) == -1
    assert lib.ccl_label(FAKE, 4, 1, 8, 8, 8, 0, 0, None, None, FAKE, 1 << 30, None) == -1
    assert lib.ccl_label(FAKE, 4, 1, 8, 8, 8, 2, 7, FAKE, None, None, 1 << 30, None) == -1
    assert lib.ccl_number(None, 1, 8, 8, FAKE, None, FAKE, 1 << 30, None) == -1
    assert lib.ccl_count(FAKE, 1, 8, 8, None, FAKE, 1 << 30, None) == -1
    assert lib.ccl_number(FAKE, 1, 8, 8, FAKE, None, FAKE, 16, None) == -6
    assert lib.ccl_count(FAKE, -1, 8, 8, FAKE, FAKE, 1 << 30, None) == -2
    # region statistics: (labels, B, H, W, counts, n_total, records, ws, bytes, stream)
    assert lib.ccl_region_stats(None, 1, 8, 8, FAKE, 5, FAKE, FAKE, 1 << 30, None) == -1
    assert lib.ccl_region_stats(FAKE, 1, 8, 8, FAKE, 5, None, FAKE, 1 << 30, None) == -1
    assert lib.ccl_region_stats(FAKE, 1, 8, 8, FAKE, -1, FAKE, FAKE, 1 << 30, None) == -2
    assert lib.ccl_region_stats(FAKE, 1, 8, 8, FAKE, 5, FAKE, FAKE, 16, None) == -6
    # no region: nothing to write, no HIP call
    assert lib.ccl_region_stats(FAKE, 1, 8, 8, FAKE, 0, None, None, 0, None) == 0


def test_empty_batches_are_noops(lib):
    # nothing to do and no counts to write: returns before any HIP call
    assert lib.ccl_label(None, 4, 0, 8, 8, 8, 1, 0, None, None, None, 0, None) == 0
    assert lib.ccl_label(None, 1, 3, 0, 8, 8, 0, 0, None, None, None, 0, None) == 0
    assert lib.ccl_label(None, 1, 3, 0, 8, 8, 3, 255, None, None, None, 0, None) == 0
    assert lib.ccl_number(None, 2, 5, 0, None, None, None, 0, None) == 0


def test_large_workspace_bytes(lib):
    f = lib.ccl_large_workspace_bytes
    assert f(0, 10, 10, 0) == 0
    assert f(1, 10, 0, 0) == 0
    assert f(-1, 10, 10, 0) == 2**64 - 1
    assert f(1, 10, 10, 63) == 2**64 - 1           # band rows not a multiple of 64
    assert f(1, 10, 10, -64) == 2**64 - 1
    assert f(1, 2**20, 2**16, 2**16) == 2**64 - 1  # a band of 2^32 pixels
    one = f(1, 300, 200, 0)                        # one band: the image itself
    banded = f(1, 300, 200, 64)
    assert one > 0 and banded > 0
    assert one % 256 == 0 and banded % 256 == 0
    # every band keeps its tile workspace (a few bytes per pixel) and each seam
    # its two tile rows of numbers and of leaders: at least the tile workspace
    # of the whole image
    assert banded >= lib.ccl_workspace_bytes(1, 300, 200) - 4096
    # beyond 2^31 pixels: the tile workspaces of all bands (about 4 bytes per
    # pixel) and a few bytes per seam pixel, no 32-bit array over the picture
    big = f(1, 46400, 46400, 0)
    assert 4 * 46400 * 46400 < big < 5 * 46400 * 46400
    # a 64-row band wider than 2^31 - 1 pixels cannot be labelled
    assert f(1, 64, 2**25 + 64, 0) == 2**64 - 1
    # tall narrow images: bands stay within the tile limit
    assert f(1, 2**31 + 64, 1, 0) < 2**64 - 1
    # short very wide images that ccl_label accepts: a single band is the whole
    # image (fewer than 64 rows), not a 64-row band
    for H, W in [(1, 2**26), (32, 40_000_000), (63, 2**31 // 64)]:
        assert lib.ccl_workspace_bytes(1, H, W) < 2**64 - 1
        assert f(1, H, W, 0) < 2**64 - 1, (H, W)
        assert f(1, H, W, 64) < 2**64 - 1, (H, W)


def test_label_large_validation(lib):
    big = 1 << 40
    L = lib.ccl_label_large
    assert L(FAKE, 4, 1, 8, 8, 6, 0, 0, 0, FAKE, None, FAKE, big, None) == -4
    assert L(FAKE, 2, 1, 8, 8, 8, 0, 0, 0, FAKE, None, FAKE, big, None) == -5
    assert L(FAKE, 4, -1, 8, 8, 8, 0, 0, 0, FAKE, None, FAKE, big, None) == -2
    assert L(FAKE, 4, 1, 8, 8, 8, 4, 0, 0, FAKE, None, FAKE, big, None) == -8
    assert L(FAKE, 1, 1, 8, 8, 8, 2, 256, 0, FAKE, None, FAKE, big, None) == -9
    assert L(FAKE, 4, 1, 8, 8, 8, 0, 0, 32, FAKE, None, FAKE, big, None) == -10
    assert L(FAKE, 4, 1, 8, 8, 8, 0, 0, -64, FAKE, None, FAKE, big, None) == -10
    assert L(FAKE, 4, 1, 8, 8, 8, 0, 0, 0, FAKE, None, FAKE, 16, None) == -6
    assert L(None, 4, 1, 8, 8, 8, 0, 0, 0, FAKE, None, FAKE, big, None) == -1
    assert L(FAKE, 4, 1, 8, 8, 8, 0, 0, 0, None, None, FAKE, big, None) == -1
    assert L(FAKE, 4, 1, 2**24, 2**24, 8, 0, 0, 0, FAKE, None, FAKE, big, None) == -3
    assert L(None, 4, 0, 8, 8, 8, 1, 0, 0, None, None, None, 0, None) == 0
    # bands of 2^31 - 64 pixels: numbers and leaders take them (both go through
    # the bands' own numbering, with no 32-bit array over the picture); the
    # workspace is checked first
    W = 2**25 - 1
    assert L(FAKE, 1, 1, 128, W, 8, 1, 0, 64, FAKE, None, FAKE, 16, None) == -6
    assert L(FAKE, 1, 1, 128, W, 8, 0, 0, 64, FAKE, None, FAKE, 16, None) == -6
    assert lib.ccl_large_workspace_bytes(1, 128, W, 64) < 2**64 - 1


def test_noalloc_validation(lib):
    """ccl_label_noalloc checks everything on the host before its first HIP
    call (the scratch address lookup): these fail without a GPU."""
    N = lib.ccl_label_noalloc
    assert N(FAKE, 4, 1, 8, 8, 6, 0, 0, FAKE, None, None) == -4
    assert N(FAKE, 2, 1, 8, 8, 8, 0, 0, FAKE, None, None) == -5
    assert N(FAKE, 4, -1, 8, 8, 8, 0, 0, FAKE, None, None) == -2
    assert N(FAKE, 4, 1, 8, 8, 8, 4, 0, FAKE, None, None) == -8
    assert N(FAKE, 1, 1, 8, 8, 8, 2, 256, FAKE, None, None) == -9
    assert N(None, 4, 1, 8, 8, 8, 0, 0, FAKE, None, None) == -1
    assert N(FAKE, 4, 1, 8, 8, 8, 0, 0, None, None, None) == -1
    assert N(FAKE, 4, 1, 65536, 65536, 8, 0, 0, FAKE, None, None) == -3
    assert N(None, 4, 0, 8, 8, 8, 1, 0, None, None, None) == 0
    # the static scratch: its size bound, and the shapes on either side of it
    from connected_component_labelling_amd import SCRATCH_BYTES
    assert SCRATCH_BYTES == 64 << 20
    assert lib.ccl_workspace_bytes(64, 512, 512) <= SCRATCH_BYTES      # the u8 batch
    assert lib.ccl_workspace_bytes(1, 4096, 4096) <= SCRATCH_BYTES     # the spiral
    assert lib.ccl_workspace_bytes(1, 8192, 4096) > SCRATCH_BYTES
    assert N(FAKE, 4, 1, 8192, 4096, 8, 1, 0, FAKE, None, None) == -11
    assert N(FAKE, 1, 1, 24000, 33600, 8, 1, 0, FAKE, None, None) == -11
    assert lib.ccl_status_string(-11)


def test_label_stats_validation(lib):
    """ccl_label_stats: numbers required, counts required, records required
    when there is room for any, a capacity of at least 0; all checked on the
    host before any HIP call."""
    S = lib.ccl_label_stats
    ws = 1 << 30
    # (colours, dtype, B, H, W, conn, flags, ignore, out, counts, stats, cap, ws, bytes, stream)
    assert S(FAKE, 4, 1, 8, 8, 8, 0, 0, FAKE, FAKE, FAKE, 5, FAKE, ws, None) == -8
    assert S(FAKE, 4, 1, 8, 8, 8, 2, 0, FAKE, FAKE, FAKE, 5, FAKE, ws, None) == -8
    assert S(FAKE, 4, 1, 8, 8, 8, 1, 0, FAKE, None, FAKE, 5, FAKE, ws, None) == -1
    assert S(FAKE, 4, 1, 8, 8, 8, 1, 0, FAKE, FAKE, None, 5, FAKE, ws, None) == -1
    assert S(FAKE, 4, 1, 8, 8, 8, 1, 0, FAKE, FAKE, FAKE, -1, FAKE, ws, None) == -2
    assert S(None, 4, 1, 8, 8, 8, 1, 0, FAKE, FAKE, FAKE, 5, FAKE, ws, None) == -1
    assert S(FAKE, 4, 1, 8, 8, 8, 1, 0, None, FAKE, FAKE, 5, FAKE, ws, None) == -1
    assert S(FAKE, 4, 1, 8, 8, 8, 1, 0, FAKE, FAKE, FAKE, 5, None, ws, None) == -1
    assert S(FAKE, 4, 1, 8, 8, 8, 1, 0, FAKE, FAKE, FAKE, 5, FAKE, 16, None) == -6
    assert S(FAKE, 4, 1, 8, 8, 6, 1, 0, FAKE, FAKE, FAKE, 5, FAKE, ws, None) == -4
    assert S(FAKE, 2, 1, 8, 8, 8, 1, 0, FAKE, FAKE, FAKE, 5, FAKE, ws, None) == -5
    assert S(FAKE, 1, 1, 8, 8, 8, 3, 256, FAKE, FAKE, FAKE, 5, FAKE, ws, None) == -9
    # an empty batch: nothing to write
    assert S(None, 4, 0, 8, 8, 8, 1, 0, None, FAKE, None, 0, None, 0, None) == 0


def test_label_host_validation(lib):
    """ccl_label_host rejects bad arguments on the host before any HIP call."""
    Hh = lib.ccl_label_host
    S1, S2, S3 = ctypes.c_void_p(0x10), ctypes.c_void_p(0x20), ctypes.c_void_p(0x30)

    def call(dtype=4, B=1, H=64, W=64, conn=8, flags=1, ign=0, hin=FAKE, hout=FAKE, din=FAKE,
             dout=FAKE, ws=FAKE, wsb=1 << 30, band=0, s=S1, s_in=S2, s_out=S3):
        return Hh(hin, dtype, B, H, W, conn, flags, ign, hout, None, din, dout, ws, wsb, band,
                  s, s_in, s_out)
    assert call(conn=6) == -4
    assert call(dtype=2) == -5
    assert call(B=-1) == -2
    assert call(flags=4) == -8
    assert call(dtype=1, flags=2, ign=300) == -9
    assert call(band=48) == -10                  # not a multiple of 32 rows
    assert call(band=-32) == -10
    assert call(hin=None) == -1
    assert call(hout=None) == -1
    assert call(din=None) == -1
    assert call(dout=None) == -1
    assert call(ws=None) == -1
    assert call(s_in=None) == -12                # the copy streams: two, and not the call's
    assert call(s_out=S1) == -12
    assert call(s_in=S3) == -12
    assert call(wsb=16) == -6                    # the batch's workspace is needed
    assert call(B=4, wsb=lib.ccl_workspace_bytes(4, 64, 64) - 1) == -6
    assert call(B=0, hin=None, hout=None, din=None, dout=None, ws=None) == 0


def test_status_strings(lib):
    for s in range(-12, 1):
        assert lib.ccl_status_string(s).decode()
    assert lib.ccl_status_string(-99) == b"unknown status"
