"""GPU parity of ccl_label_large (images of any size, 64-bit results) against
the oracle's 64-bit entry points, bit for bit: small images cut into bands of
64 or 128 rows so that regions cross many band seams (serpentines, combs,
spirals, diagonals, ignored colours, RGB bytes, batches), the workloads at full
size in bands of 1024 rows, and a 46400 x 46400 image of 2.15 G pixels, beyond
the int32 index range."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.test_gpu_parity import (max_size_image, mosaic_images, rgb_palette_image,
                                   structured_images)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ccl():
    import connected_component_labelling_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m._load()
    return m


def to_device(img: np.ndarray) -> torch.Tensor:
    if img.dtype == np.uint32:
        img = img.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(img)).cuda()


def check_large(ccl, name, img, conn=8, band_rows=64, ignore=None, rgb=False, expect=None):
    """Leaders, numbers and counts of label_large equal the oracle's (or
    ``expect`` = (leaders, labels, counts) computed by the caller from it)."""
    ign = "" if ignore is None else f" ignore=0x{int(ignore):x}"
    print(f"[gpu case] large {name} shape={tuple(img.shape)} dtype={img.dtype} conn={conn} "
          f"band_rows={band_rows}{ign}", flush=True)
    if expect is None:
        exp_leaders = oracle.label64(img, conn, ignore=ignore, rgb=rgb)
        exp_labels, exp_counts = oracle.number64(exp_leaders)
    else:
        exp_leaders, exp_labels, exp_counts = expect
    t = to_device(img)
    batch = img if img.ndim == (4 if rgb else 3) else img[None]
    B, H, W = batch.shape[:3]
    ws = torch.zeros(max(ccl.large_workspace_bytes(B, H, W, band_rows), 1), dtype=torch.uint8,
                     device="cuda")
    leaders, c0 = ccl.label_large(t, conn, number=False, ignore=ignore, rgb=rgb,
                                  band_rows=band_rows, workspace=ws)
    torch.cuda.synchronize()
    got = leaders.cpu().numpy()
    del leaders
    assert got.dtype == np.int64
    if not np.array_equal(got, exp_leaders):
        bad = np.argwhere(got != exp_leaders)
        raise AssertionError(f"{name}: leaders differ at {len(bad)} pixels, first {bad[:5].tolist()}")
    del got
    labels, c1 = ccl.label_large(t, conn, number=True, ignore=ignore, rgb=rgb,
                                 band_rows=band_rows, workspace=ws)
    torch.cuda.synchronize()
    assert ccl.error_word(ws) == 0, f"{name}: kernel safety bound hit"
    got = labels.cpu().numpy()
    del labels, t, ws
    if not np.array_equal(got, exp_labels):
        bad = np.argwhere(got != exp_labels)
        raise AssertionError(f"{name}: numbers differ at {len(bad)} pixels, first {bad[:5].tolist()}")
    assert np.array_equal(c0.cpu().numpy(), exp_counts), f"{name}: counts (leader mode) differ"
    assert np.array_equal(c1.cpu().numpy(), exp_counts), f"{name}: counts differ"
    return exp_counts


def serpentine(H, W, period=2):
    """One 1-pixel path that runs down a column, across the bottom, up the next
    column, across the top, ...: every band seam is crossed by it again and
    again, so joins must travel along the whole chain of seams."""
    img = np.zeros((H, W), np.uint8)
    cols = list(range(0, W, period))
    img[:, cols] = 1
    for k, c in enumerate(cols[:-1]):
        row = H - 1 if k % 2 == 0 else 0
        img[row, c:cols[k + 1] + 1] = 1
    return img


@pytest.mark.parametrize("conn", [8, 4])
@pytest.mark.parametrize("dtype", [np.uint32, np.uint8])
def test_large_ragged_random(ccl, conn, dtype):
    rng = np.random.default_rng(500 + conn)
    for H in (1, 63, 64, 65, 128, 129, 200, 257):
        for W in (1, 2, 63, 65, 200):
            ncol = int(rng.integers(1, 4))
            idx = rng.integers(0, ncol, size=(H, W))
            img = (idx.astype(np.uint8) if dtype == np.uint8 else
                   rng.integers(0, 2**32, size=ncol, dtype=np.uint64).astype(np.uint32)[idx])
            check_large(ccl, f"random {H}x{W}", img, conn, band_rows=64)


@pytest.mark.parametrize("conn", [8, 4])
def test_large_structured(ccl, conn):
    images = dict(structured_images())
    images.update(mosaic_images())
    images["serpentine 700x41"] = serpentine(700, 41)
    images["serpentine 1000x9 period 4"] = serpentine(1000, 9, period=4)
    images["spiral 640x480"] = synth.spiral_image(640, 480, seed=8)
    for name, img in images.items():
        for band_rows in (64, 128, 0):
            check_large(ccl, name, img, conn, band_rows=band_rows)


@pytest.mark.parametrize("conn", [8, 4])
def test_large_ignore_and_rgb(ccl, conn):
    rng = np.random.default_rng(600 + conn)
    for H, W in ((200, 130), (257, 65), (130, 1)):
        img = rng.integers(0, 3, size=(H, W)).astype(np.uint8)
        check_large(ccl, f"ignore {H}x{W}", img, conn, band_rows=64, ignore=int(img[0, 0]))
        rgb = rgb_palette_image(rng, (H, W), 3)
        check_large(ccl, f"rgb {H}x{W}", rgb, conn, band_rows=64, rgb=True)
        px = rgb[H // 2, W // 2]
        ign = int(px[0]) | (int(px[1]) << 8) | (int(px[2]) << 16)
        check_large(ccl, f"rgb {H}x{W}", rgb, conn, band_rows=64, rgb=True, ignore=ign)
    sheet = synth.sheet_image(640, 960, seed=6, density=30.0)
    check_large(ccl, "sheet 640x960, paper ignored", sheet, conn, band_rows=64, ignore=0xFFFFFF)


def test_large_batch(ccl):
    rng = np.random.default_rng(33)
    img = rng.integers(0, 3, size=(3, 150, 130)).astype(np.uint8)
    check_large(ccl, "batch 3x150x130", img, 8, band_rows=64)
    img = synth.bernoulli_batch(4, 300, 90, seed=9)
    check_large(ccl, "bernoulli batch 4x300x90", img, 8, band_rows=128)
    # an odd number of pixels per image: every other image's int64 output
    # starts 8 bytes off a 16-byte boundary (the 8-byte store path)
    img = rng.integers(0, 3, size=(3, 133, 21)).astype(np.uint8)
    check_large(ccl, "batch 3x133x21 (odd H*W)", img, 8, band_rows=64)
    check_large(ccl, "batch 3x133x21 (odd H*W)", img, 4, band_rows=0)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("config", [3, 4, 5])
def test_large_workload_full_size(ccl, config):
    """The workloads at full size in bands of 1024 rows (and, for the sheet,
    the automatic single band) against the oracle."""
    img = synth.generate(config)[0]
    leaders = oracle.label(img, 8)
    labels, counts = oracle.number(leaders)
    expect = (leaders, labels, counts.astype(np.int64))
    check_large(ccl, f"workload {config}", img, 8, band_rows=1024, expect=expect)
    if config == 5:
        check_large(ccl, f"workload {config}", img, 8, band_rows=0, expect=expect)


@pytest.mark.timeout(1100)
def test_beyond_int32(ccl):
    """46400 x 46400 = 2,152,960,000 pixels (> 2^31 - 1): the automatic bands
    (23,104 rows: two full bands and one of 192 rows) against the oracle's
    64-bit labelling, and horizontal stripes against their closed form
    (leader of row r = r*W up to 2.15e9, number r + 1) for both the GPU and
    the oracle."""
    H = W = 46400
    assert H * W > 2**31 - 1
    img = max_size_image(H, W)
    counts = check_large(ccl, "beyond int32 46400x46400", img, 8, band_rows=0)
    print(f"[gpu case] beyond int32 regions: {counts.tolist()}", flush=True)
    del img
    stripes = np.empty((H, W), np.uint8)
    stripes[0::2] = 1
    stripes[1::2] = 2
    print("[gpu case] large stripes 46400x46400 (closed form)", flush=True)
    t = to_device(stripes)
    out, c = ccl.label_large(t, 8, number=False)
    torch.cuda.synchronize()
    rows = torch.arange(H, device="cuda", dtype=torch.int64)[:, None] * W
    assert bool((out == rows).all()), "stripes: leaders are not r*W"
    assert int(c[0]) == H
    out, c = ccl.label_large(t, 8, number=True, out=out)
    torch.cuda.synchronize()
    assert bool((out == torch.arange(1, H + 1, device="cuda", dtype=torch.int64)[:, None]).all())
    assert int(c[0]) == H
    del out, t, rows
    torch.cuda.empty_cache()
    L = oracle.label64(stripes, 8)                 # the oracle at 64-bit indices
    assert np.array_equal(L[::997, ::991], np.arange(0, H, 997, dtype=np.int64)[:, None] * W
                          + np.zeros((1, len(range(0, W, 991))), np.int64))
    assert L[-1, -1] == (H - 1) * W and L[-1, 0] == (H - 1) * W
    N, cnt = oracle.number64(L)
    assert cnt[0] == H and N[-1, -1] == H and N[12345, 6789] == 12346


def test_out_argument(ccl):
    """A caller's ``out`` tensor (any shape of B*H*W values) is written and
    returned as it is, by label and label_large alike."""
    rng = np.random.default_rng(41)
    img = rng.integers(0, 3, size=(100, 70)).astype(np.uint8)
    exp = oracle.label(img, 8)
    t = to_device(img)
    o32 = torch.empty((100, 70), dtype=torch.int32, device="cuda")
    r, _ = ccl.label(t, 8, out=o32)
    assert r is o32 and np.array_equal(o32.cpu().numpy(), exp)
    o64 = torch.empty(7000, dtype=torch.int64, device="cuda")
    r, _ = ccl.label_large(t, 8, out=o64, band_rows=64)
    assert r is o64 and np.array_equal(o64.cpu().numpy().reshape(100, 70), exp)
    with pytest.raises(ValueError):
        ccl.label_large(t, 8, out=o32)             # int32 where int64 is written
