"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, bit for
bit -- leaders, numbers and counts -- on seeded inputs: ragged small shapes that
span several tiles, structured adversaries, every workload at its full size,
and the standalone number / count calls."""
import numpy as np
import pytest
import torch

import oracle
import synth

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


def announce(name, img, conn, ignore=None):
    ign = "" if ignore is None else f" ignore=0x{int(ignore):x}"
    print(f"[gpu case] {name} shape={tuple(img.shape)} dtype={img.dtype} conn={conn}{ign}",
          flush=True)


def check_case(ccl, name, img, conn=8, workspace=None, ignore=None):
    """Leaders, numbers and counts of the HIP path equal the oracle's (with
    ``ignore``: pixels of that colour are -1 / 0 and not counted)."""
    announce(name, img, conn, ignore)
    exp_leaders = oracle.label(img, conn, ignore=ignore)
    exp_labels, exp_counts = oracle.number(exp_leaders)
    t = to_device(img)
    batch = img if img.ndim == 3 else img[None]
    B, H, W = batch.shape
    if workspace is None:
        workspace = torch.zeros(max(ccl.workspace_bytes(B, H, W), 1), dtype=torch.uint8,
                                device="cuda")
    leaders, c0 = ccl.label(t, conn, number=False, workspace=workspace, ignore=ignore)
    labels, c1 = ccl.label(t, conn, number=True, workspace=workspace, ignore=ignore)
    torch.cuda.synchronize()
    got_leaders = leaders.cpu().numpy()
    got_labels = labels.cpu().numpy()
    assert ccl.error_word(workspace) == 0, f"{name}: kernel safety bound hit"
    if not np.array_equal(got_leaders, exp_leaders):
        bad = np.argwhere(got_leaders != exp_leaders)
        raise AssertionError(f"{name}: leaders differ at {len(bad)} pixels, first {bad[:5].tolist()}")
    assert np.array_equal(got_labels, exp_labels), f"{name}: numbers differ"
    assert np.array_equal(c0.cpu().numpy(), exp_counts), f"{name}: counts (leader mode) differ"
    assert np.array_equal(c1.cpu().numpy(), exp_counts), f"{name}: counts differ"
    return exp_counts


# ---------------------------------------------------------------- small shapes

HS = [1, 2, 31, 32, 33, 64, 65, 100]
WS = [1, 2, 63, 64, 65, 127, 128, 129, 200]


@pytest.mark.parametrize("conn", [8, 4])
@pytest.mark.parametrize("dtype", [np.uint32, np.uint8])
def test_ragged_shapes_random(ccl, conn, dtype):
    rng = np.random.default_rng(100 + conn)
    for H in HS:
        for W in WS:
            ncol = int(rng.integers(1, 4))
            idx = rng.integers(0, ncol, size=(H, W))
            if dtype == np.uint8:
                img = idx.astype(np.uint8)
            else:
                img = rng.integers(0, 2**32, size=ncol, dtype=np.uint64).astype(np.uint32)[idx]
            check_case(ccl, f"random {H}x{W} ncol={ncol}", img, conn)


@pytest.mark.parametrize("conn", [8, 4])
def test_ragged_shapes_blobs(ccl, conn):
    """Smooth multi-colour blobs: long runs and regions that cross many seams."""
    rng = np.random.default_rng(7)
    for H, W in [(97, 131), (64, 64), (200, 190), (33, 257), (300, 65)]:
        base = rng.random((H // 8 + 2, W // 8 + 2))
        up = np.kron(base, np.ones((8, 8)))[:H, :W]
        img = (up * 3).astype(np.uint32) + 5
        check_case(ccl, f"blobs {H}x{W}", img, conn)


# ------------------------------------------------------ structured adversaries

def structured_images():
    out = {}
    H, W = 130, 200
    yy, xx = np.mgrid[0:H, 0:W]
    out["uniform"] = np.full((H, W), 0xFFFFFF, np.uint32)
    out["checkerboard"] = ((yy + xx) % 2).astype(np.uint32)
    out["vertical stripes"] = (xx % 2).astype(np.uint8)
    out["horizontal stripes"] = (yy % 2).astype(np.uint8)
    out["wide stripes across seams"] = ((xx // 3) % 2).astype(np.uint32)
    diag = np.zeros((H, W), np.uint32)
    for d in range(-H, W, 7):                      # 1-px diagonals crossing tile corners
        idx = np.arange(H)
        c = idx + d
        ok = (c >= 0) & (c < W)
        diag[idx[ok], c[ok]] = 1
    out["diagonals"] = diag
    anti = np.zeros((H, W), np.uint32)
    for d in range(0, H + W, 5):
        idx = np.arange(H)
        c = d - idx
        ok = (c >= 0) & (c < W)
        anti[idx[ok], c[ok]] = 2
    out["anti-diagonals"] = anti
    comb = np.zeros((H, W), np.uint8)
    comb[:, ::2] = 1
    comb[H - 1, :] = 1                              # teeth joined at the very bottom
    out["comb joined at the bottom"] = comb
    stair = np.zeros((H, W), np.uint32)
    for i in range(W):                              # staircase: later teeth start higher
        stair[max(0, H - 1 - i):, i] = 3 if i % 2 == 0 else 0
    stair[H - 1, :] = 3
    out["staircase"] = stair
    out["spiral 200x300"] = synth.spiral_image(200, 300, seed=4)
    out["sheet 640x960"] = synth.sheet_image(640, 960, seed=6, density=30.0)
    out["lines 256x256"] = synth.lines_image(256, 256, seed=1)
    return out


@pytest.mark.parametrize("conn", [8, 4])
def test_structured(ccl, conn):
    for name, img in structured_images().items():
        check_case(ccl, name, img, conn)


def mosaic_images():
    """Solid areas (tiles of one colour) beside noisy ones: aligned and shifted
    against the 64x32 tile grid, solid areas that meet across tile edges only
    through a few pixels or a diagonal, and single tiles."""
    out = {}
    rng = np.random.default_rng(21)
    for H, W, bh, bw, off in [(96, 192, 32, 64, (0, 0)), (130, 260, 40, 70, (5, 17)),
                              (64, 256, 32, 64, (0, 0)), (200, 333, 50, 90, (13, 40))]:
        yy, xx = np.mgrid[0:H, 0:W]
        cell = ((yy + off[0]) // bh) * 1000 + (xx + off[1]) // bw
        solid_colour = (cell % 3).astype(np.uint32) + 7          # neighbouring cells may match
        noisy = rng.random((H // 8 + 1, W // 8 + 1)) < 0.3
        noise_cell = np.kron(noisy, np.ones((8, 8), bool))[:H, :W]
        img = np.where(noise_cell, rng.integers(0, 3, size=(H, W)).astype(np.uint32) + 7, solid_colour)
        out[f"mosaic {H}x{W} cells {bh}x{bw}"] = img
    # one-colour tiles joined to each other only through one pixel or a diagonal
    img = np.zeros((96, 192), np.uint32)
    img[0:32, 0:64] = 5
    img[32:64, 64:128] = 5                                         # diagonal corner contact
    img[31, 64] = 9                                                 # keeps tile (0,1) mixed
    img[64:96, 0:64] = 5
    img[63, 10] = 5                                                 # one-pixel bridge upward
    out["one-colour tiles meeting at corners"] = img
    out["single tile, one colour"] = np.full((32, 64), 3, np.uint32)
    out["single partial tile, one colour"] = np.full((17, 40), 3, np.uint32)
    out["two tiles, one colour"] = np.full((32, 128), 3, np.uint32)
    return out


@pytest.mark.parametrize("conn", [8, 4])
@pytest.mark.parametrize("dtype", [np.uint32, np.uint8])
def test_one_colour_tiles(ccl, conn, dtype):
    for name, img in mosaic_images().items():
        check_case(ccl, name, img.astype(dtype), conn)


def test_batch_ragged(ccl):
    rng = np.random.default_rng(3)
    img = rng.integers(0, 3, size=(3, 70, 130)).astype(np.uint8)
    check_case(ccl, "batch 3x70x130", img, 8)
    img = synth.bernoulli_batch(5, 100, 90, seed=9)
    check_case(ccl, "bernoulli batch 5x100x90", img, 8)


# ------------------------------------------------------- one ignored colour

def most_common_colour(img: np.ndarray) -> int:
    """The colour of most pixels (of a strided sample): the paper of a drawing."""
    v, c = np.unique(img.reshape(-1)[::97], return_counts=True)
    return int(v[np.argmax(c)])


@pytest.mark.parametrize("conn", [8, 4])
@pytest.mark.parametrize("dtype", [np.uint32, np.uint8])
def test_ignore_ragged_random(ccl, conn, dtype):
    rng = np.random.default_rng(200 + conn)
    for H in HS:
        for W in WS:
            ncol = int(rng.integers(1, 4))
            idx = rng.integers(0, ncol, size=(H, W))
            if dtype == np.uint8:
                img = idx.astype(np.uint8)
            else:
                img = rng.integers(0, 2**32, size=ncol, dtype=np.uint64).astype(np.uint32)[idx]
            ign = int(img.reshape(-1)[int(rng.integers(0, H * W))])
            check_case(ccl, f"ignore random {H}x{W} ncol={ncol}", img, conn, ignore=ign)
    # a colour the picture lacks changes nothing; a one-colour picture vanishes
    img = rng.integers(0, 3, size=(70, 130)).astype(dtype)
    check_case(ccl, "ignore an absent colour", img, conn, ignore=7)
    check_case(ccl, "ignore the only colour", np.full((70, 130), 2, dtype), conn, ignore=2)


@pytest.mark.parametrize("conn", [8, 4])
@pytest.mark.parametrize("dtype", [np.uint32, np.uint8])
def test_ignore_one_colour_tiles(ccl, conn, dtype):
    """Ignored one-colour tiles beside mixed tiles and one-colour tiles of other
    colours (the mosaics' solid colours are 7, 8 and 9)."""
    for name, img in mosaic_images().items():
        for ign in (7, 5, 3):
            check_case(ccl, f"ignore {ign}: {name}", img.astype(dtype), conn, ignore=ign)


@pytest.mark.parametrize("conn", [8, 4])
def test_ignore_structured(ccl, conn):
    for name, img in structured_images().items():
        check_case(ccl, f"ignore paper: {name}", img, conn, ignore=most_common_colour(img))


def test_ignore_batch_and_standalone_number(ccl):
    img = synth.bernoulli_batch(5, 100, 90, seed=9)
    check_case(ccl, "ignore 0: bernoulli batch 5x100x90", img, 8, ignore=0)
    img = synth.sheet_image(480, 700, seed=2)
    ign = most_common_colour(img)
    announce("number/count of an ignore leader image", img, 8, ign)
    L = oracle.label(img, 8, ignore=ign)
    exp_labels, exp_counts = oracle.number(L)
    Ld = torch.from_numpy(np.ascontiguousarray(L)).cuda()
    labels, counts = ccl.number(Ld)
    c2 = ccl.count(Ld)
    torch.cuda.synchronize()
    assert np.array_equal(labels.cpu().numpy(), exp_labels)
    assert int(counts.cpu()[0]) == int(exp_counts[0]) == int(c2.cpu()[0])


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_ignore_workload_full_size(ccl, config):
    """Every workload at full size with its most common colour ignored (the
    paper of the drawings, the background of the binary pictures)."""
    img = synth.generate(config)
    ign = most_common_colour(img)
    counts = check_case(ccl, f"ignore 0x{ign:x}, workload {config}: {synth.CONFIGS[config][0]}",
                        img, 8, ignore=ign)
    print(f"[gpu case] workload {config} regions per image, 0x{ign:x} ignored: "
          f"{counts[:4].tolist()}", flush=True)


# ------------------------------------------------- RGB pictures, three bytes

def check_rgb(ccl, name, img, conn=8, ignore=None):
    """An RGB picture ([.., H, W, 3] uint8) labelled in place against the oracle."""
    announce(f"rgb {name}", img, conn, ignore)
    exp_leaders = oracle.label(img, conn, ignore=ignore, rgb=True)
    exp_labels, exp_counts = oracle.number(exp_leaders)
    t = torch.from_numpy(np.ascontiguousarray(img)).cuda()
    leaders, c0 = ccl.label(t, conn, number=False, ignore=ignore, rgb=True)
    labels, c1 = ccl.label(t, conn, number=True, ignore=ignore, rgb=True)
    torch.cuda.synchronize()
    got = leaders.cpu().numpy()
    if not np.array_equal(got, exp_leaders):
        bad = np.argwhere(got != exp_leaders)
        raise AssertionError(f"rgb {name}: leaders differ at {len(bad)} pixels, first {bad[:5].tolist()}")
    assert np.array_equal(labels.cpu().numpy(), exp_labels), f"rgb {name}: numbers differ"
    assert np.array_equal(c0.cpu().numpy(), exp_counts) and np.array_equal(c1.cpu().numpy(), exp_counts)
    return exp_counts


def rgb_palette_image(rng, shape, ncol):
    """Colours that differ from one another in one byte only (each byte decides)."""
    base = rng.integers(0, 256, size=3)
    pal = np.tile(base, (ncol, 1))
    for k in range(1, ncol):
        pal[k, k % 3] = (base[k % 3] + 37 * k) % 256
    return pal[rng.integers(0, ncol, size=shape)].astype(np.uint8)


@pytest.mark.parametrize("conn", [8, 4])
def test_rgb_ragged_random(ccl, conn):
    """Ragged shapes, rows of every alignment (3*W mod 4), with and without an
    ignored colour."""
    rng = np.random.default_rng(300 + conn)
    for H in HS:
        for W in WS:
            img = rgb_palette_image(rng, (H, W), int(rng.integers(1, 5)))
            check_rgb(ccl, f"random {H}x{W}", img, conn)
            px = img[int(rng.integers(0, H)), int(rng.integers(0, W))]
            ign = int(px[0]) | (int(px[1]) << 8) | (int(px[2]) << 16)
            check_rgb(ccl, f"random {H}x{W}", img, conn, ignore=ign)


def test_rgb_structured_and_batch(ccl):
    for name, img in list(structured_images().items()) + list(mosaic_images().items()):
        if img.dtype != np.uint32:
            continue
        rgb = synth.rgb24(img)
        check_rgb(ccl, name, rgb, 8)
        # the same picture packed into 32 bits has the same regions
        assert np.array_equal(oracle.label(rgb, 8, rgb=True), oracle.label(img, 8))
    rng = np.random.default_rng(31)
    check_rgb(ccl, "batch 3x70x131", rgb_palette_image(rng, (3, 70, 131), 3), 8)


@pytest.mark.parametrize("config", [1, 3, 5])
def test_rgb_workload_full_size(ccl, config):
    """The colour workloads stored as RGB bytes at full size, with and without
    the paper (most common colour) ignored."""
    img = synth.generate(config)
    p = most_common_colour(img)                     # 0x00RRGGBB
    rgb = synth.rgb24(img)
    del img
    counts = check_rgb(ccl, f"workload {config}", rgb, 8)
    paper = ((p >> 16) & 0xFF) | (((p >> 8) & 0xFF) << 8) | ((p & 0xFF) << 16)  # bytes R, G, B
    check_rgb(ccl, f"workload {config}", rgb, 8, ignore=paper)
    print(f"[gpu case] rgb workload {config} regions: {counts[:4].tolist()}", flush=True)


# -------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_workload_full_size(ccl, config):
    img = synth.generate(config)
    counts = check_case(ccl, f"workload {config}: {synth.CONFIGS[config][0]}", img, 8)
    print(f"[gpu case] workload {config} regions per image: {counts[:4].tolist()}", flush=True)


# ------------------------------------------------------ region statistics

def check_stats(ccl, name, img, conn=8, ignore=None, rgb=False):
    """Per-region statistics on the GPU (of the GPU's own numbers, and of the
    oracle's numbers uploaded) equal the oracle's, entry for entry."""
    announce(f"stats {name}", img, conn, ignore)
    exp_labels, exp_counts = oracle.number(oracle.label(img, conn, ignore=ignore, rgb=rgb))
    exp = oracle.region_stats(exp_labels, exp_counts)
    t = torch.from_numpy(np.ascontiguousarray(img.view(np.int32) if img.dtype == np.uint32 else img)).cuda()
    labels, counts = ccl.label(t, conn, number=True, ignore=ignore, rgb=rgb)
    got = ccl.region_stats(labels, counts)
    up = torch.from_numpy(np.ascontiguousarray(exp_labels)).cuda()
    got2 = ccl.region_stats(up, torch.from_numpy(np.ascontiguousarray(exp_counts)).cuda(),
                            n_total=int(exp_counts.sum()))
    torch.cuda.synchronize()
    for key in ("area", "bbox", "sum_y", "sum_x"):
        for g in (got, got2):
            a = g[key].cpu().numpy()
            if not np.array_equal(a, exp[key]):
                bad = np.argwhere(a.reshape(len(a), -1) != exp[key].reshape(len(a), -1))
                raise AssertionError(f"stats {name}: {key} differs at {len(bad)} entries, "
                                     f"first {bad[:3].tolist()}")
    return exp_counts


def check_label_stats(ccl, name, img, conn=8, ignore=None, rgb=False, capacity=None):
    """ccl_label_stats (labels, counts and statistics in one call) equal the
    oracle's numbers and its statistics of them, entry for entry; with a
    capacity below the region count, only the records below it are written."""
    announce(f"label+stats {name}", img, conn, ignore)
    exp_labels, exp_counts = oracle.number(oracle.label(img, conn, ignore=ignore, rgb=rgb))
    exp = oracle.region_stats(exp_labels, exp_counts)
    n = int(exp_counts.sum())
    cap = n if capacity is None else capacity
    t = torch.from_numpy(np.ascontiguousarray(img.view(np.int32) if img.dtype == np.uint32 else img)).cuda()
    records = torch.full((max(n, cap, 1) + 3, 5), 0x5A5A5A5A, dtype=torch.int64, device="cuda")
    labels, counts, st = ccl.label_stats(t, cap, conn, ignore=ignore, rgb=rgb, records=records,
                                         trim=False, check=True)
    torch.cuda.synchronize()
    assert np.array_equal(labels.cpu().numpy(), exp_labels), f"label+stats {name}: numbers differ"
    assert np.array_equal(counts.cpu().numpy(), exp_counts), f"label+stats {name}: counts differ"
    got = {k: v.cpu().numpy() for k, v in st.items()}
    m = min(n, cap)
    for key in ("area", "bbox", "sum_y", "sum_x"):
        a = got[key][:m]
        e = exp[key][:m]
        if not np.array_equal(a, e):
            bad = np.argwhere(a.reshape(m, -1) != e.reshape(m, -1))
            raise AssertionError(f"label+stats {name}: {key} differs at {len(bad)} entries, "
                                 f"first {bad[:3].tolist()}")
    untouched = got["records"][m:]
    assert np.all(untouched == 0x5A5A5A5A), f"label+stats {name}: records past {m} written"
    return exp_counts


def test_label_stats_ragged_structured_batch(ccl):
    """Statistics in the labelling call: ragged shapes in every dtype and both
    connectivities, with and without an ignored colour, structured pictures,
    mosaics, a batch, RGB, and a 4-connected checkerboard (every pixel a region,
    many regions per tile, more than one pass over a tile's rows)."""
    rng = np.random.default_rng(700)
    for H, W in [(1, 1), (3, 700), (33, 65), (64, 64), (100, 129), (255, 513), (70, 90)]:
        for conn in (8, 4):
            img = rng.integers(0, 3, size=(H, W)).astype(np.uint8)
            check_label_stats(ccl, f"random u8 {H}x{W}", img, conn)
            check_label_stats(ccl, f"random u8 {H}x{W}", img, conn, ignore=0)
            col = rng.integers(0, 2**32, size=3, dtype=np.uint64).astype(np.uint32)
            check_label_stats(ccl, f"random u32 {H}x{W}", col[rng.integers(0, 3, size=(H, W))],
                              conn)
    for name, img in structured_images().items():
        check_label_stats(ccl, name, img, 8)
    for name, img in mosaic_images().items():
        check_label_stats(ccl, name, img, 8, ignore=7)
    check_label_stats(ccl, "bernoulli batch 5x100x90", synth.bernoulli_batch(5, 100, 90, seed=9), 8)
    check_label_stats(ccl, "bernoulli batch 7x64x64, 4-conn",
                      synth.bernoulli_batch(7, 64, 64, seed=4), 4, ignore=1)
    yy, xx = np.mgrid[0:300, 0:600]
    check_label_stats(ccl, "checkerboard 300x600 (every pixel a region)",
                      ((yy + xx) % 2).astype(np.uint8), 4)
    check_label_stats(ccl, "rgb drawing", synth.rgb24(synth.lines_image(256, 256, seed=1)), 8,
                      rgb=True)
    check_label_stats(ccl, "a uniform 20x30 image (one tile, one region)",
                      np.full((20, 30), 5, np.uint8), 8)


def test_label_stats_capacity(ccl):
    img = synth.lines_image(300, 400, seed=6)
    n = int(oracle.number(oracle.label(img, 8))[1].sum())
    for cap in (0, 1, n // 3, n - 1, n + 5):
        check_label_stats(ccl, f"drawing, capacity {cap} of {n}", img, 8, capacity=cap)


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_label_stats_workload_full_size(ccl, config):
    img = synth.generate(config)
    check_label_stats(ccl, f"workload {config}", img if img.shape[0] > 1 else img[0], 8)


@pytest.mark.parametrize("conn", [8, 4])
def test_stats_ragged_random(ccl, conn):
    """Shapes around the 512 x 256 areas of the statistics pass and the tiles."""
    rng = np.random.default_rng(400 + conn)
    for H, W in [(1, 1), (3, 700), (255, 513), (256, 512), (257, 511), (300, 1100), (70, 90)]:
        img = rng.integers(0, 3, size=(H, W)).astype(np.uint8)
        check_stats(ccl, f"random {H}x{W}", img, conn)
        check_stats(ccl, f"random {H}x{W}", img, conn, ignore=0)


def test_stats_structured_batch_and_overflow(ccl):
    for name, img in structured_images().items():
        check_stats(ccl, name, img, 8)
    for name, img in mosaic_images().items():
        check_stats(ccl, name, img, 8, ignore=7)
    check_stats(ccl, "bernoulli batch 5x100x90", synth.bernoulli_batch(5, 100, 90, seed=9), 8)
    # a 4-connected checkerboard: every pixel a region, 131072 labels in one
    # 512 x 256 area, far past the LDS table
    yy, xx = np.mgrid[0:300, 0:600]
    check_stats(ccl, "checkerboard 300x600 (every pixel a region)", ((yy + xx) % 2).astype(np.uint8), 4)
    rgb = synth.rgb24(synth.lines_image(256, 256, seed=1))
    check_stats(ccl, "rgb drawing", rgb, 8, rgb=True)


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_stats_workload_full_size(ccl, config):
    img = synth.generate(config)
    counts = check_stats(ccl, f"workload {config}: {synth.CONFIGS[config][0]}", img, 8)
    print(f"[gpu case] stats workload {config}: {int(counts.sum())} regions", flush=True)


# ------------------------------------------------------------ maximum size

def max_size_image(H: int, W: int) -> np.ndarray:
    """Diagonal bands crossed by a coarse checker, with a vertical line every
    4099 columns: regions that run through thousands of tiles, diagonal
    contacts, at every tile position of a maximum-size image (built in row
    chunks of 32-bit arithmetic)."""
    img = np.empty((H, W), np.uint8)
    x = np.arange(W, dtype=np.int32)[None, :]
    for y0 in range(0, H, 2048):
        y = np.arange(y0, min(H, y0 + 2048), dtype=np.int32)[:, None]
        a = ((x * 3 + y * 5) // 211) & 1
        b = ((x // 997) + (y // 613)) & 1
        img[y0:y0 + y.shape[0]] = ((a ^ b) + 2 * (x % 4099 == 0)).astype(np.uint8)
    return img


def test_maximum_size_image(ccl):
    """46340 x 46340 (2^31 - 87887 pixels, the largest square whose reading-order
    indices fit int32): leaders, numbers and counts bit-exact with the oracle,
    so no index of the path overflows at the limit."""
    H = W = 46340
    assert H * W <= 2**31 - 1
    img = max_size_image(H, W)
    counts = check_case(ccl, "maximum size 46340x46340", img, 8)
    print(f"[gpu case] maximum size regions: {counts.tolist()}", flush=True)


# ----------------------------------------------------- standalone number/count

def test_number_and_count_standalone(ccl):
    for name, img in [("sheet", synth.sheet_image(480, 700, seed=2)),
                      ("bernoulli", synth.bernoulli_batch(4, 130, 77, seed=5))]:
        announce(f"number/count {name}", img, 8)
        L = oracle.label(img, 8)
        exp_labels, exp_counts = oracle.number(L)
        Ld = torch.from_numpy(np.ascontiguousarray(L)).cuda()
        labels, counts = ccl.number(Ld)
        c2 = ccl.count(Ld)
        torch.cuda.synchronize()
        assert np.array_equal(labels.cpu().numpy(), exp_labels)
        assert np.array_equal(np.atleast_1d(counts.cpu().numpy()), np.atleast_1d(exp_counts))
        assert np.array_equal(np.atleast_1d(c2.cpu().numpy()), np.atleast_1d(oracle.count(L)))
        # in place
        labels2, _ = ccl.number(Ld, inplace=True)
        torch.cuda.synchronize()
        assert np.array_equal(Ld.cpu().numpy(), exp_labels)


def test_number_rejects_out_of_range_leaders_safely(ccl):
    L = np.arange(64 * 70, dtype=np.int32).reshape(64, 70)
    L[3, 4] = -5
    L[5, 6] = 64 * 70 + 100
    announce("number out-of-range leaders", L, 8)
    labels, counts = ccl.number(torch.from_numpy(L).cuda())
    got = labels.cpu().numpy()
    assert got[3, 4] == 0 and got[5, 6] == 0
    ok = np.ones_like(L, bool)
    ok[3, 4] = ok[5, 6] = False
    # the remaining pixels lead themselves except the two bad ones
    assert np.array_equal(np.sort(got[ok]), np.arange(1, 64 * 70 - 1))


# ----------------------------------------------- determinism, streams, sizes

def test_repeat_calls_are_identical(ccl):
    img = synth.spiral_image(1024, 1024, seed=3)
    announce("determinism spiral 1024", img, 8)
    t = to_device(img)
    ref, _ = ccl.label(t, 8, number=True)
    ref = ref.clone()
    ws = torch.zeros(ccl.workspace_bytes(1, 1024, 1024), dtype=torch.uint8, device="cuda")
    for _ in range(20):
        out, _ = ccl.label(t, 8, number=True, workspace=ws)
        assert torch.equal(out, ref)
    assert ccl.error_word(ws) == 0


def test_side_stream_and_reused_workspace(ccl):
    imgs = [synth.lines_image(256, 256, seed=s) for s in (1, 2)]
    announce("side stream", imgs[0], 8)
    s = torch.cuda.Stream()
    ws = torch.zeros(ccl.workspace_bytes(1, 256, 256), dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(s):
        outs = [ccl.label(to_device(im), 8, number=True, stream=s, workspace=ws)[0].clone()
                for im in imgs]
    s.synchronize()
    for im, o in zip(imgs, outs):
        exp, _ = oracle.number(oracle.label(im, 8))
        assert np.array_equal(o.cpu().numpy(), exp)


def test_two_streams_at_once(ccl):
    """Calls on two streams in flight together, each with its own workspace,
    on different images (the spiral and the u8 batch, whose seam passes run
    long), repeated so that they overlap; every result against the oracle."""
    work = [synth.spiral_image(2048, 2048, seed=3), synth.bernoulli_batch(8, 512, 512, seed=2)]
    exp = []
    for im in work:
        announce("two streams at once", im, 8)
        exp.append(oracle.number(oracle.label(im, 8)))
    devs = [to_device(im) for im in work]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    labs = [ccl.Labeller(tuple((im if im.ndim == 3 else im[None]).shape), device="cuda")
            for im in work]
    outs = [[], []]
    torch.cuda.synchronize()
    for _ in range(4):
        for k in (0, 1):  # enqueue both before waiting on either
            labs[k](devs[k], number=True, stream=streams[k])
            with torch.cuda.stream(streams[k]):
                outs[k].append((labs[k].out.clone(), labs[k].counts.clone()))
    torch.cuda.synchronize()
    for k in (0, 1):
        assert ccl.error_word(labs[k].workspace) == 0
        el, ec = exp[k]
        for o, c in outs[k]:
            assert np.array_equal(o.cpu().numpy().reshape(el.shape), el), f"stream {k}: labels"
            assert np.array_equal(c.cpu().numpy(), ec), f"stream {k}: counts"


def test_error_word_is_cleared_by_each_call(ccl):
    """Each call clears the workspace's error word first: a workspace full of
    ones still reads 0 after a good call, and check=True passes."""
    img = synth.lines_image(300, 500, seed=8)
    announce("error word cleared", img, 8)
    ws = torch.full((ccl.workspace_bytes(1, 300, 500),), 0xFF, dtype=torch.uint8, device="cuda")
    out, c = ccl.label(to_device(img), 8, number=True, workspace=ws, check=True)
    assert ccl.error_word(ws) == 0
    exp, ec = oracle.number(oracle.label(img, 8))
    assert np.array_equal(out.cpu().numpy(), exp) and np.array_equal(c.cpu().numpy(), ec)
    # ccl_number / ccl_count clear it too
    leaders, _ = ccl.label(to_device(img), 8)
    ws.fill_(0xFF)
    ccl.number(leaders, workspace=ws)
    torch.cuda.synchronize()
    assert ccl.error_word(ws) == 0


def test_empty_inputs(ccl):
    for shape in [(0, 5, 5), (2, 0, 7), (3, 4, 0)]:
        img = torch.zeros(shape, dtype=torch.uint8, device="cuda")
        out, counts = ccl.label(img, 8, number=True)
        torch.cuda.synchronize()
        assert out.shape == shape
        assert counts.cpu().tolist() == [0] * shape[0]
