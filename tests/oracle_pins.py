"""Checks that pin the CPU oracle to things other than itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle library it is
given disagrees with:
  * values printed for the pages' worked examples (``tests/golden/``),
  * an independent labeller (breadth-first flood fill -- in pure Python, and the
    C one built from the unmodified oracle source),
  * scipy's binary labelling run once per colour (the "one colour at a time"
    approach of "Accountable AI starts at the pixel", ch.03), compared as a
    partition,
  * closed forms (uniform, checkerboard, stripes, single rows, no row wrap),
  * for one ignored colour ("Accountable AI starts at the pixel", ch.08 idea 4):
    the TorchCC page's "Find(i) + 1, 0 for background" labels, a flood fill
    that skips the ignored colour, and scipy's binary labelling (whose numbers
    are 1..n in reading order, 0 for background) value for value,
  * for RGB pictures stored as three bytes per pixel (same page, ch.08-09): a
    flood fill comparing the three bytes as a tuple,
  * for the 64-bit entry points (images beyond 2^31 pixels): the flood fill
    and the closed form of horizontal stripes,
  * per-region statistics: the hand-derived areas, boxes and index sums of the
    TorchCC example's components, and scipy's find_objects / sum_labels /
    center_of_mass on random labellings,
  * invariants of the definition (leader = region minimum, equal-colour
    neighbours share a leader, numbers are 1..n in reading order).

``tests/test_oracle_pins.py`` runs them on the oracle; ``tests/test_oracle_mutants.py``
runs them on builds with planted mistakes and requires each to be caught.
"""
from __future__ import annotations

import itertools
from collections import deque

import numpy as np
import scipy.ndimage as ndi

import oracle
from tests.golden import fixtures

NB8 = [(-1, -1), (-1, 0), (-1, 1), (0, -1), (0, 1), (1, -1), (1, 0), (1, 1)]
NB4 = [(-1, 0), (0, -1), (0, 1), (1, 0)]


def py_bfs(img: np.ndarray, conn: int) -> np.ndarray:
    """Pure-Python flood fill, seeds in reading order (independent of the C file)."""
    H, W = img.shape
    nb = NB8 if conn == 8 else NB4
    lab = np.full((H, W), -1, dtype=np.int64)
    for s in range(H * W):
        r0, c0 = divmod(s, W)
        if lab[r0, c0] >= 0:
            continue
        v = img[r0, c0]
        lab[r0, c0] = s
        q = deque([(r0, c0)])
        while q:
            r, c = q.popleft()
            for dr, dc in nb:
                rr, cc = r + dr, c + dc
                if 0 <= rr < H and 0 <= cc < W and lab[rr, cc] < 0 and img[rr, cc] == v:
                    lab[rr, cc] = s
                    q.append((rr, cc))
    return lab.astype(np.int32)


def py_bfs_ignore(img: np.ndarray, conn: int, ignore) -> np.ndarray:
    """Pure-Python flood fill in which pixels of colour ``ignore`` are -1 and are
    neither seeds nor reached (independent of the C file)."""
    H, W = img.shape
    nb = NB8 if conn == 8 else NB4
    lab = np.full((H, W), -1, dtype=np.int64)
    for s in range(H * W):
        r0, c0 = divmod(s, W)
        v = img[r0, c0]
        if lab[r0, c0] >= 0 or v == ignore:
            continue
        lab[r0, c0] = s
        q = deque([(r0, c0)])
        while q:
            r, c = q.popleft()
            for dr, dc in nb:
                rr, cc = r + dr, c + dc
                if 0 <= rr < H and 0 <= cc < W and lab[rr, cc] < 0 and img[rr, cc] == v:
                    lab[rr, cc] = s
                    q.append((rr, cc))
    return lab.astype(np.int32)


def random_images(rng, B, H, W, ncol, dtype=np.uint32):
    """Small random images with ``ncol`` distinct values; u32 values use all bytes."""
    idx = rng.integers(0, ncol, size=(B, H, W))
    if dtype == np.uint8:
        return idx.astype(np.uint8)
    palette = rng.integers(0, 2**32, size=ncol, dtype=np.uint64).astype(np.uint32)
    return palette[idx]


def check_invariants(img: np.ndarray, leaders: np.ndarray, conn: int):
    """Definition-level properties of a leader image, checked with numpy only."""
    H, W = img.shape
    n = H * W
    L = leaders.reshape(-1).astype(np.int64)
    flat = img.reshape(-1)
    idx = np.arange(n)
    assert np.all(L >= 0) and np.all(L <= idx), "leader must be an earlier-or-same pixel"
    assert np.all(L[L] == L), "a leader must lead itself"
    assert np.all(flat[L] == flat), "a pixel and its leader must have the same colour"
    # equal-colour neighbours share a leader (no row wrap: 2-D offsets only)
    offs = [(0, 1), (1, 0)] + ([(1, 1), (1, -1)] if conn == 8 else [])
    Li = leaders.reshape(H, W)
    for dr, dc in offs:
        r0, r1 = 0, H - dr
        c0, c1 = max(0, -dc), W - max(0, dc)
        if r1 <= r0 or c1 <= c0:
            continue
        a = img[r0:r1, c0:c1]
        b = img[r0 + dr:r1 + dr, c0 + dc:c1 + dc]
        la = Li[r0:r1, c0:c1]
        lb = Li[r0 + dr:r1 + dr, c0 + dc:c1 + dc]
        same = a == b
        assert np.all(la[same] == lb[same]), f"equal-colour neighbours at offset {(dr, dc)} split"


def check_numbering(leaders: np.ndarray, labels: np.ndarray, count: int):
    """Numbers are 1..n, in reading order of the leaders (sort-based check)."""
    L = leaders.reshape(-1)
    uniq = np.unique(L)                       # sorted leaders
    expect = np.searchsorted(uniq, L) + 1     # rank among leaders, from 1
    assert count == uniq.size, "count must be the number of distinct leaders"
    assert np.array_equal(labels.reshape(-1), expect), "numbering is not 1 + leaders before"
    if labels.size:
        lab = labels.reshape(-1)
        first = np.full(count + 1, lab.size)
        np.minimum.at(first, lab, np.arange(lab.size))   # first occurrence of each number
        assert np.all(np.diff(first[1:]) > 0), "first occurrences not in reading order"


# ---------------------------------------------------------------------------
# worked examples from the pages

def pin_torchcc_4x4(lib):
    fx = fixtures.load("torchcc_4x4_binary.txt")
    img = fx["input"].astype(np.uint8)
    P = oracle.connect(img, 8, lib=lib).reshape(-1)
    for item in fx["scan_parent_foreground"].split():
        i, p = (int(v) for v in item.split(":"))
        assert P[i] == p, f"parent of {i} after the scan: {P[i]} != {p} (page)"
    L = oracle.label(img, 8, lib=lib).reshape(-1)
    fg = np.flatnonzero(img.reshape(-1) == 1)
    roots = sorted(set(int(v) for v in L[fg]))
    assert roots == [int(v) for v in fx["roots_foreground"].split()]
    assert [r + 1 for r in roots] == [int(v) for v in fx["labels_foreground_root_plus_one"].split()]


def pin_every_colour_3x3(lib):
    fx = fixtures.load("every_colour_3x3_reconstruction.txt")
    img = fx["input"]
    P = oracle.connect(img, 8, lib=lib).reshape(-1)
    assert P[5] == int(fx["after_connect_parent_5"]), "pixel 5 must point at 2 after Connect"
    assert P[2] == int(fx["after_connect_parent_2"]), "leader 2 must be re-pointed at 0"
    L = oracle.label(img, 8, lib=lib).reshape(-1)
    # both arms of colour X form one region led by 0; pixel 2 is not left behind
    assert set(L[[0, 2, 3, 5, 7]]) == {0}
    assert set(L[[1, 4, 6, 8]]) == {1}


def pin_torchcc_6x6(lib):
    fx = fixtures.load("torchcc_6x6_binary.txt")
    img = fx["input"].astype(np.uint8)
    for conn in (8, 4):
        L = oracle.label(img, conn, lib=lib)
        assert np.array_equal(L, py_bfs(img, conn))
    # the page's block init labels are the raster index of each 2x2 block's top-left pixel
    blocks = [int(v) for v in fx["block_init_labels"].split()]
    assert blocks == [r * 6 + c for r in range(0, 6, 2) for c in range(0, 6, 2)]


def pin_ignore_torchcc_4x4(lib):
    """The page's labels with background ignored are leader + 1, 0 for background."""
    fx = fixtures.load("torchcc_4x4_binary.txt")
    img = fx["input"].astype(np.uint8)
    L = oracle.label(img, 8, lib=lib, ignore=0)
    expect = np.array([int(v) for v in fx["labels_find_plus_one_raster"].split()])
    assert np.array_equal(L.reshape(-1) + 1, expect), "leader + 1 must be the page's labels"
    labels, counts = oracle.number(L, lib=lib)
    assert counts[0] == 3, "three components besides the background"
    # numbers keep 0 for background and count the components 1, 2, 3 in reading order
    assert np.array_equal(labels.reshape(-1), [1, 1, 0, 1, 0, 0, 1, 0, 0, 0, 0, 0, 2, 0, 0, 3])
    # u32 view of the same picture: the whole stored value is compared
    L32 = oracle.label(img.astype(np.uint32) * 0x01010101, 8, lib=lib, ignore=0)
    assert np.array_equal(L32, L)


# ---------------------------------------------------------------------------
# independent labellers

def pin_random_vs_python_bfs(lib, n_images=300, seed=11):
    rng = np.random.default_rng(seed)
    for k in range(n_images):
        H, W = int(rng.integers(1, 13)), int(rng.integers(1, 13))
        ncol = int(rng.integers(1, 5))
        dt = np.uint8 if k % 2 else np.uint32
        img = random_images(rng, 1, H, W, ncol, dt)[0]
        conn = 8 if k % 3 else 4
        L = oracle.label(img, conn, lib=lib)
        assert np.array_equal(L, py_bfs(img, conn)), f"case {k}: {H}x{W} conn {conn}"


def pin_random_vs_c_bfs(lib, ref_lib=None, seed=12, per_shape=200):
    """Many random images against the C flood fill of ``ref_lib``."""
    ref_lib = ref_lib or lib
    rng = np.random.default_rng(seed)
    shapes = [(1, 1), (1, 24), (24, 1), (2, 2), (3, 7), (7, 3), (5, 5), (8, 13),
              (16, 16), (24, 24), (17, 23), (23, 17)]
    for H, W in shapes:
        for ncol in (1, 2, 3, 4):
            for dt in (np.uint8, np.uint32):
                imgs = random_images(rng, per_shape, H, W, ncol, dt)
                for conn in (8, 4):
                    a = oracle.label(imgs, conn, lib=lib)
                    b = oracle.bfs_label(imgs, conn, lib=ref_lib)
                    assert np.array_equal(a, b), f"{H}x{W} ncol={ncol} {dt.__name__} conn={conn}"


def pin_exhaustive(lib, ref_lib=None):
    """Every 3-colour 3x3 image and every 2-colour 4x4 image, both connectivities."""
    ref_lib = ref_lib or lib
    for H, W, ncol in ((3, 3, 3), (4, 4, 2)):
        imgs = np.array(list(itertools.product(range(ncol), repeat=H * W)),
                        dtype=np.uint8).reshape(-1, H, W)
        for conn in (8, 4):
            a = oracle.label(imgs, conn, lib=lib)
            b = oracle.bfs_label(imgs, conn, lib=ref_lib)
            assert np.array_equal(a, b), f"exhaustive {H}x{W} conn={conn}"


def pin_scipy_partition(lib, seed=13, n_images=60):
    """Per-colour binary labelling (scipy) must give the same partition."""
    rng = np.random.default_rng(seed)
    for k in range(n_images):
        H, W = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        img = random_images(rng, 1, H, W, int(rng.integers(1, 6)))[0]
        for conn in (8, 4):
            L = oracle.label(img, conn, lib=lib)
            structure = np.ones((3, 3)) if conn == 8 else ndi.generate_binary_structure(2, 1)
            region = np.full((H, W), -1, dtype=np.int64)
            base = 0
            for v in np.unique(img):
                lab, n = ndi.label(img == v, structure=structure)
                m = lab > 0
                region[m] = lab[m] - 1 + base
                base += n
            # same partition: the maps region -> leader and leader -> region are functions
            pairs = np.unique(np.stack([region.reshape(-1), L.reshape(-1)]), axis=1)
            assert pairs.shape[1] == base == np.unique(L).size, f"case {k} conn {conn}"
            # and each region's leader is its smallest index
            flat = np.arange(H * W)
            mins = np.full(base, H * W)
            np.minimum.at(mins, region.reshape(-1), flat)
            assert np.array_equal(L.reshape(-1), mins[region.reshape(-1)])


def pin_ignore_vs_python_bfs(lib, n_images=300, seed=15):
    """One ignored colour: leaders against a flood fill that skips it; numbers
    and counts over the other regions only."""
    rng = np.random.default_rng(seed)
    for k in range(n_images):
        H, W = int(rng.integers(1, 14)), int(rng.integers(1, 14))
        ncol = int(rng.integers(1, 5))
        dt = np.uint8 if k % 2 else np.uint32
        img = random_images(rng, 1, H, W, ncol, dt)[0]
        conn = 8 if k % 3 else 4
        # usually a colour of the picture; now and then one it does not contain
        ign = img.reshape(-1)[int(rng.integers(0, H * W))] if k % 5 else int(img.max()) + 1
        L = oracle.label(img, conn, lib=lib, ignore=ign)
        E = py_bfs_ignore(img, conn, ign)
        assert np.array_equal(L, E), f"case {k}: {H}x{W} conn {conn} ignore {ign}"
        labels, counts = oracle.number(L, lib=lib)
        kept = E.reshape(-1) >= 0
        uniq = np.unique(E.reshape(-1)[kept])
        exp_num = np.zeros(H * W, np.int64)
        exp_num[kept] = np.searchsorted(uniq, E.reshape(-1)[kept]) + 1
        assert np.array_equal(labels.reshape(-1), exp_num), f"case {k}: numbers"
        assert counts[0] == uniq.size and oracle.count(L, lib=lib)[0] == uniq.size


def pin_ignore_scipy_binary(lib, seed=16, n_images=150):
    """Binary pictures with 0 ignored: numbers equal scipy's labelling value for
    value (scipy numbers components 1..n in reading order of their first pixel,
    background 0), at every foreground density."""
    rng = np.random.default_rng(seed)
    for k in range(n_images):
        H, W = int(rng.integers(1, 48)), int(rng.integers(1, 48))
        p = 0.05 + 0.9 * (k % 19) / 18
        img = (rng.random((H, W)) < p).astype(np.uint8)
        for conn in (8, 4):
            structure = np.ones((3, 3)) if conn == 8 else ndi.generate_binary_structure(2, 1)
            lab, n = ndi.label(img, structure=structure)
            L = oracle.label(img, conn, lib=lib, ignore=0)
            labels, counts = oracle.number(L, lib=lib)
            assert np.array_equal(labels, lab), f"case {k} conn {conn}: numbers differ from scipy"
            assert counts[0] == n, f"case {k} conn {conn}: count differs from scipy"
    # a batch: every image numbered on its own from 1
    imgs = (rng.random((4, 20, 30)) < 0.4).astype(np.uint8)
    labels, counts = oracle.number(oracle.label(imgs, 8, lib=lib, ignore=0), lib=lib)
    for b in range(4):
        lab, n = ndi.label(imgs[b], structure=np.ones((3, 3)))
        assert np.array_equal(labels[b], lab) and counts[b] == n


def pin_ignore_leaves_other_regions(lib, seed=17, n_images=100):
    """Regions never mix colours, so ignoring one colour changes no other
    pixel's leader; ignoring a colour the picture lacks changes nothing; an
    all-ignored picture has no regions."""
    rng = np.random.default_rng(seed)
    for k in range(n_images):
        H, W = int(rng.integers(1, 30)), int(rng.integers(1, 30))
        img = random_images(rng, 1, H, W, int(rng.integers(1, 5)),
                            np.uint32 if k % 2 else np.uint8)[0]
        conn = 8 if k % 2 else 4
        full = oracle.label(img, conn, lib=lib)
        ign = img.reshape(-1)[int(rng.integers(0, H * W))]
        L = oracle.label(img, conn, lib=lib, ignore=ign)
        keep = img != ign
        assert np.array_equal(L[keep], full[keep]) and np.all(L[~keep] == -1)
        # regions of the ignored colour, counted by scipy, are exactly the ones lost
        structure = np.ones((3, 3)) if conn == 8 else ndi.generate_binary_structure(2, 1)
        _, n_ign = ndi.label(~keep, structure=structure)
        assert oracle.count(L, lib=lib)[0] == oracle.count(full, lib=lib)[0] - n_ign
    img = np.full((5, 7), 9, np.uint8)
    L = oracle.label(img, 8, lib=lib, ignore=9)
    labels, counts = oracle.number(L, lib=lib)
    assert np.all(L == -1) and np.all(labels == 0) and counts[0] == 0
    L = oracle.label(img, 8, lib=lib, ignore=8)
    assert np.all(L == 0)


def rgb_tuples(img: np.ndarray) -> np.ndarray:
    """[H, W] object array of (b0, b1, b2) tuples: colours compared as tuples,
    with no packing into one number."""
    H, W, _ = img.shape
    out = np.empty((H, W), dtype=object)
    for r in range(H):
        for c in range(W):
            out[r, c] = tuple(int(v) for v in img[r, c])
    return out


def random_rgb(rng, B, H, W, ncol):
    """Random RGB pictures whose ``ncol`` colours differ from one another in one
    byte only (which byte varies per colour), so every byte decides."""
    base = rng.integers(0, 256, size=3)
    pal = np.tile(base, (ncol, 1))
    for k in range(1, ncol):
        pal[k, k % 3] = (base[k % 3] + k) % 256
    return pal[rng.integers(0, ncol, size=(B, H, W))].astype(np.uint8)


def pin_rgb_vs_python_bfs(lib, n_images=240, seed=18):
    """Three-byte pixels: leaders against a flood fill over byte tuples, both
    connectivities, with and without an ignored colour; a batch is labelled
    image by image."""
    rng = np.random.default_rng(seed)
    for k in range(n_images):
        H, W = int(rng.integers(1, 13)), int(rng.integers(1, 13))
        img = random_rgb(rng, 1, H, W, int(rng.integers(1, 5)))[0]
        conn = 8 if k % 3 else 4
        T = rgb_tuples(img)
        L = oracle.label(img, conn, lib=lib, rgb=True)
        assert np.array_equal(L, py_bfs(T, conn)), f"case {k}: {H}x{W} conn {conn}"
        if k % 2:
            r, c = int(rng.integers(0, H)), int(rng.integers(0, W))
            ign = int(img[r, c, 0]) | (int(img[r, c, 1]) << 8) | (int(img[r, c, 2]) << 16)
            L = oracle.label(img, conn, lib=lib, rgb=True, ignore=ign)
            assert np.array_equal(L, py_bfs_ignore(T, conn, T[r, c])), f"case {k}: ignore"
    imgs = random_rgb(rng, 3, 9, 11, 3)
    L = oracle.label(imgs, 8, lib=lib, rgb=True)
    for b in range(3):
        assert np.array_equal(L[b], py_bfs(rgb_tuples(imgs[b]), 8))


def pin_stats_torchcc_4x4(lib):
    """Statistics of the TorchCC example's three components (background
    ignored), against values worked out by hand from the page's labelling."""
    fx = fixtures.load("torchcc_4x4_binary.txt")
    img = fx["input"].astype(np.uint8)
    labels, counts = oracle.number(oracle.label(img, 8, lib=lib, ignore=0), lib=lib)
    st = oracle.region_stats(labels, counts, lib=lib)
    ints = lambda k: [int(v) for v in fx[k].split()]
    assert st["area"].tolist() == ints("stats_area")
    assert st["bbox"].reshape(-1).tolist() == ints("stats_bbox")
    assert st["sum_y"].tolist() == ints("stats_sum_y")
    assert st["sum_x"].tolist() == ints("stats_sum_x")


def pin_stats_vs_scipy(lib, seed=19, n_images=80):
    """Area, bounding box and index sums of every region against scipy's
    find_objects (boxes), sum_labels over ones and over the row / column index
    grids (areas and sums, exact in float64 at these sizes) and center_of_mass,
    with and without an ignored colour; a batch is concatenated image by image."""
    rng = np.random.default_rng(seed)
    for k in range(n_images):
        H, W = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        img = random_images(rng, 1, H, W, int(rng.integers(1, 5)), np.uint8)[0]
        ign = int(img.reshape(-1)[0]) if k % 2 else None
        labels, counts = oracle.number(oracle.label(img, 8 if k % 3 else 4, lib=lib, ignore=ign),
                                       lib=lib)
        n = int(counts[0])
        st = oracle.region_stats(labels, counts, lib=lib)
        idx = np.arange(1, n + 1)
        yy, xx = np.mgrid[0:H, 0:W]
        ones = np.ones((H, W))
        assert np.array_equal(st["area"], ndi.sum_labels(ones, labels, idx).astype(np.int64))
        assert np.array_equal(st["sum_y"], ndi.sum_labels(yy, labels, idx).astype(np.int64))
        assert np.array_equal(st["sum_x"], ndi.sum_labels(xx, labels, idx).astype(np.int64))
        boxes = ndi.find_objects(labels, max_label=n)
        none = [2147483647, 2147483647, -1, -1]  # a number with no pixels
        exp = np.array([none if b is None else [b[0].start, b[1].start, b[0].stop - 1, b[1].stop - 1]
                        for b in boxes], dtype=np.int64).reshape(-1, 4)
        assert np.array_equal(st["bbox"], exp), f"case {k}: boxes"
        if n:
            with np.errstate(invalid="ignore", divide="ignore"):  # (a mutant's empty region)
                com = np.array(ndi.center_of_mass(ones, labels, idx)).reshape(-1, 2)
                got = np.stack([st["sum_y"] / st["area"], st["sum_x"] / st["area"]], axis=1)
            assert np.allclose(got, com, rtol=0, atol=1e-9)
    imgs = random_images(rng, 3, 12, 17, 3, np.uint8)
    labels, counts = oracle.number(oracle.label(imgs, 8, lib=lib), lib=lib)
    st = oracle.region_stats(labels, counts, lib=lib)
    off = 0
    for b in range(3):
        one = oracle.region_stats(labels[b], counts[b:b + 1], lib=lib)
        n = int(counts[b])
        for key in ("area", "bbox", "sum_y", "sum_x"):
            assert np.array_equal(st[key][off:off + n], one[key])
        off += n


# ---------------------------------------------------------------------------
# closed forms and special cases

def pin_closed_forms(lib):
    for conn in (8, 4):
        # uniform image: one region led by pixel 0
        for H, W in ((1, 1), (1, 9), (9, 1), (7, 11)):
            L = oracle.label(np.full((H, W), 0xABCDEF12, np.uint32), conn, lib=lib)
            assert np.all(L == 0)
            _, c = oracle.number(L, lib=lib)
            assert c[0] == 1
        # vertical stripes of alternating colours: W regions, leader = column index
        H, W = 6, 9
        img = np.tile((np.arange(W) % 2).astype(np.uint8), (H, 1))
        L = oracle.label(img, conn, lib=lib)
        assert np.array_equal(L, np.tile(np.arange(W, dtype=np.int32), (H, 1)))
        labels, c = oracle.number(L, lib=lib)           # numbers 1..W left to right
        assert c[0] == W and np.array_equal(labels, L + 1)
        # single row: regions = colour changes + 1
        row = np.array([[3, 3, 1, 1, 1, 3, 2, 2, 3, 3]], np.uint8)
        L = oracle.label(row, conn, lib=lib)
        assert np.array_equal(L[0], [0, 0, 2, 2, 2, 5, 6, 6, 8, 8])
        # no join across a row end: (r, W-1) and (r+1, 0) only touch in the flat index
        img = np.zeros((3, 4), np.uint8)
        img[0, 3] = 1
        img[1, 0] = 1
        L = oracle.label(img, conn, lib=lib)
        assert L[0, 3] == 3 and L[1, 0] == 4
    # checkerboard: 8-connectivity joins the diagonals (2 regions), 4 does not
    for H, W in ((2, 2), (5, 6), (8, 8)):
        cb = ((np.add.outer(np.arange(H), np.arange(W))) % 2).astype(np.uint8)
        L8 = oracle.label(cb, 8, lib=lib)
        assert np.unique(L8).tolist() == [0, 1]
        L4 = oracle.label(cb, 4, lib=lib)
        assert np.array_equal(L4.reshape(-1), np.arange(H * W))
    # colours differing only in their high bytes are different colours
    img = np.array([[0x00000001, 0x01000001], [0x00010001, 0x00000001]], np.uint32)
    L = oracle.label(img, 8, lib=lib)
    assert L.reshape(-1).tolist() == [0, 1, 2, 0]
    # empty inputs
    assert oracle.label(np.zeros((0, 5, 5), np.uint8), 8, lib=lib).shape == (0, 5, 5)
    assert oracle.label(np.zeros((2, 0, 5), np.uint8), 8, lib=lib).shape == (2, 0, 5)
    _, c = oracle.number(np.zeros((2, 0, 5), np.int32), lib=lib)
    assert c.tolist() == [0, 0]


def pin_wide_vs_python_bfs(lib, n_images=160, seed=20):
    """64-bit leaders and numbers (oracle_label64 / oracle_number64, the entry
    points for images beyond 2^31 pixels) against the pure-Python flood fill,
    with and without an ignored colour, in every pixel type; and the closed
    form of horizontal stripes (row r of its own colour: leader r*W, number
    r+1), whose leaders use every index width the image has."""
    rng = np.random.default_rng(seed)
    for k in range(n_images):
        H, W = int(rng.integers(1, 24)), int(rng.integers(1, 24))
        conn = 8 if k % 2 else 4
        kind = k % 3
        if kind == 2:
            imgs = random_rgb(rng, 1, H, W, int(rng.integers(1, 5)))
            T = rgb_tuples(imgs[0])
            img, rgb = imgs[0], True
        else:
            img = random_images(rng, 1, H, W, int(rng.integers(1, 5)),
                                np.uint8 if kind == 0 else np.uint32)[0]
            T, rgb = img, False
        L = oracle.label64(img, conn, lib=lib, rgb=rgb)
        assert L.dtype == np.int64
        assert np.array_equal(L, py_bfs(T, conn)), f"case {k}: {H}x{W} conn {conn}"
        labels, counts = oracle.number64(L, lib=lib)
        assert labels.dtype == np.int64 and counts.dtype == np.int64
        check_numbering(L, labels, int(counts[0]))
        r, c = int(rng.integers(0, H)), int(rng.integers(0, W))
        ign = img[r, c]
        ign_v = int(ign[0]) | int(ign[1]) << 8 | int(ign[2]) << 16 if rgb else int(ign)
        L = oracle.label64(img, conn, lib=lib, ignore=ign_v, rgb=rgb)
        E = py_bfs_ignore(T, conn, T[r, c])
        assert np.array_equal(L, E), f"case {k}: ignore"
        labels, counts = oracle.number64(L, lib=lib)
        keep = L >= 0
        assert np.all(labels[~keep] == 0)
        uniq = np.unique(L[keep])
        assert counts[0] == uniq.size
        assert np.array_equal(labels[keep], np.searchsorted(uniq, L[keep]) + 1)
    # a batch: indices per image, counts per image
    imgs = random_images(rng, 4, 11, 13, 3)
    L = oracle.label64(imgs, 8, lib=lib)
    _, counts = oracle.number64(L, lib=lib)
    for b in range(4):
        E = py_bfs(imgs[b], 8)
        assert np.array_equal(L[b], E)
        assert counts[b] == np.unique(E).size
    # horizontal stripes: rows alternate two colours, so no row touches a row
    # of its colour (diagonals included); leader (r, c) = r*W, number r+1
    for H, W in ((7, 5), (40, 3)):
        img = np.repeat((np.arange(H) % 2).astype(np.uint8)[:, None], W, axis=1)
        for conn in (8, 4):
            L = oracle.label64(img, conn, lib=lib)
            assert np.array_equal(L, np.repeat(np.arange(H, dtype=np.int64)[:, None] * W, W, 1))
            labels, counts = oracle.number64(L, lib=lib)
            assert counts[0] == H and np.array_equal(labels, L // W + 1)


def pin_invariants_and_numbering(lib, seed=14, n_images=200):
    rng = np.random.default_rng(seed)
    for k in range(n_images):
        H, W = int(rng.integers(1, 30)), int(rng.integers(1, 30))
        img = random_images(rng, 1, H, W, int(rng.integers(1, 5)),
                            np.uint32 if k % 2 else np.uint8)[0]
        conn = 8 if k % 2 else 4
        L = oracle.label(img, conn, lib=lib)
        check_invariants(img, L, conn)
        labels, counts = oracle.number(L, lib=lib)
        check_numbering(L, labels, int(counts[0]))
        assert oracle.count(L, lib=lib)[0] == counts[0]
    # batches: each image is labelled on its own, indices per image
    imgs = random_images(rng, 5, 9, 7, 3)
    L = oracle.label(imgs, 8, lib=lib)
    for b in range(5):
        assert np.array_equal(L[b], oracle.label(imgs[b], 8, lib=lib))


ALL_PINS = [
    pin_torchcc_4x4,
    pin_every_colour_3x3,
    pin_torchcc_6x6,
    pin_closed_forms,
    pin_random_vs_python_bfs,
    pin_random_vs_c_bfs,
    pin_exhaustive,
    pin_scipy_partition,
    pin_invariants_and_numbering,
    pin_ignore_torchcc_4x4,
    pin_ignore_vs_python_bfs,
    pin_ignore_scipy_binary,
    pin_ignore_leaves_other_regions,
    pin_rgb_vs_python_bfs,
    pin_stats_torchcc_4x4,
    pin_stats_vs_scipy,
    pin_wide_vs_python_bfs,
]
