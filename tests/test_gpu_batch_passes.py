"""GPU parity of a batch with more tiles than one pass of the pipeline takes
(2^24 - 1: seam node ids are 32-bit, and a launch of one 256-thread workgroup
per tile stays below 2^32 threads): ccl_label, ccl_number, ccl_count,
ccl_label_stats and ccl_region_stats take it in passes of whole images
(ccl_label_host in its groups of images), one after another in one
workspace sized for a pass.  2^24 + 3 pictures of 2 x 2 pixels (one tile
each): the first pass holds
2^24 - 1 images, the second the last four.  Its 2^24 + 3 tile rows also take
the numbering scan over several launches; the statistics calls carry the
regions of the first pass into the records of the second.

Expected values: the oracle on images from both passes, and for every image a
closed form that holds for any 2 x 2 picture with 8 neighbours (every two of
its pixels touch, so each colour is one region whose leader is that colour's
first pixel)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TILES = (1 << 24) - 1  # tiles of one pass


@pytest.fixture(scope="module")
def ccl():
    import connected_component_labelling_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m._load()
    return m


def closed_form_2x2(c: np.ndarray):
    """Leaders, numbers and counts of 2 x 2 pictures (rows of 4 pixels in
    reading order), 8 neighbours."""
    same = c[:, :, None] == c[:, None, :]            # [B, p, q]: same colour
    leaders = same.argmax(axis=2).astype(np.int32)   # first q of p's colour
    is_leader = leaders == np.arange(4, dtype=np.int32)[None, :]
    upto = np.cumsum(is_leader, axis=1, dtype=np.int32)  # leaders at or before q
    numbers = np.take_along_axis(upto, leaders, axis=1)
    counts = is_leader.sum(axis=1, dtype=np.int32)
    return leaders, numbers, counts


def closed_form_stats_2x2(numbers: np.ndarray, counts: np.ndarray):
    """Records (area, y0, x0, y1, x1, sum_y, sum_x) of every region of 2 x 2
    pictures, regions of all images concatenated: pixel p sits at row p // 2,
    column p % 2."""
    B = numbers.shape[0]
    off = np.zeros(B, np.int64)
    np.cumsum(counts[:-1], out=off[1:])
    n = int(counts.sum(dtype=np.int64))
    rec = np.zeros((n, 7), np.int64)
    ys = np.array([0, 0, 1, 1], np.int64)
    xs = np.array([0, 1, 0, 1], np.int64)
    big = np.int64(1 << 40)
    for k in range(1, 5):
        m = numbers == k
        has = m.any(axis=1)
        idx = off[has] + (k - 1)
        mk = m[has]
        rec[idx, 0] = mk.sum(axis=1)
        rec[idx, 1] = np.where(mk, ys, big).min(axis=1)
        rec[idx, 2] = np.where(mk, xs, big).min(axis=1)
        rec[idx, 3] = np.where(mk, ys, -1).max(axis=1)
        rec[idx, 4] = np.where(mk, xs, -1).max(axis=1)
        rec[idx, 5] = (mk * ys).sum(axis=1)
        rec[idx, 6] = (mk * xs).sum(axis=1)
    return off, rec


def gpu_records(stats) -> np.ndarray:
    bbox = stats["bbox"].cpu().numpy().astype(np.int64)
    return np.column_stack([stats["area"].cpu().numpy().astype(np.int64), bbox,
                            stats["sum_y"].cpu().numpy(), stats["sum_x"].cpu().numpy()])


@pytest.mark.timeout(600)
def test_batch_beyond_tile_limit(ccl):
    B = TILES + 4
    rng = np.random.default_rng(2024)
    img = rng.integers(0, 3, size=(B, 2, 2), dtype=np.uint8)
    print(f"[gpu case] batch passes: {B} images 2x2 u8 conn=8 "
          f"workspace={ccl.workspace_bytes(B, 2, 2)} bytes", flush=True)
    # one pass's workspace, the same as for the first pass's images alone
    assert ccl.workspace_bytes(B, 2, 2) == ccl.workspace_bytes(TILES, 2, 2)
    c = img.reshape(B, 4)
    exp_leaders, exp_numbers, exp_counts = closed_form_2x2(c)
    # the closed form against the oracle, on images of both passes
    for sl in (slice(0, 2000), slice(TILES - 1000, B)):
        o = oracle.label(img[sl], 8)
        on, oc = oracle.number(o)
        assert np.array_equal(o.reshape(-1, 4), exp_leaders[sl])
        assert np.array_equal(on.reshape(-1, 4), exp_numbers[sl])
        assert np.array_equal(oc, exp_counts[sl])

    torch.cuda.empty_cache()
    t = torch.from_numpy(img).cuda()
    ws = torch.empty(ccl.workspace_bytes(B, 2, 2), dtype=torch.uint8, device="cuda")
    leaders, c0 = ccl.label(t, 8, number=False, workspace=ws, check=True)
    labels, c1 = ccl.label(t, 8, number=True, workspace=ws, check=True)
    numbered, c2 = ccl.number(leaders, workspace=ws)
    c3 = ccl.count(leaders, workspace=ws)
    torch.cuda.synchronize()
    assert ccl.error_word(ws) == 0
    got_leaders = leaders.cpu().numpy().reshape(B, 4)
    bad = np.flatnonzero((got_leaders != exp_leaders).any(axis=1))
    assert bad.size == 0, f"leaders differ in {bad.size} images, first {bad[:5].tolist()}"
    assert np.array_equal(labels.cpu().numpy().reshape(B, 4), exp_numbers)
    assert np.array_equal(numbered.cpu().numpy().reshape(B, 4), exp_numbers)
    for cnt in (c0, c1, c2, c3):
        assert np.array_equal(cnt.cpu().numpy(), exp_counts)
    del leaders, numbered

    # statistics: the records of the second pass's images follow those of
    # the first pass, in both statistics calls
    off, exp_rec = closed_form_stats_2x2(exp_numbers, exp_counts)
    n_total = exp_rec.shape[0]
    for sl in (slice(0, 2000), slice(TILES - 1000, B)):  # the closed form against the oracle
        o = oracle.region_stats(exp_numbers[sl].reshape(-1, 2, 2), exp_counts[sl])
        lo = int(off[sl.start])
        hi = lo + int(exp_counts[sl].sum(dtype=np.int64))
        orec = np.column_stack([o["area"], o["bbox"], o["sum_y"], o["sum_x"]]).astype(np.int64)
        assert np.array_equal(orec, exp_rec[lo:hi])
    print(f"[gpu case] batch passes: region_stats and label_stats, {n_total} records", flush=True)
    st = ccl.region_stats(labels, c1, n_total=n_total, workspace=ws)
    torch.cuda.synchronize()
    assert ccl.error_word(ws) == 0
    assert np.array_equal(gpu_records(st), exp_rec)
    del st
    labels2, c4, st2 = ccl.label_stats(t, n_total, 8, workspace=ws, check=True)
    assert np.array_equal(c4.cpu().numpy(), exp_counts)
    assert np.array_equal(labels2.cpu().numpy().reshape(B, 4), exp_numbers)
    assert np.array_equal(gpu_records(st2), exp_rec)
    del t, ws, labels, labels2, st2
    torch.cuda.empty_cache()

    # from page-locked host memory, in groups of images in one pass's workspace
    print("[gpu case] batch passes: label_host", flush=True)
    host = torch.from_numpy(img).pin_memory()
    hl, hc = ccl.label_host(host, 8, number=True)
    assert np.array_equal(hl.numpy().reshape(B, 4), exp_numbers)
    assert np.array_equal(hc.cpu().numpy(), exp_counts)
    del host, hl, hc
    torch.cuda.empty_cache()
