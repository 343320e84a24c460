"""ccl_label_host (a picture in page-locked host memory, copies in and out
overlapped with the labelling band by band, or group of images by group)
against the CPU oracle, bit for bit: workloads 1, 3 and 5 at full size with
band counts that leave a short last band, batches of u8 images cut into bands
or taken whole in groups (with a short last group), an ignored colour, an RGB
picture, and leaders as well as numbers."""
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


def pinned(img: np.ndarray) -> torch.Tensor:
    if img.dtype == np.uint32:
        img = img.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(img)).pin_memory()


def check_host(ccl, name, img, band_rows, number=True, ignore=None, rgb=False, conn=8):
    print(f"[gpu case] host {name} shape={img.shape} band_rows={band_rows} number={number} "
          f"ignore={ignore}", flush=True)
    exp_leaders = oracle.label(img, conn, ignore=ignore, rgb=rgb)
    exp_labels, exp_counts = oracle.number(exp_leaders)
    exp = exp_labels if number else exp_leaders
    h = pinned(img)
    x = h if (h.dim() == (4 if rgb else 3)) else h.unsqueeze(0)
    lab = ccl.HostLabeller(tuple(x.shape[:3]), dtype=x.dtype, rgb=rgb, connectivity=conn,
                           band_rows=band_rows)
    for rep in range(2):  # the second call reuses every buffer
        out, counts = lab(h, number=number, ignore=ignore)
        assert ccl.error_word(lab.workspace) == 0
        got = out.numpy().reshape(exp.shape)
        if not np.array_equal(got, exp):
            bad = np.argwhere(got != exp)
            raise AssertionError(f"{name} (call {rep}): labels differ at {len(bad)} pixels, "
                                 f"first {bad[:5].tolist()}")
        assert np.array_equal(counts.cpu().numpy(), exp_counts), f"{name}: counts differ"
        assert np.array_equal(lab.dev_out.cpu().numpy().reshape(exp.shape), exp), \
            f"{name}: device labels differ"


@pytest.mark.parametrize("config,band_rows", [(1, 96), (3, 1184), (5, 4992)])
def test_host_workloads_ragged_bands(ccl, config, band_rows):
    img = synth.generate(config)
    H = img.shape[1]
    assert H % band_rows != 0 and H // band_rows >= 2  # several bands, a short last one
    check_host(ccl, f"workload {config}", img, band_rows)


def test_host_leaders_and_automatic_bands(ccl):
    img = synth.spiral_image(4096, 4096, seed=3)
    check_host(ccl, "spiral leaders, automatic bands", img, 0, number=False)


def test_host_batch_with_ignored_colour(ccl):
    img = synth.bernoulli_batch(6, 512, 300, seed=21)
    check_host(ccl, "u8 batch, 0 ignored", img, 160, ignore=0)
    check_host(ccl, "u8 batch, 4-conn leaders", img, 32, number=False, conn=4)


def test_host_grouped_batch(ccl):
    """Small images go whole, in groups of at least 2^22 pixels: 20 images of
    512 x 512 make a group of 16 and a last group of 4."""
    img = synth.bernoulli_batch(20, 512, 512, seed=5)
    check_host(ccl, "u8 batch in two groups", img, 0)
    check_host(ccl, "u8 batch in two groups, 1 ignored", img, 0, ignore=1, number=False)


def test_host_rgb(ccl):
    img = synth.rgb24(synth.lines_image(700, 513, seed=12))
    check_host(ccl, "RGB drawing", img, 224, rgb=True)


def test_host_one_band_and_tiny(ccl):
    check_host(ccl, "one band", synth.lines_image(100, 200, seed=13), 0)
    check_host(ccl, "single pixel", np.array([[7]], np.uint32), 32)
    check_host(ccl, "one row", synth.lines_image(1, 333, seed=2, nlines=3, nrects=1), 64)
