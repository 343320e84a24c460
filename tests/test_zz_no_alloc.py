"""ccl_label_noalloc (the entry point with no workspace argument, for callers
that cannot allocate) against ccl_label on the same inputs, bit for bit,
through the C ABI: calls in a row on one GPU, each smaller than the one
before, so that every call but the first runs on a scratch array that still
holds the previous call's contents."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ccl():
    import connected_component_labelling_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m._load()
    return m


def _dev(img):
    if img.dtype == np.uint32:
        img = img.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(img)).cuda()


def _both(ccl, img, dtype, flags, ignore=0, conn=8):
    """(out, counts) of ccl_label_noalloc and of ccl_label with its own workspace."""
    lib = ccl._load()
    x = _dev(img if img.ndim == 3 else img[None])
    B, H, W = x.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for entry in ("noalloc", "label"):
        out = torch.full((B, H, W), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        if entry == "noalloc":
            rc = lib.ccl_label_noalloc(ccl._ptr(x), dtype, B, H, W, conn, flags, ignore,
                                       ccl._ptr(out), ccl._ptr(cnt), stream)
        else:
            ws = torch.empty(lib.ccl_workspace_bytes(B, H, W), dtype=torch.uint8, device="cuda")
            rc = lib.ccl_label(ccl._ptr(x), dtype, B, H, W, conn, flags, ignore, ccl._ptr(out),
                               ccl._ptr(cnt), ccl._ptr(ws), ws.numel(), stream)
        assert rc == 0, f"{entry}: status {rc}"
        outs.append((out, cnt))
    torch.cuda.synchronize()
    return [(o.cpu().numpy(), c.cpu().numpy()) for o, c in outs]


def test_noalloc_matches_label_on_shrinking_calls(ccl):
    cases = [
        # (name, image, dtype code, flags, ignore, connectivity): each smaller
        ("spiral 4096x4096 u32 numbered", synth.spiral_image(4096, 4096, seed=3), 4, 1, 0, 8),
        ("bernoulli 16x512x512 u8 leaders, 4-conn", synth.bernoulli_batch(16, 512, 512, seed=2),
         1, 0, 0, 4),
        ("drawing 700x900 u32 numbered, paper ignored", synth.lines_image(700, 900, seed=4), 4,
         3, 0xFFFFFF, 8),
        ("drawing 256x256 u32 leaders", synth.lines_image(256, 256, seed=1), 4, 0, 0, 8),
        ("drawing 37x45 u32 numbered", synth.lines_image(37, 45, seed=9, nlines=6, nrects=2), 4,
         1, 0, 8),
    ]
    for name, img, dt, flags, ign, conn in cases:
        print(f"[gpu case] noalloc vs label: {name} shape={img.shape}", flush=True)
        (a, ac), (b, bc) = _both(ccl, img, dt, flags, ign, conn)
        assert np.array_equal(ac, bc), f"{name}: counts differ"
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{name}: labels differ at {len(bad)} pixels, first "
                                 f"{bad[:5].tolist()}")


def test_noalloc_binding_allocates_nothing_given_outputs(ccl):
    img = _dev(synth.lines_image(300, 200, seed=5))
    out = torch.empty((1, 300, 200), dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    got, c = ccl.label_noalloc(img, number=True, out=out, counts=cnt)
    torch.cuda.synchronize()
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    assert got is out and c is cnt
    assert after == before, "label_noalloc allocated through torch"
    exp, ec = ccl.label(img, number=True)
    assert torch.equal(out[0], exp) and torch.equal(cnt, ec)
