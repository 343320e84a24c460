"""The labelling calls recorded into a HIP graph (torch.cuda.CUDAGraph) and
replayed: every kernel of a call is an ordinary launch on the caller's stream
(no memory-set or copy nodes: what must start empty is cleared by the
kernels themselves), so a captured call replays with the same results as an
eager one.  Each replay follows eager work of the program (a new picture
copied into the captured input, another labelling on its own buffers, a
synchronisation) and is checked against the oracle."""
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


def _pictures(n, H, W):
    return [synth.lines_image(H, W, seed=100 + k) for k in range(n)]


@pytest.mark.parametrize("entry", ["label", "label_noalloc", "label_stats"])
def test_captured_call_replays(ccl, entry):
    H, W = 300, 420  # ragged: partial tiles on the right and at the bottom
    pics = _pictures(4, H, W)
    print(f"[gpu case] graph replay of {entry} {H}x{W} u32 conn=8", flush=True)
    static_in = torch.from_numpy(pics[0].view(np.int32)).cuda()
    out = torch.empty((H, W), dtype=torch.int32, device="cuda")
    counts = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(ccl.workspace_bytes(1, H, W), dtype=torch.uint8, device="cuda")
    cap = 1 << 14
    records = torch.empty((cap, 5), dtype=torch.int64, device="cuda")

    def call():
        if entry == "label":
            return ccl.label(static_in, 8, number=True, workspace=ws, out=out)
        if entry == "label_noalloc":
            return ccl.label_noalloc(static_in, 8, number=True, out=out, counts=counts)
        return ccl.label_stats(static_in, cap, 8, workspace=ws, out=out, records=records,
                               trim=False)

    res = call()  # eager first (the no-alloc entry looks up its scratch array here)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            res = call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_out, g_counts = res[0], res[1]

    other = torch.from_numpy(pics[-1].view(np.int32)).cuda()
    for k in range(3):
        # the program's own eager work between replays
        static_in.copy_(torch.from_numpy(pics[k].view(np.int32)))
        eager_other, _ = ccl.label(other, 8, number=True)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        lead = oracle.label(pics[k], 8)
        exp, exp_counts = oracle.number(lead)
        got = g_out.cpu().numpy().reshape(H, W)
        assert np.array_equal(got, exp), f"replay {k}: numbers differ"
        assert np.array_equal(g_counts.cpu().numpy(), exp_counts), f"replay {k}: counts differ"
        if entry == "label_stats":
            n = int(exp_counts.sum())
            st = oracle.region_stats(exp, exp_counts)
            r32 = records.view(torch.int32)
            assert np.array_equal(r32[:n, 4].cpu().numpy(), st["area"]), f"replay {k}: areas"
            assert np.array_equal(r32[:n, 5:9].cpu().numpy(), st["bbox"]), f"replay {k}: boxes"
            assert np.array_equal(records[:n, 0].cpu().numpy(), st["sum_y"]), f"replay {k}: sum_y"
            assert np.array_equal(records[:n, 1].cpu().numpy(), st["sum_x"]), f"replay {k}: sum_x"
        o_lead = oracle.label(pics[-1], 8)
        o_exp, _ = oracle.number(o_lead)
        assert np.array_equal(eager_other.cpu().numpy(), o_exp), f"replay {k}: eager call differs"
    del graph
