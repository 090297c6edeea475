"""Graph capture of the entry points beyond the persistent kernel.

Every call only enqueues kernels on the caller's stream (no allocation, copy,
memset or synchronisation), so a sequence of calls can be captured into one HIP
graph.  The graphs here hold an n_offsets, a k_offsets, a block-scaled and a
quantiser call, a pre-shuffled stacked call (persistent grid) with a padded call
that zeroes its padding rows, and a decode-sized call (register kernel) with the
offsets and batched layouts, a K = 0 call and the weight shuffle; each is replayed
several times with eager work on other buffers in between, and every replay must
reproduce the eager results bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp8_rowwise_scaled_amd as F
    F.load()
    return F


def test_new_entry_points_under_graph_replay(F):
    n = wl.make_n_offsets([40, 0, 200, 17], 70, 336, seed=1401, total_N=264)
    k = wl.make_k_offsets([48, 0, 400, 16], 45, 136, seed=1402)
    b = wl.make_stacked_blockscale([3, 0, 130], 256, 384, seed=1403)
    rng = np.random.default_rng(1404)
    xb = torch.from_numpy(rng.normal(0, 1, (37, 1040)).astype(np.float32)).to(torch.bfloat16).cuda()

    nin = [P.dev(a) for a in (n.XQ, n.WQ, n.x_scale, n.w_scale, n.n_offsets)]
    kin = [P.dev(a) for a in (k.XQ, k.WQ, k.x_scale, k.w_scale, k.k_offsets)]
    bin_ = [P.dev(a) for a in (b.XQ, b.WQ, b.x_scale, b.w_scale, b.M_sizes)]
    yn = torch.empty((n.M, n.N), dtype=torch.bfloat16, device="cuda")
    yk = torch.empty((k.G, k.M, k.N), dtype=torch.bfloat16, device="cuda")
    yb = torch.empty((b.total_M, b.N), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((37, 1040), dtype=torch.uint8, device="cuda")
    s = torch.empty((37,), dtype=torch.float32, device="cuda")
    outs = (yn, yk, yb, q, s)

    def calls():
        F.f8f8bf16_rowwise_grouped_n_offsets(*nin, out=yn)
        F.f8f8bf16_rowwise_grouped_k_offsets(*kin, out=yk)
        F.f8f8bf16_groupwise_grouped_stacked(*bin_, out=yb)
        F.f8f8bf16_quantize_rowwise(xb, q, s)

    def reset():
        # the same starting state for the eager run and every replay (the n_offsets
        # output keeps columns of no group untouched, so they must start equal)
        for o in outs:
            o.view(torch.uint8).fill_(0xC1)

    reset()
    calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        calls()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        calls()
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        reset()                                   # eager work between replays
        scratch.add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(("n_offsets", "k_offsets", "blockscale", "codes", "scales"), outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), \
                f"replay {rep}: {name} differs from the eager result"


def test_preshuffled_and_padded_entry_points_under_graph_replay(F):
    # stacked, 354 rows per group on average: the persistent grid on pre-shuffled W
    st = wl.make_stacked([600, 0, 517, 300], 512, 1024, seed=1410)
    # padded slabs of 200 rows, valid counts 0, 64, full and 129, padding zeroed
    dy = wl.make_dynamic([0, 64, 200, 129], 200, 384, 640, seed=1411)
    sin = [P.dev(a) for a in (st.XQ, st.WQ, st.x_scale, st.w_scale, st.M_sizes)]
    sin[1] = F.f8f8bf16_shuffle_b(sin[1])          # once, as at weight load
    din = [P.dev(a) for a in (dy.XQ, dy.WQ, dy.x_scale, dy.w_scale, dy.zero_start_index_M)]
    ys = torch.empty((st.total_M, st.N), dtype=torch.bfloat16, device="cuda")
    yd = torch.empty((dy.XQ.shape[0], dy.XQ.shape[1], dy.WQ.shape[1]), dtype=torch.bfloat16, device="cuda")
    outs = (ys, yd)
    assert F.plan(F.LAYOUT_STACKED, True, 4, st.total_M, st.N, st.K)["persistent"] == 1

    def calls():
        F.f8f8bf16_rowwise_grouped_stacked_preshuffle(*sin, out=ys)
        F.f8f8bf16_rowwise_grouped_dynamic(*din, zeroing_output_tensor=True, out=yd)

    def reset():
        for o in outs:
            o.view(torch.uint8).fill_(0xC1)

    reset()
    calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    assert bool((yd[0].view(torch.int16) == 0).all()), "the empty slab's padding was not zeroed"

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        calls()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        calls()
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        reset()
        scratch.add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(("stacked_preshuffle", "dynamic"), outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), \
                f"replay {rep}: {name} differs from the eager result"


def test_decode_offsets_batched_zero_fill_and_shuffle_under_graph_replay(F):
    """The calls a decode step or a weight reload would capture: one token over eight
    groups (the small-M register kernel), the offsets and batched layouts, a call with
    K = 0 (the zero-fill kernel) and the weight shuffle."""
    dec = wl.make_stacked([0, 0, 1, 0, 0, 0, 0, 0], 1024, 512, seed=1420)
    off = wl.make_stacked([37, 0, 130, 64], 264, 336, seed=1421)
    bat = wl.make_dynamic([77, 77, 77], 77, 256, 448, seed=1422)
    assert F.plan(F.LAYOUT_STACKED, False, 8, 1, 1024, 512)["config_id"] in (13, 14, 15)   # the register kernel
    din = [P.dev(a) for a in (dec.XQ, dec.WQ, dec.x_scale, dec.w_scale, dec.M_sizes)]
    oin = [P.dev(a) for a in (off.XQ, off.WQ, off.x_scale, off.w_scale)] + \
        [P.dev(np.cumsum(off.M_sizes).astype(np.int32))]
    bin_ = [P.dev(a) for a in (bat.XQ, bat.WQ, bat.x_scale, bat.w_scale)]
    zin = [torch.empty((40, 0), dtype=torch.uint8, device="cuda"), torch.empty((2, 96, 0), dtype=torch.uint8,
                                                                               device="cuda"),
           torch.empty((40,), dtype=torch.float32, device="cuda"), torch.ones((2, 96), device="cuda"),
           P.dev(np.array([25, 15], np.int64))]
    yd = torch.empty((1, 1024), dtype=torch.bfloat16, device="cuda")
    yo = torch.empty((off.total_M, off.N), dtype=torch.bfloat16, device="cuda")
    yb = torch.empty((bat.G, bat.expected_m, bat.N), dtype=torch.bfloat16, device="cuda")
    yz = torch.empty((40, 96), dtype=torch.bfloat16, device="cuda")
    wsrc = P.dev(bat.WQ)                           # N = 256, K = 448: whole shuffle granules
    ws = torch.empty_like(wsrc)
    outs = (yd, yo, yb, yz, ws)

    def calls():
        F.f8f8bf16_rowwise_grouped_stacked(*din, out=yd)
        F.f8f8bf16_rowwise_grouped_offsets(*oin, out=yo)
        F.f8f8bf16_rowwise_grouped_batched(*bin_, out=yb)
        F.f8f8bf16_rowwise_grouped_stacked(*zin, out=yz)
        F.f8f8bf16_shuffle_b(wsrc, out=ws)

    def reset():
        for o in outs:
            o.view(torch.uint8).fill_(0xC1)

    reset()
    calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    assert bool((yz.view(torch.int16) == 0).all()), "K = 0 did not zero-fill the output"

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        calls()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        calls()
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        reset()
        scratch.add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(("decode", "offsets", "batched", "zero fill", "shuffle"), outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), \
                f"replay {rep}: {name} differs from the eager result"
