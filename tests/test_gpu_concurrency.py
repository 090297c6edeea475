"""GPU tests of overlapping calls.

The library keeps no state between calls (no workspace, no device memory of its
own) and no kernel waits for another workgroup, so calls on different streams may
run at the same time on the device, and several host threads may call at once.
Each case first runs its calls one after another on the default stream (checked
against the oracle), then runs them again overlapped, and requires every
overlapped output to equal its serial output bit for bit.
"""
import threading

import numpy as np
import pytest
import torch

import oracle
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


@pytest.fixture(scope="module")
def calls(F):
    """Four kinds of call, each as (name, launch(out), out shape, oracle result or None):
    a stacked call on the persistent grid (at least 256 rows per group on average),
    a padded call on the data-parallel grid, a small-M call on the register kernel,
    and the quantiser."""
    out = []
    s = wl.make_stacked(np.array([600, 0, 700, 300], np.int64), 768, 1024, seed=2601)
    sa = [P.dev(a) for a in (s.XQ, s.WQ, s.x_scale, s.w_scale, s.M_sizes)]
    out.append(("stacked persistent",
                lambda y: F.f8f8bf16_rowwise_grouped_stacked(*sa, out=y), (s.total_M, s.N),
                oracle.grouped_stacked(s.XQ, s.WQ, s.x_scale, s.w_scale, s.M_sizes)))
    d = wl.make_dynamic(np.array([0, 300, 137, 211], np.int64), 300, 512, 896, seed=2602)
    da = [P.dev(a) for a in (d.XQ, d.WQ, d.x_scale, d.w_scale, d.zero_start_index_M)]
    out.append(("padded",
                lambda y: F.f8f8bf16_rowwise_grouped_dynamic(*da, zeroing_output_tensor=True, out=y),
                (d.G, d.expected_m, d.N),
                oracle.grouped_dynamic(d.XQ, d.WQ, d.x_scale, d.w_scale, d.zero_start_index_M, True)))
    m = wl.make_stacked(np.array([0, 2, 0, 0, 1, 0, 0, 0], np.int64), 2048, 1024, seed=2603)
    ma = [P.dev(a) for a in (m.XQ, m.WQ, m.x_scale, m.w_scale, m.M_sizes)]
    out.append(("small M",
                lambda y: F.f8f8bf16_rowwise_grouped_stacked(*ma, out=y), (m.total_M, m.N),
                oracle.grouped_stacked(m.XQ, m.WQ, m.x_scale, m.w_scale, m.M_sizes)))
    g = torch.Generator(device="cuda").manual_seed(2604)
    xb = torch.randn((512, 1024), generator=g, device="cuda").to(torch.bfloat16)

    def quantise(y):
        q, sc = F.f8f8bf16_quantize_rowwise(xb)
        y.view(torch.uint8)[:, :1024].copy_(q.view(torch.uint8))
        y.view(torch.uint8)[:, 1024:].copy_(sc.view(torch.uint8).view(512, 4))
    out.append(("quantiser", quantise, (512, 514), None))
    torch.cuda.synchronize()
    return out


def serial(calls):
    res = []
    for name, launch, shape, ref in calls:
        print(f"case serial {name}", flush=True)
        whole, y = P.guarded_output(shape)
        launch(y)
        torch.cuda.synchronize()
        P.check_guards(whole)
        bits = P.bits_of(y)
        if ref is not None:
            P.assert_rows_match(bits.reshape(ref.row_class.shape[0], -1), ref, label=f"serial {name}")
        res.append(bits)
    return res


def test_calls_on_two_streams_overlap(F, calls):
    """The four calls alternate between two streams, four rounds, with no
    synchronisation until the end."""
    expect = serial(calls)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [(i, rnd, *P.guarded_output(calls[i][2])) for rnd in range(4) for i in range(len(calls))]
    torch.cuda.synchronize()                    # the sentinel fills are done before the side streams write
    print("case two streams", flush=True)
    for i, rnd, whole, y in outs:
        with torch.cuda.stream(streams[(i + rnd) % 2]):
            calls[i][1](y)
    torch.cuda.synchronize()
    for i, rnd, whole, y in outs:
        P.check_guards(whole)
        assert np.array_equal(P.bits_of(y), expect[i]), f"{calls[i][0]} round {rnd}"


def test_calls_from_several_host_threads(F, calls):
    """Four host threads, each on its own stream, each runs the four calls three
    times; the GIL is released inside the library calls, so the host side overlaps
    too."""
    expect = serial(calls)
    outs = {t: [] for t in range(4)}
    for t in range(4):
        for rep in range(3):
            for i, (_, _, shape, _) in enumerate(calls):
                outs[t].append((i, *P.guarded_output(shape)))
    torch.cuda.synchronize()
    errors = []

    def work(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for i, whole, y in outs[t]:
                    calls[i][1](y)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((t, repr(e)))

    print("case four host threads", flush=True)
    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(4):
        for i, whole, y in outs[t]:
            P.check_guards(whole)
            assert np.array_equal(P.bits_of(y), expect[i]), f"thread {t}: {calls[i][0]}"


def test_binding_launches_on_the_current_stream(F):
    """The binding hands the library the handle of torch's current stream, on the
    default stream and inside a side stream's context."""
    from fp8_rowwise_scaled_amd import ops
    dev = torch.device("cuda", 0)
    assert ops._stream(dev) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert ops._stream(dev) == s.cuda_stream
        assert ops._stream(dev) != torch.cuda.default_stream(dev).cuda_stream
    assert ops._stream(dev) == torch.cuda.current_stream(dev).cuda_stream
