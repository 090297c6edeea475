"""GPU parity past 2 GiB: 64-bit addressing of X, W and Y on every layout family.

Each case puts the group that is checked beyond the first 2^31 bytes of one
operand, so a 32-bit byte offset anywhere on its path (copy descriptors, the
pre-shuffled block index, the epilogue's row pointer, the padding-row zero fill)
would read or write the wrong place.  The large buffers are made on the device
(zeros, or seeded torch random bytes with the two NaN codes moved to their
neighbours); only the rows and columns that are checked travel to the host, where
the oracle computes them from the same bytes.  Guard bands around Y are checked
on the device.
"""
import os
from contextlib import contextmanager

import numpy as np
import pytest
import torch

import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu

TWO_GIB = 1 << 31


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp8_rowwise_scaled_amd as F
    F.load()
    return F


@pytest.fixture(autouse=True)
def free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@contextmanager
def config(cfg):
    old = os.environ.get("FP8GG_CONFIG")
    if cfg is None:
        os.environ.pop("FP8GG_CONFIG", None)
    else:
        os.environ["FP8GG_CONFIG"] = str(cfg)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("FP8GG_CONFIG", None)
        else:
            os.environ["FP8GG_CONFIG"] = old


def host_codes(rng, shape):
    """Random e4m3fn codes without the NaN codes 0x7F / 0xFF."""
    b = rng.integers(0, 256, size=shape, dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] -= 1
    return b


def device_codes(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    b = torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=g)
    # elementwise: masked indexing builds an index list, which breaks past 2^31 elements
    return torch.where((b & 0x7F) == 0x7F, b - 1, b)


def scales(rng, n):
    return rng.uniform(0.5, 2.0, n).astype(np.float32)


def guarded(n_elems):
    whole = torch.full((n_elems + 2 * P.GUARD,), P.SENTINEL, dtype=torch.int16, device="cuda")
    return whole, whole[P.GUARD:P.GUARD + n_elems]


def guards_intact(whole):
    s = torch.tensor(P.SENTINEL, dtype=torch.int16, device="cuda")
    return bool((whole[:P.GUARD] == s).all()) and bool((whole[-P.GUARD:] == s).all())


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("cfg", [None, 9, 20, 15])
def test_x_rows_past_2gib(F, cfg):
    """Stacked, K = 32768: group 0 holds 65 600 zero rows (2.15 GB of X), group 1's
    37 rows start past 2^31 bytes."""
    rng = np.random.default_rng(9600)
    K, N, R0, R1 = 32768, 128, 65600, 37
    assert R0 * K > TWO_GIB
    X = torch.zeros((R0 + R1, K), dtype=torch.uint8, device="cuda")
    X1 = host_codes(rng, (R1, K))
    X[R0:] = P.dev(X1)
    W = host_codes(rng, (2, N, K))
    xs = scales(rng, R0 + R1)
    ws = scales(rng, 2 * N).reshape(2, N)
    sizes = np.array([R0, R1], np.int64)
    whole, y = guarded((R0 + R1) * N)
    print(f"case X past 2 GiB cfg={cfg}", flush=True)
    with config(cfg):
        F.f8f8bf16_rowwise_grouped_stacked(X, P.dev(W), P.dev(xs), P.dev(ws), P.dev(sizes),
                                           out=y.view(torch.bfloat16).view(R0 + R1, N))
    torch.cuda.synchronize()
    assert guards_intact(whole)
    y2 = y.view(R0 + R1, N)
    assert not bool((y2[:R0] & 0x7FFF).any()), "zero rows of group 0 must give +-0"
    ref = oracle.grouped_stacked(X1, W[1:2], xs[R0:], ws[1:2], np.array([R1], np.int64))
    P.assert_rows_match(bits(y2[R0:]), ref, label=f"X past 2 GiB cfg={cfg}")


@pytest.mark.parametrize("cfg,pre", [(None, False), (15, False), (9, False), (16, False),
                                     (None, True), (6, True), (26, True)])
def test_w_rows_past_2gib(F, cfg, pre):
    """Stacked, G = 2, N = 36000, K = 32768 (2.36 GB of W, 2.36 GB more when
    pre-shuffled); only group 1 has rows, and its last W rows lie past 2^31 bytes.
    The first 64 and the last 512 columns are checked."""
    rng = np.random.default_rng(9700)
    G, N, K, R = 2, 36000, 32768, 16
    assert G * N * K > TWO_GIB and (N + N - 512) * K > TWO_GIB
    W = torch.zeros((G, N, K), dtype=torch.uint8, device="cuda")
    W[1] = device_codes((N, K), 9700)
    X = host_codes(rng, (R, K))
    xs = scales(rng, R)
    ws = scales(rng, G * N).reshape(G, N)
    sizes = np.array([0, R], np.int64)
    cols = np.concatenate([np.arange(64), np.arange(N - 512, N)])
    W1 = W[1, torch.from_numpy(cols).cuda()].cpu().numpy()
    Wd = F.f8f8bf16_shuffle_b(W) if pre else W
    if pre:
        del W
    whole, y = guarded(R * N)
    print(f"case W past 2 GiB cfg={cfg} pre={pre}", flush=True)
    fn = F.f8f8bf16_rowwise_grouped_stacked_preshuffle if pre else F.f8f8bf16_rowwise_grouped_stacked
    with config(cfg):
        fn(P.dev(X), Wd, P.dev(xs), P.dev(ws), P.dev(sizes), out=y.view(torch.bfloat16).view(R, N))
    torch.cuda.synchronize()
    assert guards_intact(whole)
    ref = oracle.grouped_stacked(X, W1[None], xs, ws[1:2, cols], np.array([R], np.int64))
    got = bits(y.view(R, N)[:, torch.from_numpy(cols).cuda()])
    P.assert_rows_match(got, ref, label=f"W past 2 GiB cfg={cfg} pre={pre}")


@pytest.mark.parametrize("cfg", [None, 9, 20])
def test_y_rows_past_2gib(F, cfg):
    """Stacked, N = 16384, K = 16: group 1's 64 output rows start exactly 2^31
    bytes into Y; a few rows of group 0 at both ends are checked as well."""
    rng = np.random.default_rng(9800)
    N, K, R0, R1 = 16384, 16, 65536, 64
    assert R0 * N * 2 == TWO_GIB
    X = host_codes(rng, (R0 + R1, K))
    W = host_codes(rng, (2, N, K))
    xs = scales(rng, R0 + R1)
    ws = scales(rng, 2 * N).reshape(2, N)
    sizes = np.array([R0, R1], np.int64)
    whole, y = guarded((R0 + R1) * N)
    print(f"case Y past 2 GiB cfg={cfg}", flush=True)
    with config(cfg):
        F.f8f8bf16_rowwise_grouped_stacked(P.dev(X), P.dev(W), P.dev(xs), P.dev(ws), P.dev(sizes),
                                           out=y.view(torch.bfloat16).view(R0 + R1, N))
    torch.cuda.synchronize()
    assert guards_intact(whole)
    y2 = y.view(R0 + R1, N)
    ref1 = oracle.grouped_stacked(X[R0:], W[1:2], xs[R0:], ws[1:2], np.array([R1], np.int64))
    P.assert_rows_match(bits(y2[R0:]), ref1, label=f"Y past 2 GiB group 1 cfg={cfg}")
    rows0 = np.r_[0:8, R0 - 8:R0]
    ref0 = oracle.grouped_stacked(X[rows0], W[0:1], xs[rows0], ws[0:1], np.array([len(rows0)], np.int64))
    P.assert_rows_match(bits(y2[torch.from_numpy(rows0).cuda()]), ref0, label=f"Y group 0 ends cfg={cfg}")


@pytest.mark.parametrize("cfg", [None, 9])
def test_padded_zero_fill_past_2gib(F, cfg):
    """Padded, 2 slabs of 32 800 rows, N = 16384, K = 16 (2.15 GB of Y): slab 0 is
    all padding, slab 1 has 20 valid rows; its padding rows, zeroed by the kernel,
    run past 2^31 bytes."""
    rng = np.random.default_rng(9900)
    G, EM, N, K, V = 2, 32800, 16384, 16, 20
    assert G * EM * N * 2 > TWO_GIB
    X = host_codes(rng, (G, EM, K))
    W = host_codes(rng, (G, N, K))
    xs = scales(rng, G * EM).reshape(G, EM)
    ws = scales(rng, G * N).reshape(G, N)
    zsi = np.array([0, V], np.int64)
    whole, y = guarded(G * EM * N)
    print(f"case padded zero fill past 2 GiB cfg={cfg}", flush=True)
    with config(cfg):
        F.f8f8bf16_rowwise_grouped_dynamic(P.dev(X), P.dev(W), P.dev(xs), P.dev(ws), P.dev(zsi),
                                           zeroing_output_tensor=True,
                                           out=y.view(torch.bfloat16).view(G, EM, N))
    torch.cuda.synchronize()
    assert guards_intact(whole)
    y3 = y.view(G, EM, N)
    assert not bool((y3[0] & 0x7FFF).any()), "slab 0 is padding: +-0"
    assert not bool((y3[1, V:] & 0x7FFF).any()), "padding rows of slab 1: +-0"
    ref = oracle.grouped_stacked(X[1, :V], W[1:2], xs[1, :V], ws[1:2], np.array([V], np.int64))
    P.assert_rows_match(bits(y3[1, :V]), ref, label=f"padded past 2 GiB cfg={cfg}")


def test_quantiser_rows_past_2gib(F):
    """bf16 X of 65 600 x 16 384 (2.15 GB in, 1.07 GB of codes out): the last 40
    rows start past 2^31 bytes of X; their codes and scales bit-equal the oracle's."""
    rows, K, tail = 65600, 16384, 40
    assert (rows - tail) * K * 2 > TWO_GIB
    g = torch.Generator(device="cuda")
    g.manual_seed(9950)
    X = torch.randn((rows, K), dtype=torch.float32, device="cuda", generator=g).to(torch.bfloat16)
    print("case quantiser past 2 GiB", flush=True)
    q, s = F.f8f8bf16_quantize_rowwise(X)
    torch.cuda.synchronize()
    x_tail = X[rows - tail:].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    q_ref, s_ref = oracle.quantize_rowwise(x_tail)
    assert np.array_equal(s[rows - tail:].cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q[rows - tail:].cpu().numpy(), q_ref)


def test_n_offsets_w_rows_past_2gib(F):
    """n_offsets, K = 32768: group 0 owns W rows [0, 65600) (2.15 GB), group 1's 64
    rows start past 2^31 bytes; group 1's output columns are checked."""
    rng = np.random.default_rng(9960)
    K, M, N0, N1 = 32768, 16, 65600, 64
    assert N0 * K > TWO_GIB
    W = device_codes((N0 + N1, K), 9960)
    X = host_codes(rng, (2, M, K))
    xs = scales(rng, 2 * M).reshape(2, M)
    ws = scales(rng, N0 + N1)
    offs = np.array([N0, N0 + N1], np.int32)
    whole, y = guarded(M * (N0 + N1))
    print("case n_offsets W past 2 GiB", flush=True)
    F.f8f8bf16_rowwise_grouped_n_offsets(P.dev(X), W, P.dev(xs), P.dev(ws), P.dev(offs),
                                         out=y.view(torch.bfloat16).view(M, N0 + N1))
    torch.cuda.synchronize()
    assert guards_intact(whole)
    ref = oracle.grouped_n_offsets(X[1:2], W[N0:].cpu().numpy(), xs[1:2], ws[N0:], np.array([N1], np.int32))
    got = bits(y.view(M, N0 + N1)[:, N0:])
    assert np.all(ref.col_class == oracle.ROW_WRITTEN)
    P.assert_rows_match(got, ref, label="n_offsets group 1")


def test_k_offsets_rows_past_2gib(F):
    """k_offsets with total_K = 2^21 and 1100 rows (2.3 GB of X): group 1 contracts
    over the last 2048 columns, which for rows 1024 on lie past 2^31 bytes."""
    rng = np.random.default_rng(9970)
    M, N, K, S = 1100, 64, 1 << 21, 2048
    assert 1024 * K + K - S > TWO_GIB
    X = device_codes((M, K), 9971)
    W = device_codes((N, K), 9972)
    xs = scales(rng, 2 * M).reshape(2, M)
    ws = scales(rng, 2 * N).reshape(2, N)
    offs = np.array([K - S, K], np.int32)
    whole, y = guarded(2 * M * N)
    print("case k_offsets rows past 2 GiB", flush=True)
    F.f8f8bf16_rowwise_grouped_k_offsets(X, W, P.dev(xs), P.dev(ws), P.dev(offs),
                                         out=y.view(torch.bfloat16).view(2, M, N))
    torch.cuda.synchronize()
    assert guards_intact(whole)
    ref = oracle.grouped_k_offsets(X[:, K - S:].cpu().numpy(), W[:, K - S:].cpu().numpy(), xs[1:2], ws[1:2],
                                   np.array([S], np.int32))
    P.assert_rows_match(bits(y.view(2, M, N)[1]), ref, label="k_offsets group 1")
