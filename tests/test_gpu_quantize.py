"""GPU parity for rowwise fp8 quantisation (f8f8bf16_quantize_rowwise).

Codes and scales are integer/float decisions taken in fp32 on both sides, so the
bar is bit equality with the oracle: every code and every scale.  Shapes cover
rows held in registers (K <= 8192) and rows read twice (K > 8192), K = 8 and
K = 0, zero rows, subnormal-range rows and exact ties between two codes.  The
quantiser feeding the stacked GEMM is checked end to end against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp8_rowwise_scaled_amd as F
    F.load()
    return F


def bf16_rows(rows, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (rows, K)).astype(np.float32)
    x *= (2.0 ** rng.uniform(-20, 20, (rows, 1))).astype(np.float32)
    if rows > 2:
        x[1] = 0.0                                   # a zero row: scale 1, codes 0
        x[2] *= np.float32(2.0 ** -30)               # tiny values
    if rows > 3:
        # amax near 2^-119: the scale is an fp32 subnormal (the IEEE-division rows)
        x[3] = rng.normal(0, 1, K).astype(np.float32) * np.float32(2.0 ** -120)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def run(F, bits):
    X = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, s = F.f8f8bf16_quantize_rowwise(X)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("rows,K", [(1, 8), (3, 16), (37, 1040), (128, 7168), (64, 8192), (5, 8200),
                                    (17, 28672), (300, 2048)])
def test_quantize_matches_oracle_bitwise(F, rows, K):
    bits = bf16_rows(rows, K, seed=rows * 7 + K)
    print(f"case quantize rows={rows} K={K}", flush=True)
    q, s = run(F, bits)
    q_ref, s_ref = oracle.quantize_rowwise(bits)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    mism = np.argwhere(q != q_ref)
    assert mism.size == 0, f"{len(mism)} codes differ, first at {mism[:5].tolist()}"


def test_quantize_exact_ties_and_boundaries(F):
    """Rows whose amax is 448 (scale exactly 1): the quotients are the values
    themselves, placed on every midpoint between two codes, next to them, and
    across the subnormal / normal boundary."""
    pos = oracle.e4m3fn_table()[:0x7F]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([mids, -mids, pos.astype(np.float32)])
    bf = torch.from_numpy(vals).to(torch.bfloat16).float().numpy()   # keep what bf16 can hold
    K = 8 * ((bf.size + 1 + 7) // 8)
    row = np.zeros(K, np.float32)
    row[0] = 448.0
    row[1:1 + bf.size] = bf
    bits = torch.from_numpy(np.stack([row, -row])).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, s = run(F, bits)
    q_ref, s_ref = oracle.quantize_rowwise(bits)
    assert np.all(s == 1.0) and np.array_equal(s, s_ref)
    assert np.array_equal(q, q_ref)


def _bf16_bits_of(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_quantize_quotients_next_to_code_midpoints(F):
    """Non-power-of-two scales, each row holding the two bf16 neighbours of every
    midpoint between two codes times its scale: the code then hangs on the last
    bits of the fp32 quotient x / s, which must be the correctly rounded one."""
    rng = np.random.default_rng(91)
    pos = oracle.e4m3fn_table()[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2
    rows = []
    for _ in range(64):
        amax_bits = int(_bf16_bits_of(rng.uniform(1, 2) * 2.0 ** int(rng.integers(-40, 40)))[()])
        amax = np.array([amax_bits << 16], np.uint32).view(np.float32)[0]
        s = np.float32(amax) / np.float32(448.0)
        t = (mids * np.float64(s)).astype(np.float32)
        lo = (t.view(np.uint32) >> np.uint32(16)).astype(np.uint16)        # bf16 toward zero
        row = np.concatenate([[amax_bits], lo, lo + np.uint16(1)]).astype(np.uint16)
        row = np.concatenate([row, np.zeros((-row.size) % 8, np.uint16)])
        rows += [row, row | np.uint16(0x8000)]
    bits = np.stack(rows)
    q, s_gpu = run(F, bits)
    q_ref, s_ref = oracle.quantize_rowwise(bits)
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32))
    mism = np.argwhere(q != q_ref)
    assert mism.size == 0, f"{len(mism)} codes differ, first at {mism[:5].tolist()}"


def test_quantize_k_zero_gives_unit_scales(F):
    X = torch.empty((4, 0), dtype=torch.bfloat16, device="cuda")
    q, s = F.f8f8bf16_quantize_rowwise(X)
    torch.cuda.synchronize()
    assert q.shape == (4, 0) and torch.all(s == 1.0)


def test_quantize_then_stacked_gemm_end_to_end(F):
    """bf16 activations -> quantiser -> stacked GEMM, against the oracle's
    quantisation followed by the oracle's GEMM."""
    sizes = [70, 0, 129, 300]
    N, K = 264, 1040
    bits = bf16_rows(sum(sizes), K, seed=77)
    rng = np.random.default_rng(78)
    WQ = rng.integers(0, 0x7E, size=(len(sizes), N, K), dtype=np.uint8) | \
        (rng.integers(0, 2, size=(len(sizes), N, K), dtype=np.uint8) << 7)
    ws = (2.0 ** rng.uniform(-8, -2, (len(sizes), N))).astype(np.float32)
    q, s = run(F, bits)
    X = torch.from_numpy(q).cuda()
    whole, out = P.guarded_output((sum(sizes), N))
    F.f8f8bf16_rowwise_grouped_stacked(X, P.dev(WQ), torch.from_numpy(s).cuda(), P.dev(ws),
                                       torch.tensor(sizes, dtype=torch.int64, device="cuda"), out=out)
    torch.cuda.synchronize()
    P.check_guards(whole)
    q_ref, s_ref = oracle.quantize_rowwise(bits)
    ref = oracle.grouped_stacked(q_ref, WQ, s_ref, ws, np.array(sizes))
    P.assert_rows_match(P.bits_of(out), ref, label="quantise + GEMM")
