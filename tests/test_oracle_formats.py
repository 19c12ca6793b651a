"""Pins of the oracle's number formats and of its NVFP4 residual coder against
things other than itself: torch's bf16 and float8_e4m3fn conversions, the OCP
MX E2M1 value table (tests/golden/e2m1_ties.txt), exact round trips on inputs
the format represents, and the rounding error bound of the format."""
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, np.inf, -np.inf],
                 np.float32),
    ])
    # exact ties: half-way patterns with odd and even kept LSB
    ties = (np.arange(0x3f80, 0x3f90, dtype=np.uint32) << 16) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    ours = O.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = O.bf16_to_f32(ours)
    ref_back = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(back, ref_back)


def test_e4m3_decode_all_codes_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    ours = np.array([O.e4m3_decode(c) for c in range(256)], np.float32)
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), ~fin)
    assert np.array_equal(ours[fin], ref[fin])
    assert ours[0x7E] == 448.0 and np.isnan(ours[0x7F])


def test_e4m3_encode_decode_identity_on_every_finite_code():
    for c in range(0x7F):
        assert O.e4m3_encode(O.e4m3_decode(c)) == c


def test_e4m3_encode_matches_torch_in_range_and_on_ties():
    vals = [O.e4m3_decode(c) for c in range(0x7F)]
    mids = [(vals[i] + vals[i + 1]) / 2 for i in range(0x7E)]
    rng = np.random.default_rng(2)
    x = np.concatenate([
        np.array(mids, np.float32),
        np.nextafter(np.array(mids, np.float32), np.float32(0)),
        np.nextafter(np.array(mids, np.float32), np.float32(1e9)),
        rng.uniform(0, 448, 5000).astype(np.float32),
        np.exp(rng.uniform(np.log(1e-5), np.log(448), 5000)).astype(np.float32),
        np.array([2.0 ** -10, 1.5 * 2.0 ** -10, 2.0 ** -11, 1e-30, 447.99], np.float32),
    ])
    x = x[(x > 0) & (x <= 448)]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([O.e4m3_encode(v) for v in x], np.uint8)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (x[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_e4m3_saturates_and_handles_nonpositive():
    assert O.e4m3_encode(449.0) == 0x7E
    assert O.e4m3_encode(1e30) == 0x7E
    assert O.e4m3_encode(float("inf")) == 0x7E
    assert O.e4m3_encode(0.0) == 0
    assert O.e4m3_encode(-3.0) == 0
    assert O.e4m3_encode(float("nan")) == 0


def test_e2m1_golden_tie_table():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e2m1_ties.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) > 20
    for x, idx, val in rows:
        x = float(np.float32(float(x)))
        assert O.e2m1_encode(x) == int(idx), x
        assert O.e2m1_decode(int(idx)) == float(val)
        if int(idx) != 0:
            assert O.e2m1_encode(-x) == (8 | int(idx))
        else:
            assert O.e2m1_encode(-x) == 0  # zero magnitude is always +0


def test_e2m1_decode_table():
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for n in range(16):
        v = O.e2m1_decode(n)
        assert v == (-1 if n & 8 else 1) * mags[n & 7]


def _shape(N, d, K=1):
    return O.Shape(W=1, N=N, d=d, K=K)


def test_nvfp4_round_trip_exact_on_representable_rows():
    """quant(dequant(codes)) == codes bit-exactly when every block holds a +-6,
    the largest block scale is 448 and the row scale is a power of two: then
    every fp32 step of the coder is exact (C = 0, row_norm = 1)."""
    rng = np.random.default_rng(3)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    N, d = 64, 256
    nb = d // 16
    nib = rng.integers(0, 16, size=(N, d)).astype(np.uint8)
    nib[nib == 8] = 0  # -0 is never produced
    for j in range(N):
        for b in range(nb):
            nib[j, 16 * b + rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
    sc = rng.integers(0x08, 0x7E, size=(N, nb)).astype(np.uint8)  # normal-range scales
    sc[np.arange(N), rng.integers(0, nb, size=N)] = 0x7E
    gexp = rng.integers(-20, -6, size=N)
    g = np.ldexp(1.0, gexp)
    sval = np.array([[O.e4m3_decode(c) for c in row] for row in sc])
    vals = np.where(nib & 8, -1.0, 1.0) * mags[nib & 7]
    H = (vals * np.repeat(sval, 16, axis=1) * g[:, None]).astype(np.float32)
    s = _shape(N, d)
    r = O.residual_nvfp4(s, O.F32, H[None], np.ones((1, N), np.float32),
                         np.zeros((1, 1, d), np.float32), np.zeros((1, N), np.int32))
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(r["rscale"][0], g.astype(np.float32))
    assert np.array_equal(r["bscale"][0], sc)
    assert np.array_equal(r["codes"][0], codes)


def _dequant(codes, bscale, rscale):
    N, half = codes.shape
    d = half * 2
    nib = np.empty((N, d), np.uint8)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    v = np.where(nib & 8, -1.0, 1.0) * mags[nib & 7]
    s = np.array([[O.e4m3_decode(c) for c in row] for row in bscale], np.float64)
    return v * np.repeat(s, 16, axis=1) * rscale[:, None].astype(np.float64), np.repeat(s, 16, 1)


def test_nvfp4_error_bound_random_rows():
    """|r - rhat| <= eff * (half the E2M1 spacing at |v|), |v| = |r| / eff, for
    blocks whose decoded scale is in the E4M3 normal range; saturation of the
    scale rounding keeps |v| <= 6 * 16/15."""
    rng = np.random.default_rng(4)
    N, d, K = 48, 512, 3
    H = (rng.standard_normal((N, d)) * np.exp(rng.uniform(-3, 3, (N, 1)))).astype(np.float32)
    H[6, 64:80] *= 1e-4                     # a block far below the row maximum
    C = rng.standard_normal((K, d)).astype(np.float32) * 0.01
    C[:, 16:32] = 0.0
    H[5, 16:32] = 0.0                       # a block whose residual is exactly zero
    assign = rng.integers(0, K, size=N).astype(np.int32)
    rn = np.linalg.norm(H.astype(np.float64), axis=1).astype(np.float32)
    s = _shape(N, d, K)
    r = O.residual_nvfp4(s, O.F32, H[None], rn[None], C[None], assign[None])
    x = (H / rn[:, None]).astype(np.float32)
    res = (x - C[assign]).astype(np.float64)
    rhat, sdec = _dequant(r["codes"][0], r["bscale"][0], r["rscale"][0])
    eff = sdec * r["rscale"][0][:, None].astype(np.float64)
    err = np.abs(res - rhat)
    ok_blocks = sdec >= 2.0 ** -6
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.abs(res) / eff
    half = np.where(v <= 2, 0.25, np.where(v <= 4, 0.5, 1.0))
    over = np.maximum(v - 6.0, 0.0)
    bound = eff * np.maximum(half, over) * (1 + 1e-6) + 1e-30
    assert np.all(err[ok_blocks] <= bound[ok_blocks])
    assert np.all(v[ok_blocks] <= 6 * 16 / 15 + 1e-6)
    # the row maximum lands on the largest scale and code
    assert np.all(r["bscale"][0].max(axis=1) == 0x7E)
    # zero residual block: zero scale and zero codes
    assert r["bscale"][0][5, 1] == 0 and not r["codes"][0][5, 8:16].any()


def test_nvfp4_zero_residual_row():
    d = 64
    H = np.zeros((1, 2, d), np.float32)
    H[0, 1] = np.arange(d, dtype=np.float32) + 1
    rn = np.linalg.norm(H[0].astype(np.float64), axis=1).astype(np.float32)[None]
    C = np.zeros((1, 1, d), np.float32)
    C[0, 0] = (H[0, 1] / rn[0, 1]).astype(np.float32)  # exactly the unit row
    r = O.residual_nvfp4(_shape(2, d), O.F32, H, rn, C, np.zeros((1, 2), np.int32))
    # row 1 has residual exactly zero: all scales and codes zero
    assert r["rscale"][0, 1] == 0.0
    assert not r["codes"][0, 1].any() and not r["bscale"][0, 1].any()
    # row 0 is a zero row: x = 0, residual = -c
    assert r["rscale"][0, 0] > 0
