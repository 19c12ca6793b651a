"""Sweeps, on the GPU, over every input of the ranges on which the NVFP4
coder's fast path uses gfx950's conversions and its Newton reciprocal
(drift_aware_kv_amd/csrc/ps_nvfp4_fast.h), against expectations that come from
outside the library:

* fp32 -> E2M1 over every finite fp32 pattern (2^32 minus the non-finite
  ones), written into every nibble position the coder uses, against the step
  function of the OCP microscaling E2M1 rounding table (tests/golden/
  e2m1_ties.txt: nearest, ties to even, saturating at 6, zero as +0);
* fp32 -> E4M3 over every pattern in [0, 464), the range of the coder's
  block-scale quotients, against nearest-even rounding onto the E4M3 values
  that the CPU oracle decodes (whose encoder is pinned against torch's
  float8_e4m3fn elsewhere); the thresholds are checked against the oracle's
  encoder on both sides of every one;
* E4M3 -> fp32 for every code 0 .. 0x7e against the oracle's decoder;
* the Newton reciprocal over every normal fp32 b in [2^-126, 2^126): the
  relative error |1 - b y| below 2^-52 (the coder's quotient argument needs
  2^-51).

The kernels live in a test-only library (tests/hwcheck) built from the same
header the coder includes."""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "hwcheck", "libps_hwcheck.so")
GOLDEN = os.path.join(HERE, "golden", "e2m1_ties.txt")
CHUNK = 1 << 28
U64 = (1 << 64) - 1


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def X():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(LIB), f"{LIB} is not built (python tests/hwcheck/build.py)"
    L = ctypes.CDLL(LIB)
    L.psx_e2m1_sweep.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32),
                                 ctypes.c_void_p]
    L.psx_e4m3_sweep.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p]
    L.psx_e4m3_decode.argtypes = [ctypes.c_void_p, ctypes.c_int]
    L.psx_recip_sweep.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p]
    return L


def f32bits(x):
    return int(np.float32(x).view(np.uint32))


def e2m1_thresholds_from_golden():
    """Bit pattern at which each E2M1 magnitude index 1..7 begins: at each
    midpoint between neighbouring values, the table says which way the tie
    goes."""
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if line:
            rows.append((np.float32(line[0]), int(line[1]), float(line[2])))
    value = {}
    for _, idx, v in rows:
        value.setdefault(idx, v)
    assert sorted(value) == list(range(8))
    at = {float(x): idx for x, idx, _ in rows}
    thr = []
    for i in range(1, 8):
        m = np.float32((value[i - 1] + value[i]) / 2)
        assert float(m) in at, f"the table gives no tie case at {m}"
        thr.append(f32bits(m) if at[float(m)] == i else f32bits(m) + 1)
    return thr


def e4m3_thresholds():
    """Bit pattern at which each E4M3 code 1..0x7e begins under nearest-even
    rounding onto the values the oracle decodes (the midpoint goes to the
    even code; 0x7e = 448 takes everything above)."""
    vals = [O.e4m3_decode(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:])) and vals[-1] == 448.0
    thr = []
    for c in range(1, 0x7F):
        m = np.float32((vals[c - 1] + vals[c]) / 2)
        assert float(m) == (vals[c - 1] + vals[c]) / 2          # midpoints are fp32 numbers
        thr.append(f32bits(m) if c % 2 == 0 else f32bits(m) + 1)
    return thr


def _run(sweep, lo, hi, out):
    for base in range(lo, hi, CHUNK):
        assert sweep(base, min(CHUNK, hi - base)) == 0, "launch failed"
    torch.cuda.synchronize()
    return [int(v) & U64 for v in out.cpu().tolist()]


def test_e2m1_every_finite_fp32(X):
    thr = e2m1_thresholds_from_golden()
    assert [np.uint32(t).view(np.float32) for t in thr][0] > 0.25     # 0.25 is a tie to zero
    t7 = (ctypes.c_uint32 * 7)(*thr)
    out = torch.tensor([0, -1], dtype=torch.int64, device="cuda")
    say("E2M1 sweep over 2^32 patterns")
    bad, first = _run(lambda b, n: X.psx_e2m1_sweep(b, n, t7, out.data_ptr()), 0, 1 << 32, out)
    assert bad == 0, f"{bad} patterns differ; first {first:#010x}"


def test_e4m3_every_quotient_below_464(X):
    thr = e4m3_thresholds()
    for c, t in enumerate(thr, start=1):       # the oracle's encoder agrees on both sides
        assert O.e4m3_encode(np.uint32(t).view(np.float32)) == c
        assert O.e4m3_encode(np.uint32(t - 1).view(np.float32)) == c - 1
    thr_dev = torch.tensor(np.array(thr, np.uint32).view(np.int32), device="cuda")
    out = torch.tensor([0, -1], dtype=torch.int64, device="cuda")
    hi = f32bits(464.0)
    say(f"E4M3 sweep over [0, 464): {hi} patterns")
    bad, first = _run(lambda b, n: X.psx_e4m3_sweep(b, n, thr_dev.data_ptr(), len(thr), out.data_ptr()),
                      0, hi, out)
    assert bad == 0, f"{bad} patterns differ; first {first:#010x}"


def test_e4m3_decode_every_code(X):
    out = torch.zeros(0x7F, dtype=torch.float32, device="cuda")
    assert X.psx_e4m3_decode(out.data_ptr(), 0x7F) == 0
    got = out.cpu().numpy()
    want = np.array([O.e4m3_decode(c) for c in range(0x7F)], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_newton_reciprocal_every_normal_divisor(X):
    out = torch.tensor([0, -1, 0], dtype=torch.int64, device="cuda")
    lo, hi = f32bits(2.0 ** -126), f32bits(2.0 ** 126)
    say(f"reciprocal sweep over [2^-126, 2^126): {hi - lo} patterns")
    bad, first, worst = _run(lambda b, n: X.psx_recip_sweep(b, n, 2.0 ** -52, out.data_ptr()), lo, hi, out)
    worst = float(np.array([worst], np.uint64).view(np.float64)[0])
    say(f"  largest |1 - b y| = {worst:.3e} = 2^{np.log2(worst):.2f}")
    assert bad == 0, f"{bad} divisors with |1 - b y| >= 2^-52; first {first:#010x}"
