"""Float32 lemmas the HIP quantizers rely on, checked on the CPU.

The HIP kernels encode an element x against an E4M3 scale s = 2^E * m
(m in [1, 2) with at most 3 fraction bits) without comparing x to the seven
midpoints times s. Instead they form the float32 quotient y = RN(x / m) with
one multiply and two FMA corrections, then let the gfx950 E2M1 down-convert
divide by 2^E and round to nearest even with saturation. These tests pin the
two facts that make this bit-identical to the rounding of the exact ratio
x / s (the definition the oracle implements):

* the corrected quotient equals the IEEE quotient bit for bit (exhaustive
  over every float32 significand of two binades, both signs, in C);
* rounding x / m to float32 never lands on an E2M1 midpoint unless x / m is
  exactly that midpoint, so the E2M1 code of RN(x / s) is the code of x / s
  (checked against the oracle's midpoint encoder for every positive E4M3
  scale, with x swept over +-64 ulps of every midpoint and grid point times
  s, plus random x).

The hardware down-convert itself (round to nearest even of y / 2^E, ties to
the even code, saturation, sign kept) is covered by the bit-exact GPU tests
of the row, probability-block and page quantizers.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle.formats import E2M1_GRID, e2m1_encode, e4m3_value

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_corrected_quotient_is_the_ieee_quotient():
    src = os.path.join(HERE, "arith", "quotient_check.c")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "qc")
        subprocess.run(["gcc", "-O2", "-o", exe, src, "-lm"], check=True)
        # -122: the lowest binade where the FMA remainder is still exact;
        # 0: any normal binade (the computation commutes with powers of two)
        r = subprocess.run([exe, "-122", "0"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout


def _rne_e2m1_of_f32(y: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code of float32 values y >= 0 (round to nearest, ties
    to the even code, saturating), by exact float64 midpoint compares."""
    y = y.astype(np.float64)
    code = np.zeros(y.shape, dtype=np.uint8)
    for k in range(7):
        mid = 0.5 * (E2M1_GRID[k] + E2M1_GRID[k + 1])
        code += ((y > mid) | ((y == mid) & ((k + 1) % 2 == 0))).astype(np.uint8)
    return code


def test_quotient_route_matches_exact_ratio_codes():
    rng = np.random.default_rng(7)
    codes = np.arange(1, 127, dtype=np.uint8)            # every positive finite E4M3 scale
    s_all = e4m3_value(codes).astype(np.float32)
    bases = np.concatenate([E2M1_GRID, 0.5 * (E2M1_GRID[:-1] + E2M1_GRID[1:]), [6.5, 7.0]])
    steps = np.arange(-64, 65, dtype=np.int64)
    checked = 0
    for s in s_all:
        xs = (bases * np.float64(s)).astype(np.float32)  # exact: few significant bits
        xi = xs.view(np.int32).astype(np.int64)[:, None] + steps[None, :]
        xi = xi[(xi >= 0) & (xi < 0x7F800000)]
        x = np.concatenate([xi.astype(np.int32).view(np.float32),
                            (rng.random(8192) * 7.0 * np.float64(s)).astype(np.float32)])
        fr, e = np.frexp(np.float64(s))                  # s = fr * 2^e, fr in [0.5, 1)
        m = np.float32(fr * 2.0)
        big_e = e - 1
        y = (x / m).astype(np.float32)                   # IEEE float32 quotient
        y = np.ldexp(y.astype(np.float64), -big_e)       # exact power-of-two scaling
        got = _rne_e2m1_of_f32(y)
        want = e2m1_encode(x, np.float32(s)) & np.uint8(7)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"s={s!r} x={x[bad[:4]]!r} got={got[bad[:4]]} want={want[bad[:4]]}"
        checked += x.size
    assert checked > 1_000_000
