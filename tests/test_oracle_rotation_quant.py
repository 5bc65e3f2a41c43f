"""Oracle pins for the rotation and the block quantizers (CPU only).

Rotation: Sylvester Hadamard orthogonality (integers), agreement with a dense
float64 matrix product, round trip. Quantizers: exact reproduction of on-grid
blocks, brute-force choice between the scale candidates in exact rational
arithmetic, the float32 pairwise error tree, tau = 0 reducing to amax6 (the
config's "scaling disabled" mode), and c = 1 / c = 8 consistency.
"""
from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import quant as Q
from oracle import rotation as R

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E4M3 = [float(v) for v in F.e4m3_value(np.arange(0x7F, dtype=np.uint8))]


# ----------------------------------------------------------------- rotation

def test_hadamard_is_orthogonal():
    H = R.hadamard_matrix()
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    assert np.array_equal(H, H.T)


def test_fwht_equals_dense_product():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    H = R.hadamard_matrix().astype(np.float64)
    ref = x.astype(np.float64) @ H.T
    got = R.fwht(x).astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    # unit vectors map to Hadamard columns exactly
    e = np.eye(128, dtype=np.float32)
    assert np.array_equal(R.fwht(e), H.astype(np.float32))


def test_rotation_round_trip_and_constant():
    assert np.float32(R.INV_SQRT_D).view(np.uint32) == 0x3DB504F3
    rng = np.random.default_rng(1)
    x = rng.standard_normal((256, 128)).astype(np.float32)
    back = R.rotate(R.rotate(x))
    assert np.max(np.abs(back - x)) <= 1e-6 * np.max(np.abs(x)) * 8
    # norm preserving
    n0 = np.linalg.norm(x.astype(np.float64), axis=1)
    n1 = np.linalg.norm(R.rotate(x).astype(np.float64), axis=1)
    assert np.allclose(n0, n1, rtol=1e-6)


def test_fwht_stage_order_is_fixed():
    # a row whose float32 result depends on the order of the additions
    x = np.zeros(128, np.float32)
    x[0], x[1], x[2], x[3] = 2.0 ** 24, 1.0, 1.0, -2.0 ** 24
    y = R.fwht(x)
    # h=1: (x0+x1, x0-x1) = (2^24, 2^24-1), (x2+x3, x2-x3) = (1-2^24, 2^24);
    # h=2: y0 = 2^24 + (1-2^24) = 1 (a left-to-right sum of the four gives 0)
    assert y[0] == np.float32(1.0)
    assert y[1] == np.float32(2.0 ** 24 - 1 + 2.0 ** 24)


# ----------------------------------------------------------------- sse tree

def test_sse_tree_is_pairwise():
    e = np.array([2.0 ** 24, 1.0, 1.0, -2.0 ** 24], np.float32)
    assert Q.sse_tree(e) == np.float32(1.0)          # sequential order gives 0
    rng = np.random.default_rng(2)
    v = rng.random((100, 16)).astype(np.float32)
    assert np.allclose(Q.sse_tree(v), v.astype(np.float64).sum(-1), rtol=1e-6)


# ----------------------------------------------------------------- on-grid

def _on_grid_blocks(rng, n, gmax, nblk=16):
    s = np.array([E4M3[i] for i in rng.integers(8, len(E4M3) - 10, n)], np.float32)
    g = rng.choice(GRID, size=(n, nblk)) * rng.choice([-1.0, 1.0], size=(n, nblk))
    g[:, rng.integers(0, nblk)] = gmax * rng.choice([-1.0, 1.0])
    g = np.where(np.abs(g) > gmax, np.sign(g) * gmax, g)
    return s, (g * s[:, None]).astype(np.float32), g


def test_amax6_reproduces_on_grid_blocks():
    rng = np.random.default_rng(3)
    s, x, _ = _on_grid_blocks(rng, 500, 6.0)
    nib, sc = Q.quantize_amax6(x)
    assert np.array_equal(F.e4m3_value(sc[:, 0]).astype(np.float32), s)
    assert np.array_equal(Q.dequantize(nib, sc, Q.AMAX6), x.astype(np.float64))


def test_four_six_picks_four_on_grid_blocks():
    rng = np.random.default_rng(4)
    s, x, _ = _on_grid_blocks(rng, 500, 4.0)
    nib, sc = Q.quantize_four_six(x)
    assert np.array_equal(Q.dequantize(nib, sc, Q.FOUR_SIX), x.astype(np.float64))


def _exact_sse(xb, s):
    tot = Fraction(0)
    for xv in xb:
        fx = Fraction(float(xv))
        m = _nearest(fx, s)
        sign = -1 if np.signbit(xv) else 1
        tot += (fx - sign * Fraction(GRID[m]) * s) ** 2
    return tot


def _nearest(x: Fraction, s: Fraction) -> int:
    if s == 0:
        return 0
    r = abs(x) / s
    return min(range(8), key=lambda m: (abs(r - Fraction(GRID[m])), m % 2))


def test_four_six_choice_matches_exact_bruteforce():
    rng = np.random.default_rng(5)
    checked = 0
    for _ in range(300):
        x = (rng.standard_normal(16) * np.exp(rng.uniform(-3, 3))).astype(np.float32)
        a = float(np.max(np.abs(x)))
        s6 = Fraction(float(F.e4m3_value(F.e4m3_encode(np.float32(a) / np.float32(6)))))
        s4 = Fraction(float(F.e4m3_value(F.e4m3_encode(np.float32(a) / np.float32(4)))))
        e6, e4 = _exact_sse(x, s6), _exact_sse(x, s4)
        if e6 != 0 and abs(e4 - e6) / e6 < Fraction(1, 10 ** 5):
            continue                      # too close for a float32 error sum
        nib, sc = Q.quantize_four_six(x)
        want = s4 if e4 < e6 else s6
        assert Fraction(float(F.e4m3_value(sc[0]))) == want
        for xv, nv in zip(x, nib):
            assert (nv & 7) == _nearest(Fraction(float(xv)), want)
        checked += 1
    assert checked > 250


def test_mx_exponent_is_least_with_amax_le_6_pow2():
    rng = np.random.default_rng(6)
    a = np.exp(rng.uniform(-40, 40, 5000)).astype(np.float32)
    a = np.concatenate([a, np.float32(6.0) * np.exp2(np.arange(-30, 30)).astype(np.float32)])
    e = Q.mx_exponent_hi(a)
    for ai, ei in zip(a, e):
        fa = Fraction(float(ai))
        assert fa <= 6 * Fraction(2) ** int(ei)
        assert fa > 6 * Fraction(2) ** int(ei - 1)
        ocp = int(np.floor(np.log2(float(ai)))) - 2          # OCP MX floor rule, emax(E2M1) = 2
        assert ocp in (int(ei), int(ei) - 1)


def test_mxfp4_choice_matches_exact_bruteforce():
    rng = np.random.default_rng(7)
    checked = 0
    for _ in range(200):
        x = (rng.standard_normal(32) * np.exp(rng.uniform(-4, 4))).astype(np.float32)
        a = float(np.max(np.abs(x)))
        ehi = int(Q.mx_exponent_hi(np.array([a], np.float32))[0])
        shi, slo = Fraction(2) ** ehi, Fraction(2) ** (ehi - 1)
        ehi_err, elo_err = _exact_sse(x, shi), _exact_sse(x, slo)
        if abs(elo_err - ehi_err) / max(ehi_err, Fraction(1, 10 ** 30)) < Fraction(1, 10 ** 5):
            continue
        nib, sc = Q.quantize_mxfp4_search(x)
        want = ehi - 1 if elo_err < ehi_err else ehi
        assert int(sc[0]) == want + 127
        s = Fraction(2) ** want
        for xv, nv in zip(x, nib):
            assert (nv & 7) == _nearest(Fraction(float(xv)), s)
        checked += 1
    assert checked > 150


def test_mxfp4_zero_block_and_on_grid():
    nib, sc = Q.quantize_mxfp4_search(np.zeros((2, 32), np.float32))
    assert not nib.any() and not sc.any()
    rng = np.random.default_rng(8)
    g = rng.choice(GRID, size=(50, 32)) * rng.choice([-1.0, 1.0], size=(50, 32))
    g[:, 0] = 6.0
    E = rng.integers(-20, 20, size=50)
    x = (g * np.exp2(E)[:, None]).astype(np.float32)
    nib, sc = Q.quantize_mxfp4_search(x)
    assert np.array_equal(sc.astype(np.int64)[:, 0], E + 127)
    assert np.array_equal(Q.dequantize(nib, sc, Q.MXFP4_SEARCH), x.astype(np.float64))


# ----------------------------------------------------------------- P quantizer

def test_p_tau_zero_is_amax6_and_large_tau_is_amax2():
    rng = np.random.default_rng(9)
    pp = (8.0 * np.exp(-rng.exponential(3.0, size=(400, 16)))).astype(np.float32)
    n0, s0 = Q.quantize_p(pp, Q.AMAX2_OR_AMAX6, np.float32(0.0))
    n6, s6 = Q.quantize_p(pp, Q.AMAX6, None)
    assert np.array_equal(n0, n6) and np.array_equal(s0, s6)
    nb, sb = Q.quantize_p(pp, Q.AMAX2_OR_AMAX6, np.float32(448.0))
    a = pp.max(axis=1)
    assert np.array_equal(sb[:, 0], F.e4m3_encode((a / np.float32(2)).astype(np.float32)))


def test_p_branch_direction_and_bruteforce():
    rng = np.random.default_rng(10)
    tau = np.float32(1.0)
    pp = (8.0 * np.exp(-rng.exponential(2.0, size=(300, 16)))).astype(np.float32)
    nib, sc = Q.quantize_p(pp, Q.AMAX2_OR_AMAX6, tau)
    for row, nr, s in zip(pp, nib, sc):
        a = np.max(row)
        k = np.float32(2.0) if a < tau else np.float32(6.0)
        want = F.e4m3_encode(np.float32(a) / k)
        assert s == want
        sv = Fraction(float(F.e4m3_value(want)))
        for xv, nv in zip(row, nr):
            assert nv == _nearest(Fraction(float(xv)), sv)


def test_p_c1_c8_codes_agree_and_scales_differ_by_8():
    rng = np.random.default_rng(11)
    p = np.exp(-rng.exponential(1.0, size=(300, 16)))
    p[:, 0] = 1.0
    n1, s1 = Q.quantize_p(p.astype(np.float32), Q.AMAX6, None)
    n8, s8 = Q.quantize_p((8.0 * p).astype(np.float32), Q.AMAX6, None)
    s1, s8 = s1[:, 0], s8[:, 0]
    normal = F.e4m3_value(s1) >= 2.0 ** -6
    assert normal.all()
    assert np.array_equal(n1[normal], n8[normal])
    assert np.array_equal(F.e4m3_value(s8)[normal], 8.0 * F.e4m3_value(s1)[normal])


# ----------------------------------------------------------------- query

def test_two_term_query_residual():
    rng = np.random.default_rng(12)
    q = R.rotate(rng.standard_normal((200, 128)).astype(np.float32))
    terms1, q1 = Q.quantize_query(q, Q.AMAX6, 1)
    terms2, q2 = Q.quantize_query(q, Q.AMAX6, 2)
    e1 = np.linalg.norm(q - q1, axis=1)
    e2 = np.linalg.norm(q - q2, axis=1)
    assert len(terms1) == 1 and len(terms2) == 2
    assert np.all(e2 < e1 * 0.5)
    r = (q - Q.dequantize(*terms2[0], Q.AMAX6).astype(np.float32)).astype(np.float32)
    nib, sc = Q.quantize_amax6(r)
    assert np.array_equal(nib, terms2[1][0]) and np.array_equal(sc, terms2[1][1])
    # an on-grid query leaves a zero second term
    s, x, _ = _on_grid_blocks(rng, 8, 6.0)
    t, qh = Q.quantize_query(x.reshape(1, 128), Q.AMAX6, 2)
    assert not t[1][0].any() and np.array_equal(qh[0], x.reshape(-1).astype(np.float64))
