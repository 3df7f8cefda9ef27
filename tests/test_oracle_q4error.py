"""Pins for the oracle's quantization-error measurement (no GPU): the uniform
grid's spacing, codes at the grid values and at the midpoints, brute-force
loops, the h^2/12 mean square error of evenly spread values, and the
half-gap bound on the maximum error."""

import numpy as np

import oracle


def test_uniform_grid_is_evenly_spaced_on_minus_one_to_one():
    u = oracle.UNIFORM4.astype(np.float64)
    assert u[0] == -1.0 and u[-1] == 1.0 and u.size == 16
    assert np.allclose(np.diff(u), 2.0 / 15.0, rtol=0, atol=2e-7)
    assert np.array_equal(u, -u[::-1])  # symmetric, no value at zero


def test_codes_at_grid_values_and_midpoints():
    u = oracle.UNIFORM4
    # a block whose absmax is exactly 1 (first element): x equals w
    for i in range(16):
        w = np.zeros(64, dtype=np.float32)
        w[0] = 1.0
        w[1] = u[i]
        codes = oracle.nf4_codes(w, oracle.blockwise_absmax(w), table=u)
        assert codes[1] == i
    # the midpoint of codes 7 and 8 is exactly 0: a tie, so the lower code
    w = np.zeros(64, dtype=np.float32)
    w[0] = 1.0
    codes = oracle.nf4_codes(w, oracle.blockwise_absmax(w), table=u)
    assert codes[1] == 7
    # just above a midpoint goes up, just below stays
    for j in range(15):
        m = (float(u[j]) + float(u[j + 1])) / 2.0
        lo = np.nextafter(np.float32(m), np.float32(-2.0))
        hi = np.nextafter(np.float32(m), np.float32(2.0))
        w = np.array([1.0, lo, hi] + [0.0] * 61, dtype=np.float32)
        c = oracle.nf4_codes(w, oracle.blockwise_absmax(w), table=u)
        assert c[1] == j and c[2] == j + 1


def test_quant_error_matches_brute_force_loops():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(200) * 0.1).astype(np.float32)  # three whole blocks and a short one
    for name, table in oracle.GRIDS.items():
        sse, ssw, mx = 0.0, 0.0, 0.0
        for b0 in range(0, w.size, 64):
            blk = w[b0:b0 + 64]
            a = np.float32(max(abs(float(v)) for v in blk))
            inv = np.float32(1.0) / a
            for v in blk:
                x = float(np.float32(v * inv))
                best = min(range(16), key=lambda c: (abs(x - float(table[c])), c))
                wq = float(np.float32(table[best] * a))
                e = float(v) - wq
                sse += e * e
                ssw += float(v) * float(v)
                mx = max(mx, abs(e))
        got = oracle.quant_error(w, table)
        assert abs(got[0] - sse) <= 1e-12 * sse, name
        assert abs(got[1] - ssw) <= 1e-12 * ssw, name
        assert got[2] == mx, name


def test_uniform_grid_mse_of_evenly_spread_values_is_h2_over_12():
    # every block: absmax exactly 1, the other 63 values spread evenly over
    # [-1, 1]; the squared error of a value uniform on a cell of width h
    # averages h^2 / 12
    rng = np.random.default_rng(4)
    nb = 4096
    w = rng.uniform(-1.0, 1.0, size=(nb, 64)).astype(np.float32)
    w[:, 0] = 1.0
    sse, _, mx = oracle.quant_error(w, oracle.UNIFORM4)
    h = 2.0 / 15.0
    assert abs(sse / w.size - h * h / 12.0) < 0.02 * h * h / 12.0
    assert mx <= h / 2.0 + 1e-6


def test_max_error_within_half_the_largest_gap():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    a = oracle.blockwise_absmax(w)
    for name, table in oracle.GRIDS.items():
        gap = float(np.max(np.diff(table.astype(np.float64))))
        _, _, mx = oracle.quant_error(w, table)
        assert mx <= gap / 2.0 * float(np.max(a)) * (1 + 1e-6), name


def test_zero_and_empty_inputs():
    for table in oracle.GRIDS.values():
        assert oracle.quant_error(np.zeros(100, dtype=np.float32), table) == (0.0, 0.0, 0.0)
        assert oracle.quant_error(np.zeros(0, dtype=np.float32), table) == (0.0, 0.0, 0.0)
