"""Pins of the oracle's ladder: binary16 rounding against numpy's float16 conversion, and the
ladder's own invariants.  The rule itself is a reading (the pages take the ladder from a
converter whose source is not on them); its parity with the pages' bytes is unpinned."""
import numpy as np

import oracle


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(4000) * 10.0,
        rng.standard_normal(1000) * 1e-5,           # subnormal range of binary16
        rng.standard_normal(500) * 3e4,
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 6.103515625e-05, 5.960464477539063e-08,
                  2.98e-08, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -(2.0 + 2.0 ** -10)]),
    ])
    for x in xs:
        ref = float(np.float16(x))
        got = oracle.f16_round(float(x))
        assert got == ref or (np.isinf(ref) and np.isinf(got)), (x, got, ref)


def test_ladder_invariants():
    rng = np.random.default_rng(1)
    rows, n = 20, 256
    W = (rng.standard_normal((rows, n)) * np.exp(rng.standard_normal((rows, 1)))).astype(np.float32)
    W[3, :] = 0.0                       # an all-zero row
    W[5, 64:] = 0.0                     # zero groups do not count
    dead = np.zeros(n, dtype=bool)
    dead[[7, 100]] = True
    lost, tab = oracle.ladder(W, dead)
    for r in range(rows):
        lo, st = float(lost[r, 0]), float(lost[r, 1])
        assert oracle.f16_round(lo) == lo and oracle.f16_round(st) == st
        if r == 3:
            assert lo == 0.0 and st == 0.0 and np.all(tab[r] == 1.0)
            continue
        Wz = W[r].copy()
        Wz[dead] = 0.0
        a = np.abs(Wz.reshape(-1, 32)).max(axis=1)
        a = a[a > 0]
        np.testing.assert_allclose(lo, np.log2(a.min() / 7.0), atol=2 ** -10 * max(1, abs(lo)))
        assert tab[r, 0] == np.float32(2.0 ** lo)
        assert np.all(np.diff(tab[r]) >= 0)
        top = lo + 31 * st
        np.testing.assert_allclose(top, np.log2(a.max() / 7.0), atol=31 * 2 ** -10 * max(st, 1e-3) + 2 ** -9)


def test_dead_columns_are_ignored_by_the_ladder():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((4, 64)) * 0.01).astype(np.float32)
    dead = np.zeros(64, dtype=bool)
    dead[10] = True
    W2 = W.copy()
    W2[:, 10] = 50.0
    a = oracle.ladder(W, dead)
    b = oracle.ladder(W2, dead)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
