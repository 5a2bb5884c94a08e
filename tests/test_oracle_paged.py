"""Pins for the oracle's paged-cache quantize / dequantize (no GPU): with the identity block
table they reduce to the dense calls with one group per page (pinned elsewhere); a
permuted table moves whole pages and nothing else; skipped entries touch nothing; a page
named twice is gathered twice."""
import numpy as np

import oracle
from tests.test_oracle_quant import _gauss


def _setup(n_blocks=9, rpp=24, d=128, seed=7):
    return _gauss(n_blocks * rpp, d, seed), n_blocks, rpp, d


def test_identity_table_equals_dense_groups():
    x, nb, rpp, d = _setup()
    tab = np.arange(nb, dtype=np.int32)
    for rule in ("static_6", "mse"):
        c, s, a = oracle.quantize_paged(x, tab, rpp, nb, rule)
        dc, ds, da = oracle.quantize(x, rpp, rule)
        assert np.array_equal(c.reshape(dc.shape), dc) and np.array_equal(s.reshape(ds.shape), ds)
        assert np.array_equal(a, da)
        y = oracle.dequantize_paged(c, s, a, tab, rpp)
        assert np.array_equal(y, oracle.dequantize(dc, ds, da, rpp))


def test_permuted_table_moves_whole_pages():
    x, nb, rpp, d = _setup(seed=8)
    perm = np.random.default_rng(1).permutation(nb + 3)[:nb].astype(np.int32)  # 3 spare pages
    c, s, a = oracle.quantize_paged(x, perm, rpp, nb + 3, "mse")
    dc, ds, da = oracle.quantize(x, rpp, "mse")
    for b, pg in enumerate(perm):
        assert np.array_equal(c[pg], dc[b * rpp:(b + 1) * rpp])
        assert np.array_equal(s[pg], ds[b * rpp:(b + 1) * rpp])
        assert a[pg] == da[b]
    unused = sorted(set(range(nb + 3)) - set(perm.tolist()))
    assert not c[unused].any() and not s[unused].any() and not a[unused].any()
    y = oracle.dequantize_paged(c, s, a, perm, rpp)
    assert np.array_equal(y, oracle.dequantize(dc, ds, da, rpp))


def test_skipped_entries_and_repeated_pages():
    x, nb, rpp, d = _setup(seed=9)
    tab = np.arange(nb, dtype=np.int32)
    c, s, a = oracle.quantize_paged(x, tab, rpp, nb, "static_6")
    gather = np.array([3, -1, 3, nb, 0], dtype=np.int32)   # -1 and nb are outside the pages
    y0 = np.full((gather.size * rpp, d), 0x1234, np.uint16)
    y = oracle.dequantize_paged(c, s, a, gather, rpp, y=y0.copy())
    ref3 = oracle.dequantize_rows(c[3], s[3], a[3])
    assert np.array_equal(y[0:rpp], ref3) and np.array_equal(y[2 * rpp:3 * rpp], ref3)
    assert np.all(y[rpp:2 * rpp] == 0x1234) and np.all(y[3 * rpp:4 * rpp] == 0x1234)
    assert np.array_equal(y[4 * rpp:], oracle.dequantize_rows(c[0], s[0], a[0]))
    # quantize with a skipped entry leaves that page's bytes as they were
    c2 = np.full_like(c, 0x77)
    s2 = np.full_like(s, 0x11)
    a2 = np.full_like(a, 5.0)
    tab2 = tab.copy()
    tab2[4] = -7
    oracle.quantize_paged(x, tab2, rpp, nb, "static_6", c2, s2, a2)
    assert np.all(c2[4] == 0x77) and np.all(s2[4] == 0x11) and a2[4] == 5.0
    assert np.array_equal(c2[5], c[5]) and a2[5] == a[5]
