"""The seeded input generators (CPU): determinism and the structure the
benchmarks and GPU tests rely on (sorted, distinct, in-range picks; the
drafted tokens' shared fraction)."""

import numpy as np

import synth


def test_draft_picks_structure():
    T, S, L, k, M, n = 60_000, 64, 1024, 512, 4, 6
    base = synth.drift_picks(2, T, S, L, k, n, seed=9, window=8192)
    d = synth.draft_picks(base, M, 0.75, seed=9)
    assert d.shape == (n, 2, M, k) and d.dtype == np.int32
    assert np.array_equal(d, synth.draft_picks(base, M, 0.75, seed=9))        # seeded
    for s in range(n):
        for b in range(2):
            bs = np.sort(base[s, b])
            assert np.array_equal(d[s, b, 0], bs)
            for j in range(M):
                row = d[s, b, j]
                assert np.all(np.diff(row) > 0)                                   # sorted, distinct
                assert row[0] >= bs[0] and row[-1] <= bs[-1]                      # in the base range
                if j:
                    assert np.intersect1d(row, bs).size == round(0.75 * k)        # shared picks


def test_drift_picks_structure():
    T, S, L, k = 40_000, 16, 256, 300
    p = synth.drift_picks(3, T, S, L, k, 5, seed=4, window=4096)
    assert p.shape == (5, 3, k)
    assert np.array_equal(p, synth.drift_picks(3, T, S, L, k, 5, seed=4, window=4096))
    assert np.all(np.diff(p, axis=-1) > 0) and p.min() >= S and p.max() < T - L
