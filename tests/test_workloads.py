"""Seeded input generators: encodings and window draws (CPU only)."""

import numpy as np

import workloads as W


def test_e2m1_rne_ties_and_saturation():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.75, -3.0, 0.3, 0.0])
    codes = W.e2m1_codes(x).tolist()
    # ties go to the even code: 0.25->0 (0), 0.75->1.0 (2), 1.25->1.0 (2), 1.75->2.0 (4),
    # 2.5->2.0 (4), 3.5->4.0 (6), 5.0->4.0 (6); beyond 6 saturates to code 7
    assert codes == [0, 2, 2, 4, 4, 6, 6, 7, 7, 0x8 | 2, 0x8 | 5, 1, 0]


def test_pack_order():
    assert W.pack_nibbles(np.array([[1, 2, 3, 4]], np.uint8)).tolist() == [[0x21, 0x43]]
    assert int(W.pack_e8m0(np.array([1, 2, 3, 4], np.uint8))) == 0x04030201


def test_irregular_window_categories():
    for S_q, S_k, counts in ((8192, 65536, (6554, 1229, 409)), (129, 4100, (103, 19, 7))):
        s, e, kinds = W.irregular_windows(S_q, S_k, np.random.default_rng(5))
        assert tuple(int((kinds == c).sum()) for c in range(3)) == counts
        i = np.arange(S_q)
        c = kinds == 0
        assert np.all(e[c] == S_k - S_q + i[c]) and np.all(s[c] >= 1) and np.all(s[c] < e[c])
        sub = kinds == 1
        assert np.all(e[sub] > s[sub]) and np.all(e[sub] <= S_k) and np.all(s[sub] >= 0)
        em = kinds == 2
        assert np.all(s[em] == e[em]) and np.all((s[em] >= 0) & (s[em] <= S_k))


def test_named_shapes_and_determinism():
    a = W.make("c1")
    b = W.make("c1")
    assert a.q.shape == (1, 128, 64, 128) and a.q.dtype == np.uint16
    assert np.array_equal(a.q, b.q) and np.array_equal(a.w, b.w)
    m4 = W.make_random("mxfp4", 1, 4, 8, seed=3)
    assert m4.q.shape == (1, 4, 64, 64) and m4.k.shape == (1, 8, 64)
    by = m4.q_scale.view(np.uint8)
    assert by.min() >= 125 and by.max() <= 129
    z = W.make_random("mxfp8", 1, 4, 8, zero=True)
    assert np.all(z.q == 0) and np.all(z.q_scale == W.ONE_SCALE_WORD)
