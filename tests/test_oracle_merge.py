"""Pins for the merge oracle (CPU only).

Fixed by the pages: the two-split hand computation of "5.1.1 · 从索引到 Kernel"
§3.2 eq. (7) and the four-split denominator of §7.1 eq. (14).  Fixed by
mathematics: the normalised-partition form of the PagedAttention page §1.4
gives the same result; an empty split takes no part.
"""

import math

import numpy as np

import oracle


def test_two_split_example(golden):
    g = golden("merge_examples.txt")
    m = np.asarray(g["two_split_m"], float)[:, None]
    l = np.asarray(g["two_split_l"], float)[:, None]
    o = np.asarray(g["two_split_o"], float)[:, None, None]
    out, lse = oracle.merge(o, m, l)
    L = 3 + 4 / math.e
    assert abs(L - g["two_split_l_merged"][0]) < 5e-4          # page rounds to 3 decimals
    assert abs(6 + 8 / math.e - g["two_split_o_merged"][0]) < 5e-4
    assert abs(out[0, 0] - g["two_split_out"][0]) < 1e-12      # exactly 2
    assert abs(lse[0] - (2 + math.log(L))) < 1e-12
    naive = (o[:, 0, 0] / l[:, 0]).sum()
    assert naive == g["two_split_naive_wrong"][0] and abs(naive - out[0, 0]) > 1


def test_four_split_denominator(golden):
    g = golden("merge_examples.txt")
    m = np.asarray(g["four_split_m"], float)[:, None]
    l = np.asarray(g["four_split_l"], float)[:, None]
    o = np.ones((4, 1, 1))
    _, lse = oracle.merge(o, m, l)
    L = math.exp(lse[0] - 9)
    assert abs(L - g["four_split_l_merged"][0]) < 5e-3          # page: ~17.85
    assert abs(L - (12 / math.e + 18 / math.e**2 + 10 + 20 / math.e**3)) < 1e-12


def test_empty_split_is_ignored():
    o = np.asarray([[[1.0, 2.0]], [[0.0, 0.0]], [[5.0, 1.0]]])
    m = np.asarray([[0.5], [np.inf], [1.5]])       # the empty split's m is garbage
    l = np.asarray([[2.0], [0.0], [3.0]])
    out, lse = oracle.merge(o, m, l)
    keep = oracle.merge(o[[0, 2]], m[[0, 2]], l[[0, 2]])
    assert np.allclose(out, keep[0]) and np.allclose(lse, keep[1])
    out_e, lse_e = oracle.merge(np.zeros((2, 1, 3)), np.full((2, 1), -np.inf), np.zeros((2, 1)))
    assert np.all(out_e == 0) and np.isneginf(lse_e).all()


def test_normalized_form_agrees():
    rng = np.random.default_rng(1)
    S, H, dv = 5, 3, 7
    m = rng.normal(size=(S, H)) * 3
    l = rng.uniform(0.5, 4, size=(S, H))
    l[2, 1] = 0.0
    o = rng.normal(size=(S, H, dv))
    o[2, 1] = 0.0
    a = oracle.merge(o, m, l)
    On = np.where(l[..., None] > 0, o / np.where(l > 0, l, 1)[..., None], 0)
    b = oracle.merge_normalized(On, m, l)
    assert np.allclose(a[0], b[0], atol=1e-13) and np.allclose(a[1], b[1], atol=1e-13)
