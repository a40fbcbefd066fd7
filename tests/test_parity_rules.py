"""CPU: the comparison rules the GPU parity tests use are strict where they should be."""
import numpy as np

from tests.parity import REL_TOL, elemrel, maxrel


def test_elemrel_catches_a_small_element_that_maxrel_lets_through():
    rs = np.random.RandomState(0)
    ref = np.exp(rs.uniform(-6, 0, 4096))          # statistics spanning orders of magnitude
    x = ref.copy()
    small = int(np.argmin(ref))
    x[small] *= 1.2                                 # 20% off on an element 400x below the max
    assert maxrel(x, ref) <= REL_TOL                # a head-wide maximum does not see it
    assert elemrel(x, ref) > REL_TOL                # the element-wise rule does


def test_elemrel_passes_rounding_level_noise_and_uses_the_floor():
    rs = np.random.RandomState(1)
    ref = np.exp(rs.uniform(-6, 0, 4096))
    x = ref * (1 + rs.uniform(-1e-5, 1e-5, ref.size))
    assert elemrel(x, ref) < 1e-4
    ref2 = ref.copy()
    ref2[0] = 1e-40                                  # underflows to 0 in fp32 on the GPU
    x2 = ref2.copy()
    x2[0] = 0.0
    assert elemrel(x2, ref2) <= REL_TOL


def test_elemrel_signed_sums_against_their_term_magnitudes():
    ref = np.array([1e-9, -2.0, 3.0])               # first sum cancels almost exactly
    mag = np.array([5.0, 2.0, 3.0])                 # sum of its terms' magnitudes
    x = ref + np.array([1e-6, 0.0, 0.0])
    assert elemrel(x, ref, mag) <= REL_TOL
    assert elemrel(x, ref) > REL_TOL


def test_selection_read_back_from_compaction_sources():
    from oracle import kvs_oracle as O
    from tests.parity import selection_from_src
    rs = np.random.RandomState(3)
    for N, S, R in ((40, 3, 5), (41, 0, 0), (7, 2, 1)):
        P = O.num_pairs(N, S, R)
        sel = rs.rand(P) < 0.4
        K = rs.randn(N, 4)
        _, _, _, src = O.compact(K, K, np.ones(N, np.int64), np.full((P, 2), 0.5), sel, S)
        assert np.array_equal(selection_from_src(src, S, P), sel)
