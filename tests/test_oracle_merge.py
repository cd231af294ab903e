"""Pins of the oracle's LSE merge (O5).

P5  * equals the pages' own way of merging ("Add Unified Sequence Parallel
      attention", review thread: the Ring loop folds each step's (out, lse)
      into the running pair, in fp32 there): two partials at a time, the
      result is the mean of the two outputs weighted by e^lse of each, and
      its LSE is log(e^lse_a + e^lse_b); folded left to right over N
      partials, in fp64 here;
    * commutative and associative;
    * a partial with LSE = -inf is the identity; all -inf gives (0, -inf);
    * merging the halves of an attention equals the whole (see P4 too).
"""

import math

import numpy as np
import pytest

import oracle


def _pairwise_fold(o_parts, lse_parts):
    """Fold the partials two at a time: (a, la) and (b, lb) become the mean
    of a and b weighted e^la : e^lb -- b's weight is the logistic function of
    lb - la -- with LSE log(e^la + e^lb).  Valid for finite LSEs."""
    out = np.array(o_parts[0], dtype=np.float64)
    lse = np.array(lse_parts[0], dtype=np.float64)
    for o_n, l_n in zip(o_parts[1:], lse_parts[1:]):
        w = 1.0 / (1.0 + np.exp(lse - l_n))
        out = out + w[..., None] * (o_n - out)
        lse = np.logaddexp(lse, l_n)
    return out, lse


@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_p5_equals_pairwise_fold(n):
    rng = np.random.default_rng(n)
    o = [rng.standard_normal((5, 7, 3, 16)) for _ in range(n)]
    l = [rng.standard_normal((5, 7, 3)) * 4 + 8 for _ in range(n)]
    got_o, got_l = oracle.lse_merge(o, l)
    ref_o, ref_l = _pairwise_fold(o, l)
    np.testing.assert_allclose(got_o, ref_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(got_l, ref_l, rtol=0, atol=1e-13)


def test_p5_pairwise_lse_update_breaks_on_an_empty_partial():
    # Why the merge is written max-shifted (reading 6): the pages fold the
    # new LSE in as the running LSE plus log(1 + e^(new - running)).  With
    # no key seen so far the running LSE is -inf, the exponent +inf, and the
    # sum -inf + inf is NaN in IEEE arithmetic; the max-shifted merge gives
    # the other partial unchanged.
    with np.errstate(over="ignore", invalid="ignore"):
        run, new = np.float64(-np.inf), np.float64(1.5)
        assert np.isnan(run + np.log1p(np.exp(new - run)))
    o = [np.zeros((1, 4)), np.arange(4.0)[None]]
    l = [np.array([-math.inf]), np.array([1.5])]
    got_o, got_l = oracle.lse_merge(o, l)
    np.testing.assert_array_equal(got_o, o[1])
    np.testing.assert_array_equal(got_l, l[1])


def test_p5_commutative_and_associative():
    rng = np.random.default_rng(7)
    o = [rng.standard_normal((64, 32)) for _ in range(3)]
    l = [rng.standard_normal(64) * 3 for _ in range(3)]
    a = oracle.lse_merge(o, l)
    b = oracle.lse_merge(o[::-1], l[::-1])
    left = oracle.lse_merge([oracle.lse_merge(o[:2], l[:2])[0], o[2]],
                            [oracle.lse_merge(o[:2], l[:2])[1], l[2]])
    right = oracle.lse_merge([o[0], oracle.lse_merge(o[1:], l[1:])[0]],
                             [l[0], oracle.lse_merge(o[1:], l[1:])[1]])
    for x in (b, left, right):
        np.testing.assert_allclose(x[0], a[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(x[1], a[1], rtol=0, atol=1e-13)


def test_p5_neg_inf_partial_is_identity():
    rng = np.random.default_rng(8)
    o1, l1 = rng.standard_normal((10, 8)), rng.standard_normal(10)
    o0, l0 = rng.standard_normal((10, 8)), np.full(10, -math.inf)
    got = oracle.lse_merge([o0, o1, o0], [l0, l1, l0])
    np.testing.assert_array_equal(got[0], o1)
    np.testing.assert_array_equal(got[1], l1)


def test_p5_all_neg_inf_gives_zero_and_neg_inf():
    o = [np.ones((3, 4)), np.ones((3, 4))]
    l = [np.full(3, -math.inf)] * 2
    got = oracle.lse_merge(o, l)
    assert (got[0] == 0).all() and np.isneginf(got[1]).all()


def test_p5_single_partial_is_copy():
    rng = np.random.default_rng(9)
    o, l = rng.standard_normal((6, 8)), rng.standard_normal(6)
    got = oracle.lse_merge([o], [l])
    np.testing.assert_array_equal(got[0], o)
    np.testing.assert_array_equal(got[1], l)


def test_p5_large_lse_gap_does_not_overflow():
    o = [np.full((1, 2), 1.0), np.full((1, 2), 3.0)]
    l = [np.array([1000.0]), np.array([-1000.0])]
    got = oracle.lse_merge(o, l)
    np.testing.assert_allclose(got[0], 1.0, rtol=0, atol=1e-300)
    np.testing.assert_allclose(got[1], 1000.0, rtol=0, atol=1e-12)
