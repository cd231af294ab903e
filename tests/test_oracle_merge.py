"""Pins of the oracle's LSE merge (O5).

P5  * equals the pages' own pairwise update on finite inputs ("Add Unified
      Sequence Parallel attention", review thread: the Ring loop's
      out = prev_out - sigmoid(lse - prev_lse) * (prev_out - out),
      lse = prev_lse - logsigmoid(prev_lse - lse), in fp32 there, fp64 here),
      folded left to right over N partials;
    * commutative and associative;
    * a partial with LSE = -inf is the identity; all -inf gives (0, -inf);
    * merging the halves of an attention equals the whole (see P4 too).
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _pairwise_pages_form(o_parts, lse_parts):
    out = torch.from_numpy(o_parts[0].copy())
    lse = torch.from_numpy(lse_parts[0].copy())[..., None]
    for o_n, l_n in zip(o_parts[1:], lse_parts[1:]):
        o_n = torch.from_numpy(o_n)
        l_n = torch.from_numpy(l_n)[..., None]
        prev_out, prev_lse = out, lse
        out = prev_out - torch.sigmoid(l_n - prev_lse) * (prev_out - o_n)
        lse = prev_lse - torch.nn.functional.logsigmoid(prev_lse - l_n)
    return out.numpy(), lse[..., 0].numpy()


@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_p5_equals_pages_pairwise_update(n):
    rng = np.random.default_rng(n)
    o = [rng.standard_normal((5, 7, 3, 16)) for _ in range(n)]
    l = [rng.standard_normal((5, 7, 3)) * 4 + 8 for _ in range(n)]
    got_o, got_l = oracle.lse_merge(o, l)
    ref_o, ref_l = _pairwise_pages_form(o, l)
    np.testing.assert_allclose(got_o, ref_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(got_l, ref_l, rtol=0, atol=1e-13)


def test_p5_pages_form_gives_nan_on_empty_first_partial():
    # The reading replaces the pages' pairwise form where it breaks down: a
    # first partial with no allowed key (LSE = -inf) makes it NaN, the
    # max-shifted form returns the other partial unchanged.
    o = [np.zeros((1, 4)), np.arange(4.0)[None]]
    l = [np.array([-math.inf]), np.array([1.5])]
    ref_o, ref_l = _pairwise_pages_form(o, l)
    assert np.isnan(ref_l).all() or np.isnan(ref_o).any()
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
