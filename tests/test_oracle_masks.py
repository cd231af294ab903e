"""Pins of the oracle's position maps (O4) and of the Unified pass (O8).

The USP / yunchang summary ("How It Works", "Highlighted Details") names
the zigzag, stripe and basic ring layouts for load balancing but does not
define them; the readings live in oracle.positions.  What pins them is that
every layout, run as a full Ring (and Unified) pass with position-causal
masking and the LSE merge, must give plain causal attention over the whole
sequence (P8).  A wrong chunk assignment or a wrong position formula breaks
that equality.
"""

import numpy as np
import pytest

import oracle
from oracle.oracle import ring_layout_tokens, zigzag_chunks


def test_zigzag_chunk_assignment_of_the_long_context_share():
    # rank 1 of a 4-rank zigzag ring holds global chunks 1 and 6 of 8
    assert zigzag_chunks(1, 4) == [1, 6]
    assert [zigzag_chunks(r, 4) for r in range(4)] == [[0, 7], [1, 6], [2, 5], [3, 4]]
    pos = oracle.positions({"kind": "zigzag", "chunk": 4096, "ids": [1, 6]}, 8192)
    assert pos[0] == 4096 and pos[4095] == 8191 and pos[4096] == 6 * 4096 and pos[-1] == 7 * 4096 - 1


def test_layouts_partition_the_sequence():
    for layout, S, R in (("basic", 37, 3), ("zigzag", 48, 3), ("stripe", 36, 4)):
        toks = np.concatenate(ring_layout_tokens(S, R, layout))
        assert sorted(toks.tolist()) == list(range(S))


def test_stripe_positions():
    pos = oracle.positions({"kind": "stripe", "rank": 2, "world": 4}, 5)
    assert pos.tolist() == [2, 6, 10, 14, 18]


@pytest.mark.parametrize("layout,S,R", [("basic", 61, 3), ("zigzag", 64, 4), ("stripe", 60, 4),
                                        ("zigzag", 48, 2), ("stripe", 45, 3)])
def test_p8_ring_layouts_equal_plain_causal(layout, S, R):
    H, D = 2, 8
    rng = np.random.default_rng(S + R)
    q, k, v = (rng.standard_normal((1, S, H, D)) for _ in range(3))
    o, lse = oracle.usp_pass(q, k, v, 0.4, ulysses=1, ring=R, layout=layout, causal=True)
    pos = np.arange(S, dtype=np.int64)
    o_ref, lse_ref = oracle.attention(q, k, v, 0.4, qpos=pos, kpos=pos)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout,S,P,R", [("zigzag", 48, 2, 2), ("basic", 50, 2, 2), ("stripe", 40, 3, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_p8_unified_grid_equals_unsplit(layout, S, P, R, causal):
    H, D = 5, 8
    rng = np.random.default_rng(S * P + R)
    q, k, v = (rng.standard_normal((1, S, H, D)) for _ in range(3))
    o, lse = oracle.usp_pass(q, k, v, 0.4, ulysses=P, ring=R, layout=layout, causal=causal)
    pos = np.arange(S, dtype=np.int64) if causal else None
    o_ref, lse_ref = oracle.attention(q, k, v, 0.4, qpos=pos, kpos=pos)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_p8_zigzag_share_equals_rows_of_full_causal():
    # scaled-down long-context share: 8 chunks, this rank holds chunks {1, 6}
    C, R, H, D = 6, 4, 2, 8
    S = 2 * R * C
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, S, H, D)) for _ in range(3))
    qpos = oracle.positions({"kind": "zigzag", "chunk": C, "ids": [1, 6]}, 2 * C)
    kc = [k[:, c * C:(c + 1) * C] for c in range(2 * R)]
    vc = [v[:, c * C:(c + 1) * C] for c in range(2 * R)]
    kp = [np.arange(c * C, (c + 1) * C, dtype=np.int64) for c in range(2 * R)]
    o, lse = oracle.ring_pass(q[:, qpos], kc, vc, 0.3, qpos=qpos, kpos_chunks=kp)
    pos = np.arange(S, dtype=np.int64)
    o_ref, lse_ref = oracle.attention(q, k, v, 0.3, qpos=pos, kpos=pos)
    np.testing.assert_allclose(o, o_ref[:, qpos], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref[:, qpos], rtol=0, atol=1e-12)
    # chunk 7 lies after every query position: its partial is empty
    o7, l7 = oracle.attention(q[:, qpos], kc[7], vc[7], 0.3, qpos=qpos, kpos=kp[7])
    assert (o7 == 0).all() and np.isneginf(l7).all()


def test_p8_wrong_zigzag_assignment_is_detected():
    # a plausible mistake (rank r holding chunks r and 2R-r) must break P8
    C, R, H, D = 4, 3, 1, 4
    S = 2 * R * C
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((1, S, H, D)) for _ in range(3))
    good = oracle.positions({"kind": "zigzag", "chunk": C, "ids": [1, 2 * R - 2]}, 2 * C)
    bad = oracle.positions({"kind": "zigzag", "chunk": C, "ids": [1, 2 * R - 1]}, 2 * C)
    pos = np.arange(S, dtype=np.int64)
    o_ref, _ = oracle.attention(q, k, v, 0.5, qpos=pos, kpos=pos)
    o_bad, _ = oracle.attention(q[:, good], k, v, 0.5, qpos=bad, kpos=pos)
    assert not np.allclose(o_bad, o_ref[:, good])
