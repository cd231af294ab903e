"""Pins of the oracle's Ulysses permute (O2) and of the UAA pass (O7).

P6  * seq2head equals "concatenate the shards along the sequence, keep the
      rank's heads" and head2seq equals "concatenate the head shards along
      heads, keep the rank's tokens" (numpy slicing, bit-exact);
    * head2seq after seq2head is the identity, bit-exact, for every rank;
    * the emitted index map equals an index map built with numpy;
    * one rank is a plain copy.
P7  The Ulysses Anything pass with uneven (and empty) shards and uneven heads
    equals unsplit attention BIT-EXACTLY ("Context parallelism" docs,
    "Ulysses Anything Attention": any sequence length or head count, no
    padding; "UAA: Ulysses Anything Attention": zero padding).
"""

import numpy as np
import pytest

import oracle


def _shards(x, off):
    return [x[:, off[p]:off[p + 1]] for p in range(len(off) - 1)]


SPLITS = [
    ([0, 129, 257], [0, 1, 2]),            # the tiny ragged share
    ([0, 5, 5, 12, 20], [0, 2, 3, 3, 7]),   # empty shard, uneven heads
    ([0, 0, 9], [0, 3, 5]),
    ([0, 4, 8, 12], [0, 1, 2, 3]),
]


@pytest.mark.parametrize("seq_off,head_off", SPLITS)
@pytest.mark.parametrize("dtype", [np.uint16, np.float32, np.int32, np.float64])
def test_p6_seq2head_is_concat_then_head_slice(seq_off, head_off, dtype):
    B, H, D = 2, head_off[-1], 3
    S = seq_off[-1]
    x = np.random.default_rng(1).integers(0, 60000, size=(B, S, H, D)).astype(dtype)
    shards = _shards(x, seq_off)
    world = len(seq_off) - 1
    for r in range(world):
        y = oracle.seq2head(shards, r, seq_off, head_off)
        ref = np.concatenate(shards, axis=1)[:, :, head_off[r]:head_off[r + 1]]
        assert y.dtype == x.dtype and y.shape == ref.shape
        assert y.tobytes() == ref.tobytes()


@pytest.mark.parametrize("seq_off,head_off", SPLITS)
def test_p6_head2seq_is_concat_then_token_slice(seq_off, head_off):
    B, H, D = 2, head_off[-1], 4
    S = seq_off[-1]
    world = len(seq_off) - 1
    rng = np.random.default_rng(2)
    heads = [rng.standard_normal((B, S, head_off[r + 1] - head_off[r], D)).astype(np.float32)
             for r in range(world)]
    for p in range(world):
        z = oracle.head2seq(heads, p, seq_off, head_off)
        ref = np.concatenate(heads, axis=2)[:, seq_off[p]:seq_off[p + 1]]
        assert z.tobytes() == ref.tobytes()


@pytest.mark.parametrize("seq_off,head_off", SPLITS)
def test_p6_round_trip_is_identity(seq_off, head_off):
    B, H, D = 1, head_off[-1], 5
    x = np.random.default_rng(3).standard_normal((B, seq_off[-1], H, D)).astype(np.float32)
    world = len(seq_off) - 1
    shards = _shards(x, seq_off)
    heads = [oracle.seq2head(shards, r, seq_off, head_off) for r in range(world)]
    back = [oracle.head2seq(heads, p, seq_off, head_off) for p in range(world)]
    for p in range(world):
        assert back[p].tobytes() == np.ascontiguousarray(shards[p]).tobytes()


@pytest.mark.parametrize("seq_off,head_off", SPLITS)
def test_p6_index_map_matches_numpy_map(seq_off, head_off):
    B, H, D = 2, head_off[-1], 2
    world = len(seq_off) - 1
    # numpy-built map: element (b, s, h, d) of the global tensor, sliced
    for r in range(world):
        shard, elem = oracle.seq2head_index(r, world, seq_off, head_off, B, H, D)
        b, s, h, d = np.meshgrid(np.arange(B), np.arange(seq_off[-1]),
                                 np.arange(head_off[r], head_off[r + 1]), np.arange(D), indexing="ij")
        p_ref = np.searchsorted(np.asarray(seq_off), s, side="right") - 1
        # zero-length shards share an offset: the owner is the last of them
        t = s - np.asarray(seq_off)[p_ref]
        Sp = np.diff(seq_off)[p_ref]
        e_ref = ((b * Sp + t) * H + h) * D + d
        np.testing.assert_array_equal(shard, p_ref)
        np.testing.assert_array_equal(elem, e_ref)


def test_p6_single_rank_is_copy():
    x = np.random.default_rng(4).standard_normal((2, 9, 3, 4))
    y = oracle.seq2head([x], 0, [0, 9], [0, 3])
    assert y.tobytes() == x.tobytes()
    z = oracle.head2seq([x], 0, [0, 9], [0, 3])
    assert z.tobytes() == x.tobytes()


def test_p6_rejects_bad_offsets():
    x = np.zeros((1, 4, 2, 2))
    with pytest.raises(ValueError):
        oracle.seq2head([x, x], 0, [0, 4, 3], [0, 1, 2])
    with pytest.raises(ValueError):
        oracle.seq2head([x, x], 0, [1, 4, 8], [0, 1, 2])


def test_o1_split_policy():
    assert oracle.split_offsets(257, 2) == [0, 129, 257]
    assert oracle.split_offsets(4481, 2) == [0, 2241, 4481]
    assert oracle.split_offsets(4608, 2) == [0, 2304, 4608]
    assert oracle.split_offsets(3, 5) == [0, 1, 2, 3, 3, 3]
    assert oracle.split_offsets(24, 2) == [0, 12, 24]


# ---------------------------------------------------------------- P7 ----
@pytest.mark.parametrize("S,H,P,seq_off,head_off", [
    (257, 2, 2, None, None),
    (61, 3, 2, None, None),                       # uneven heads 2/1
    (40, 4, 3, [0, 0, 17, 40], None),
    (26, 4, 3, [0, 9, 18, 26], [0, 1, 1, 4]),     # a rank with no heads
    (33, 5, 3, [0, 11, 11, 33], [0, 2, 4, 5]),
])
@pytest.mark.parametrize("causal", [False, True])
def test_p7_uaa_pass_equals_unsplit_bit_exact(S, H, P, seq_off, head_off, causal):
    D = 8
    rng = np.random.default_rng(S * 10 + H)
    q, k, v = (rng.standard_normal((1, S, H, D)) for _ in range(3))
    o, lse = oracle.uaa_pass(q, k, v, 0.3, P, causal=causal, seq_off=seq_off, head_off=head_off)
    pos = np.arange(S, dtype=np.int64) if causal else None
    o_ref, lse_ref = oracle.attention(q, k, v, 0.3, qpos=pos, kpos=pos)
    assert o.tobytes() == o_ref.tobytes()
    assert lse.tobytes() == lse_ref.tobytes()
