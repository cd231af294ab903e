"""Pins of the oracle's attention backward (oracle.attention_bwd) to things
other than itself.

B1  central finite differences of the oracle's forward (oracle.c, pinned on
    its own in test_oracle_attention.py) along random directions, for every
    mask kind, ragged shapes, rows with no allowed key and a non-zero LSE
    gradient, and element by element on a tiny case;
B2  a library routine: torch autograd through scaled_dot_product_attention
    on float64 CPU tensors;
B3  closed forms: one key (P = 1 everywhere); dK and dV sums fixed by the
    softmax's invariances (a common shift of every key moves each score
    row by a constant, the rows of P sum to one); the scaling identity
    <dQ, Q> = <dK, K> (scores are unchanged by Q -> aQ, K -> K / a).
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, scale, qpos, kpos, dout, dlse):
    """L = sum(dout * O) + sum(dlse * LSE) over rows that see a key."""
    o, lse = oracle.attention(q, k, v, scale, qpos=qpos, kpos=kpos)
    live = np.isfinite(lse)
    return float((dout * o).sum() + (np.where(live, dlse, 0.0) * np.where(live, lse, 0.0)).sum())


CASES = {
    # name: (B, Sq, Sk, H, D, qpos, kpos)
    "full": (2, 7, 5, 2, 8, None, None),
    "full_one_query": (1, 1, 9, 1, 4, None, None),
    "causal_square": (1, 9, 9, 2, 8, np.arange(9), np.arange(9)),
    "causal_offset_dead_rows": (1, 6, 8, 1, 8, np.arange(6) + 3, np.arange(8) + 5),
    "zigzag_ring_chunk": (1, 8, 8, 2, 4,
                          oracle.positions({"kind": "zigzag", "chunk": 4, "ids": [1, 2]}, 8),
                          oracle.positions({"kind": "zigzag", "chunk": 4, "ids": [0, 3]}, 8)),
    "stripe": (2, 5, 6, 1, 8, oracle.positions({"kind": "stripe", "rank": 0, "world": 2}, 5),
               oracle.positions({"kind": "stripe", "rank": 1, "world": 2}, 6)),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("with_dlse", [False, True])
def test_b1_directional_finite_differences(name, with_dlse):
    B, Sq, Sk, H, D, qpos, kpos = CASES[name]
    seed = sum(map(ord, name)) + (7 if with_dlse else 0)
    q, k, v = _rand(seed, B, Sq, H, D), _rand(seed + 1, B, Sk, H, D), _rand(seed + 2, B, Sk, H, D)
    dout = _rand(seed + 3, B, Sq, H, D)
    dlse = _rand(seed + 4, B, Sq, H) if with_dlse else np.zeros((B, Sq, H))
    scale = 0.6
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, scale, qpos, kpos, dlse if with_dlse else None)
    eps = 1e-6
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        u = _rand(seed + 10 + len(which) * 3 + ord(which), *grad.shape)
        args = {"q": q, "k": k, "v": v}

        def f(t):
            a = dict(args)
            a[which] = args[which] + t * u
            return _loss(a["q"], a["k"], a["v"], scale, qpos, kpos, dout, dlse)

        fd = (f(eps) - f(-eps)) / (2 * eps)
        an = float((grad * u).sum())
        assert abs(fd - an) <= 1e-7 * (1 + abs(an)), (which, fd, an)


def test_b1_elementwise_finite_differences():
    # every element of every gradient, causal with one dead query row
    B, Sq, Sk, H, D = 1, 3, 4, 1, 2
    qpos, kpos = np.array([0, 2, 5]), np.array([1, 2, 3, 4])
    q, k, v = _rand(31, B, Sq, H, D), _rand(32, B, Sk, H, D), _rand(33, B, Sk, H, D)
    dout, dlse = _rand(34, B, Sq, H, D), _rand(35, B, Sq, H)
    scale = 1.3
    grads = oracle.attention_bwd(q, k, v, dout, scale, qpos, kpos, dlse)
    eps = 1e-6
    for t_idx, grad in enumerate(grads):
        for idx in np.ndindex(grad.shape):
            plus = [q.copy(), k.copy(), v.copy()]
            minus = [q.copy(), k.copy(), v.copy()]
            plus[t_idx][idx] += eps
            minus[t_idx][idx] -= eps
            fd = (_loss(*plus, scale, qpos, kpos, dout, dlse) - _loss(*minus, scale, qpos, kpos, dout, dlse)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-8 * (1 + abs(fd)), (t_idx, idx, fd, grad[idx])
    # the dead row (query 0 sees no key) gets no gradient
    assert np.all(grads[0][0, 0] == 0.0)


def _torch_grads(q, k, v, dout, scale, mask):
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).clone().requires_grad_(True)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).clone().requires_grad_(True)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).clone().requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale)
    o.backward(torch.from_numpy(dout).permute(0, 2, 1, 3))
    return [t.grad.permute(0, 2, 1, 3).numpy() for t in (tq, tk, tv)]


@pytest.mark.parametrize("B,Sq,Sk,H,D,causal", [(1, 33, 47, 2, 16, False), (2, 40, 40, 3, 32, True),
                                                 (1, 3, 130, 1, 64, False)])
def test_b2_matches_torch_autograd(B, Sq, Sk, H, D, causal):
    q, k, v = _rand(41, B, Sq, H, D), _rand(42, B, Sk, H, D), _rand(43, B, Sk, H, D)
    dout = _rand(44, B, Sq, H, D)
    scale = 1.0 / math.sqrt(D)
    qpos = kpos = mask = None
    if causal:
        qpos, kpos = np.arange(Sq), np.arange(Sk)
        mask = kpos[None, :] <= qpos[:, None]
    got = oracle.attention_bwd(q, k, v, dout, scale, qpos, kpos)
    ref = _torch_grads(q, k, v, dout, scale, mask)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


def test_b3_single_key_closed_form():
    # one key: P = 1, O_i = v_0, LSE_i = scale q_i . k_0
    B, Sq, H, D = 2, 5, 2, 8
    q, k, v = _rand(51, B, Sq, H, D), _rand(52, B, 1, H, D), _rand(53, B, 1, H, D)
    dout, dlse = _rand(54, B, Sq, H, D), _rand(55, B, Sq, H)
    scale = 0.8
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, scale, dlse=dlse)
    np.testing.assert_allclose(dv[:, 0], dout.sum(axis=1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, scale * dlse[..., None] * k, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk[:, 0], scale * (dlse[..., None] * q).sum(axis=1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["full", "causal_offset_dead_rows", "zigzag_ring_chunk"])
def test_b3_invariances(name):
    B, Sq, Sk, H, D, qpos, kpos = CASES[name]
    q, k, v = _rand(61, B, Sq, H, D), _rand(62, B, Sk, H, D), _rand(63, B, Sk, H, D)
    dout, dlse = _rand(64, B, Sq, H, D), _rand(65, B, Sq, H)
    scale = 0.45
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, scale, qpos, kpos, dlse)
    live = np.ones(Sq, dtype=bool) if qpos is None else (kpos[None, :] <= qpos[:, None]).any(axis=1)
    lw = live[None, :, None, None]
    # k_j -> k_j + c for every j: every score of row i moves by scale q_i . c
    np.testing.assert_allclose(dk.sum(axis=1), scale * (np.where(lw, dlse[..., None] * q, 0)).sum(axis=1),
                               rtol=0, atol=1e-11)
    # v_j -> v_j + c for every j: every live O row moves by c
    np.testing.assert_allclose(dv.sum(axis=1), np.where(lw, dout, 0).sum(axis=1), rtol=0, atol=1e-11)
    # Q -> a Q, K -> K / a leaves the scores unchanged
    assert abs((dq * q).sum() - (dk * k).sum()) <= 1e-11 * (1 + abs((dq * q).sum()))
