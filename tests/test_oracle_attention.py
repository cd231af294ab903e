"""Pins of the oracle's attention (O3) to things other than itself.

P1  a library routine: torch's scaled_dot_product_attention and logsumexp
    on float64 CPU tensors;
P2  exhaustive brute force with correctly rounded sums (math.fsum) on tiny
    shapes, every mask kind, empty rows and empty key sets;
P3  closed forms (zero queries, constant values, one allowed key, identical
    keys);
P4  Ring chunk invariance: any split of the keys, merged by LSE, equals the
    unsplit call ("Context parallelism" docs, "Ring Attention": after one
    loop every GPU has seen every token's K/V).
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_sdpa(q, k, v, scale, mask=None, is_causal=False):
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=None if mask is None else torch.from_numpy(mask),
        is_causal=is_causal, scale=scale)
    scores = torch.matmul(tq, tk.transpose(-1, -2)) * scale
    if is_causal:
        Sq, Sk = q.shape[1], k.shape[1]
        keep = torch.ones(Sq, Sk, dtype=torch.bool).tril()
        scores = scores.masked_fill(~keep, float("-inf"))
    if mask is not None:
        scores = scores.masked_fill(~torch.from_numpy(mask), float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


@pytest.mark.parametrize("B,Sq,Sk,H,D", [(1, 37, 53, 2, 16), (2, 64, 64, 3, 64), (1, 5, 129, 1, 128)])
def test_p1_full_matches_torch_sdpa(B, Sq, Sk, H, D):
    q, k, v = _rand(1, B, Sq, H, D), _rand(2, B, Sk, H, D), _rand(3, B, Sk, H, D)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale)
    o_ref, lse_ref = _torch_sdpa(q, k, v, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,H,D", [(1, 1, 8), (57, 2, 32), (130, 2, 64)])
def test_p1_causal_matches_torch_sdpa(S, H, D):
    q, k, v = _rand(4, 1, S, H, D), _rand(5, 1, S, H, D), _rand(6, 1, S, H, D)
    scale = 0.37
    pos = oracle.positions({"kind": "causal", "off": 0}, S)
    o, lse = oracle.attention(q, k, v, scale, qpos=pos, kpos=pos)
    o_ref, lse_ref = _torch_sdpa(q, k, v, scale, is_causal=True)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_p1_offset_causal_matches_boolean_mask():
    # Sq != Sk, both sides offset; compared with torch using an explicit mask.
    Sq, Sk, H, D = 40, 70, 2, 16
    q, k, v = _rand(7, 1, Sq, H, D), _rand(8, 1, Sk, H, D), _rand(9, 1, Sk, H, D)
    qpos = oracle.positions({"kind": "causal", "off": 100}, Sq)
    kpos = oracle.positions({"kind": "causal", "off": 75}, Sk)
    mask = kpos[None, :] <= qpos[:, None]
    assert mask.any(axis=1).all()
    o, lse = oracle.attention(q, k, v, 0.25, qpos=qpos, kpos=kpos)
    o_ref, lse_ref = _torch_sdpa(q, k, v, 0.25, mask=mask)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P2 ----
def _brute(q, k, v, scale, qpos, kpos):
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    o = np.zeros((B, Sq, H, D))
    lse = np.full((B, Sq, H), -math.inf)
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                J = [j for j in range(Sk) if qpos is None or kpos[j] <= qpos[i]]
                if not J:
                    continue
                s = {j: scale * math.fsum(q[b, i, h, d] * k[b, j, h, d] for d in range(D)) for j in J}
                # softmax weights through the LSE rather than a running max
                L = max(s.values()) + math.log(math.fsum(math.exp(s[j] - max(s.values())) for j in J))
                for d in range(D):
                    o[b, i, h, d] = math.fsum(math.exp(s[j] - L) * v[b, j, h, d] for j in J)
                lse[b, i, h] = L
    return o, lse


MASKS = [
    ("full", None, None),
    ("causal", {"kind": "causal", "off": 3}, {"kind": "causal", "off": 0}),
    ("causal_empty_rows", {"kind": "causal", "off": 0}, {"kind": "causal", "off": 2}),
    ("zigzag", {"kind": "zigzag", "chunk": 2, "ids": [1, 6]}, {"kind": "zigzag", "chunk": 2, "ids": [0, 7]}),
    ("stripe", {"kind": "stripe", "rank": 1, "world": 3}, {"kind": "stripe", "rank": 2, "world": 3}),
]


@pytest.mark.parametrize("name,qd,kd", MASKS, ids=[m[0] for m in MASKS])
@pytest.mark.parametrize("Sq,Sk,D", [(4, 4, 4), (3, 4, 1), (4, 3, 2)])
def test_p2_brute_force_tiny(name, qd, kd, Sq, Sk, D):
    rng = np.random.default_rng(zlib.crc32(f"{name}/{Sq}/{Sk}/{D}".encode()))
    B, H = 2, 2
    q, k, v = (rng.standard_normal((B, n, H, D)) for n in (Sq, Sk, Sk))
    qpos = oracle.positions(qd, Sq)
    kpos = oracle.positions(kd, Sk)
    o, lse = oracle.attention(q, k, v, 0.7, qpos=qpos, kpos=kpos)
    o_ref, lse_ref = _brute(q, k, v, 0.7, qpos, kpos)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-14)
    if name == "causal_empty_rows":
        # query positions 0,1 precede every key position (>= 2): no key allowed
        assert np.isneginf(lse[:, :2]).all() and (o[:, :2] == 0).all()


def test_p2_empty_kv():
    q = _rand(10, 1, 3, 2, 4)
    k = np.zeros((1, 0, 2, 4))
    o, lse = oracle.attention(q, k, k, 1.0)
    assert (o == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------- P3 ----
def test_p3_zero_queries_give_mean_and_log_count():
    S, H, D = 23, 2, 8
    q = np.zeros((1, S, H, D))
    k, v = _rand(11, 1, S, H, D), _rand(12, 1, S, H, D)
    pos = oracle.positions({"kind": "causal", "off": 0}, S)
    o, lse = oracle.attention(q, k, v, 0.5, qpos=pos, kpos=pos)
    for i in range(S):
        np.testing.assert_allclose(o[0, i], v[0, : i + 1].mean(axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, i], math.log(i + 1), rtol=0, atol=1e-14)


def test_p3_constant_values_give_the_constant():
    q, k = _rand(13, 1, 9, 1, 16), _rand(14, 1, 31, 1, 16)
    v = np.full((1, 31, 1, 16), 2.5)
    o, _ = oracle.attention(q, k, v, 1.3)
    np.testing.assert_allclose(o, 2.5, rtol=0, atol=1e-14)


def test_p3_single_allowed_key():
    S, D = 12, 8
    q, k, v = _rand(15, 1, S, 1, D), _rand(16, 1, S, 1, D), _rand(17, 1, S, 1, D)
    pos = oracle.positions({"kind": "causal", "off": 0}, S)
    o, lse = oracle.attention(q, k, v, 0.9, qpos=pos, kpos=pos)
    # first causal row sees key 0 only
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])
    np.testing.assert_allclose(lse[0, 0, 0], 0.9 * float(np.dot(q[0, 0, 0], k[0, 0, 0])), rtol=0, atol=1e-14)
    # Sk = 1
    o1, l1 = oracle.attention(q, k[:, 5:6], v[:, 5:6], 0.9)
    np.testing.assert_array_equal(o1[0, :, 0], np.broadcast_to(v[0, 5, 0], (S, D)))
    np.testing.assert_allclose(l1[0, :, 0], 0.9 * q[0, :, 0] @ k[0, 5, 0], rtol=0, atol=1e-13)


def test_p3_identical_keys_give_uniform_weights():
    q, v = _rand(18, 1, 6, 2, 8), _rand(19, 1, 17, 2, 8)
    k = np.broadcast_to(_rand(20, 1, 1, 2, 8), (1, 17, 2, 8)).copy()
    o, lse = oracle.attention(q, k, v, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), rtol=0, atol=1e-14)
    s = 0.3 * np.einsum("bihd,bhd->bih", q, k[:, 0])
    np.testing.assert_allclose(lse, s + math.log(17), rtol=0, atol=1e-13)


def test_p3_scale_enters_once():
    # doubling the scale equals doubling the queries
    q, k, v = _rand(21, 1, 7, 1, 8), _rand(22, 1, 11, 1, 8), _rand(23, 1, 11, 1, 8)
    a = oracle.attention(q, k, v, 0.8)
    b = oracle.attention(2 * q, k, v, 0.4)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P4 ----
@pytest.mark.parametrize("bounds", [[0, 129, 257], [0, 100, 101, 257], [0, 0, 257],
                                    [0, 32, 64, 96, 128, 160, 192, 224, 257], [0, 3, 250, 257, 257]])
@pytest.mark.parametrize("causal", [False, True])
def test_p4_ring_chunks_equal_unsplit(bounds, causal):
    S, H, D = 257, 2, 16
    q, k, v = _rand(24, 1, S, H, D), _rand(25, 1, S, H, D), _rand(26, 1, S, H, D)
    pos = np.arange(S, dtype=np.int64)
    kc = [k[:, a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    vc = [v[:, a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    kp = [pos[a:b] for a, b in zip(bounds[:-1], bounds[1:])] if causal else None
    o, lse = oracle.ring_pass(q, kc, vc, 0.125, qpos=pos if causal else None, kpos_chunks=kp)
    o_ref, lse_ref = oracle.attention(q, k, v, 0.125, qpos=pos if causal else None,
                                      kpos=pos if causal else None)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_rows_subset_equals_full_rows():
    q, k, v = _rand(27, 2, 19, 3, 8), _rand(28, 2, 23, 3, 8), _rand(29, 2, 23, 3, 8)
    o, lse = oracle.attention(q, k, v, 0.5)
    rows = [0, 5, 18, 19, 37]
    os_, ls_ = oracle.attention(q, k, v, 0.5, rows=rows)
    for n, r in enumerate(rows):
        np.testing.assert_array_equal(os_[n], o[r // 19, r % 19])
        np.testing.assert_array_equal(ls_[n], lse[r // 19, r % 19])
