"""Hand-derived worked examples (tests/golden/*.json, each with the page it
follows and its derivation) checked against the oracle.  The pages print no
numeric example of their own; these values come from the definitions by hand,
not from any code in this repository."""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f(x):
    return -math.inf if x == "-inf" else float(x)


def test_golden_attention_two_keys():
    g = _load("attention_two_keys.json")
    q = np.array(g["q"])[None, :, None, :]
    k = np.array(g["k"])[None, :, None, :]
    v = np.array(g["v"])[None, :, None, :]
    o, lse = oracle.attention(q, k, v, g["scale"])
    np.testing.assert_allclose(o[0, :, 0], g["full"]["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, :, 0], g["full"]["lse"], rtol=0, atol=1e-15)
    c = g["causal"]
    o, lse = oracle.attention(q, k, v, g["scale"], qpos=np.array(c["qpos"]), kpos=np.array(c["kpos"]))
    np.testing.assert_allclose(o[0, :, 0], c["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, :, 0], c["lse"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("case", range(4))
def test_golden_merge(case):
    c = _load("merge_partials.json")["cases"][case]
    o_parts = [np.array([row]) for row in c["o"]]
    l_parts = [np.array([_f(x)]) for x in c["lse"]]
    o, lse = oracle.lse_merge(o_parts, l_parts)
    np.testing.assert_allclose(o[0], c["o_out"], rtol=0, atol=1e-15)
    if c["lse_out"] == "-inf":
        assert np.isneginf(lse[0])
    else:
        np.testing.assert_allclose(lse[0], c["lse_out"], rtol=0, atol=1e-15)


def test_golden_permute():
    g = _load("permute_small.json")
    shards = [np.array(s, dtype=np.int32).reshape(shape) for s, shape in zip(g["shards"], g["shard_shapes"])]
    for r in range(2):
        y = oracle.seq2head(shards, r, g["seq_off"], g["head_off"])
        assert y.reshape(-1).tolist() == g["seq2head"][r]
    heads = [oracle.seq2head(shards, r, g["seq_off"], g["head_off"]) for r in range(2)]
    z = oracle.head2seq(heads, 1, g["seq_off"], g["head_off"])
    assert z.reshape(-1).tolist() == g["head2seq_rank1"]


def test_golden_positions():
    g = _load("positions_small.json")
    for z in g["zigzag"]:
        pos = oracle.positions({"kind": "zigzag", "chunk": z["chunk"], "ids": z["ids"]}, z["n"])
        assert pos.tolist() == z["pos"]
    for s in g["stripe"]:
        pos = oracle.positions({"kind": "stripe", "rank": s["rank"], "world": s["world"]}, s["n"])
        assert pos.tolist() == s["pos"]
