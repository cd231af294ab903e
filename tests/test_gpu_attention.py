"""GPU parity of usp_attn_fwd_lse (and of the Ring step that merges its
partials) against the fp64 oracle.

* small shapes that span several tiles and ragged tails, every mask kind,
  bf16 (both output dtypes) and fp32, all rows checked;
* the workloads' attention calls at full size (one call over all keys of
  the FLUX shares, the Qwen chunks, the long-context chunks with their
  8-way merge), checked on sampled rows the oracle computes one by one; the
  exact step the bench times (its launches, kernels and streams) is checked
  on every row in test_gpu_step.py;
* edge cases: empty key set, rows with no allowed key, a key chunk after
  every query (O = 0, LSE = -inf), single rows, large scores.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import sequence_attention_dits_amd as uaa
from gpu_common import check_pair, dev, host_f64, sample_rows, say

pytestmark = pytest.mark.gpu


def _attn(q, k, v, scale, mask=None, out_dtype=None):
    B, Sq, H, D = q.shape
    odt = out_dtype or q.dtype
    o = torch.empty((B, Sq, H, D), device="cuda", dtype=odt)
    lse = torch.empty((B, Sq, H), device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale, mask)
    return o, lse


def _mask_and_positions(kind, Sq, Sk, **kw):
    """(usp_mask, qpos, kpos) for the oracle, from one description."""
    if kind == "full":
        return uaa.mask_full(), None, None
    if kind == "causal":
        qd = {"kind": "causal", "off": kw["q_off"]}
        kd = {"kind": "causal", "off": kw["k_off"]}
        m = uaa.mask_causal(kw["q_off"], kw["k_off"])
    elif kind == "zigzag":
        qd = {"kind": "zigzag", "chunk": kw["chunk"], "ids": kw["q_chunks"]}
        kd = {"kind": "zigzag", "chunk": kw["chunk"], "ids": kw["k_chunks"]}
        m = uaa.mask_zigzag(kw["chunk"], kw["q_chunks"], kw["k_chunks"])
    elif kind == "stripe":
        qd = {"kind": "stripe", "rank": kw["q_rank"], "world": kw["world"]}
        kd = {"kind": "stripe", "rank": kw["k_rank"], "world": kw["world"]}
        m = uaa.mask_stripe(kw["world"], kw["q_rank"], kw["k_rank"])
    else:
        raise ValueError(kind)
    return m, oracle.positions(qd, Sq), oracle.positions(kd, Sk)


SMALL = [
    # (name, B, Sq, Sk, H, D, mask kind, mask kwargs)
    ("full_ragged", 1, 257, 129, 2, 128, "full", {}),
    ("full_tiles", 2, 256, 192, 3, 64, "full", {}),
    ("full_tail1", 1, 129, 65, 1, 128, "full", {}),
    ("single_row", 1, 1, 300, 2, 128, "full", {}),
    ("single_key", 1, 200, 1, 2, 64, "full", {}),
    ("causal_square", 1, 300, 300, 2, 128, "causal", {"q_off": 0, "k_off": 0}),
    ("causal_offset_empty_rows", 1, 190, 250, 2, 128, "causal", {"q_off": 0, "k_off": 60}),
    ("causal_past_chunk", 1, 160, 140, 1, 64, "causal", {"q_off": 500, "k_off": 100}),
    ("zigzag_two_chunks", 1, 192, 96, 2, 128, "zigzag", {"chunk": 96, "q_chunks": [1, 6], "k_chunks": [3]}),
    ("zigzag_both_sides", 1, 100, 100, 2, 64, "zigzag", {"chunk": 50, "q_chunks": [1, 6], "k_chunks": [0, 7]}),
    ("stripe", 1, 150, 170, 2, 128, "stripe", {"world": 4, "q_rank": 1, "k_rank": 2}),
]


@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("bf16", "fp32"), ("fp32", "fp32")])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_all_rows(case, dtype, out):
    name, B, Sq, Sk, H, D, kind, kw = case
    say("attn small", name, dtype, out)
    cfg = 900 + SMALL.index(case)
    qb, qv = synth.tensor(cfg, 0, (B, Sq, H, D), dtype, rms_norm=True)
    kb, kv_ = synth.tensor(cfg, 1, (B, Sk, H, D), dtype, rms_norm=True)
    vb, vv = synth.tensor(cfg, 2, (B, Sk, H, D), dtype)
    scale = 1.0 / math.sqrt(D)
    m, qpos, kpos = _mask_and_positions(kind, Sq, Sk, **kw)
    o, lse = _attn(dev(qb, dtype), dev(kb, dtype), dev(vb, dtype), scale, m,
                   out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qv, kv_, vv, np.float32(scale), qpos=qpos, kpos=kpos)
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16" if "bf16" in (dtype, out) else "fp32", name)


def test_empty_key_set_gives_zero_and_neg_inf():
    q = torch.randn(1, 70, 2, 128, device="cuda").to(torch.bfloat16)
    k = torch.empty(1, 0, 2, 128, device="cuda", dtype=torch.bfloat16)
    o, lse = _attn(q, k, k, 0.1)
    torch.cuda.synchronize()
    assert (o.float() == 0).all() and torch.isneginf(lse).all()


def test_large_scores_stay_finite():
    # scores of magnitude ~ 1e3 must not overflow the exponentials
    q = (torch.randn(1, 130, 1, 128, device="cuda") * 8).to(torch.bfloat16)
    k = (torch.randn(1, 150, 1, 128, device="cuda") * 8).to(torch.bfloat16)
    v = torch.randn(1, 150, 1, 128, device="cuda").to(torch.bfloat16)
    o, lse = _attn(q, k, v, 1.0)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(host_f64(q), host_f64(k), host_f64(v), 1.0)
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "large scores")


def test_rejects_unsupported_head_dim_and_bad_scale():
    q = torch.zeros(1, 4, 1, 96, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(uaa.UaaError) as e:
        _attn(q, q, q, 0.1)
    assert e.value.status == uaa.UAA_ERR_UNSUPPORTED
    q = torch.zeros(1, 4, 1, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(uaa.UaaError):
        _attn(q, q, q, -1.0)


# ---------------------------------------------------------------- full size
def _load(cfg, tag, shape, dtype, rms):
    bits, vals = synth.tensor(cfg, tag, shape, dtype, rms_norm=rms)
    return bits, vals


def test_tiny_fp32_share_ring_pass():
    """Tiny ragged fp32 share: attention over the full 257 tokens per head
    shard, and a 2-chunk Ring pass (129/128 keys) with LSE merge."""
    c = synth.CONFIGS[1]
    B, S, H, D = c["B"], c["S"], c["H"], c["D"]
    qb, qv = _load(1, 0, (B, S, H, D), "fp32", False)
    kb, kv_ = _load(1, 1, (B, S, H, D), "fp32", False)
    vb, vv = _load(1, 2, (B, S, H, D), "fp32", False)
    scale = np.float32(1.0 / math.sqrt(D))
    q, k, v = dev(qb, "fp32"), dev(kb, "fp32"), dev(vb, "fp32")
    o, lse = _attn(q, k, v, float(scale))
    o_ref, l_ref = oracle.attention(qv, kv_, vv, scale)
    torch.cuda.synchronize()
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "fp32", "cfg1 full")
    parts = [_attn(q, k[:, a:b].contiguous(), v[:, a:b].contiguous(), float(scale)) for a, b in ((0, 129), (129, 257))]
    o_m = torch.empty_like(o)
    l_m = torch.empty_like(lse)
    uaa.usp_lse_merge([p[0] for p in parts], [p[1] for p in parts], o_m, l_m)
    torch.cuda.synchronize()
    check_pair(host_f64(o_m), host_f64(l_m), o_ref, l_ref, "fp32", "cfg1 ring")


@pytest.mark.parametrize("cfg", [2, 3])
def test_flux_shares_sampled_rows(cfg):
    """FLUX-shaped Ulysses shares: 12 of 24 heads over the full sequence."""
    c = synth.CONFIGS[cfg]
    B, S, H, D = c["B"], c["S"], c["H"], c["D"]
    Hr = H // 2
    say("attn cfg%d: generating inputs" % cfg)
    qb, qv = _load(cfg, 0, (B, S, H, D), "bf16", True)
    kb, kv_ = _load(cfg, 1, (B, S, H, D), "bf16", True)
    vb, vv = _load(cfg, 2, (B, S, H, D), "bf16", False)
    # rank 0's head shard: heads 0..11
    q, k, v = (dev(np.ascontiguousarray(x[:, :, :Hr]), "bf16") for x in (qb, kb, vb))
    scale = np.float32(1.0 / math.sqrt(D))
    say("attn cfg%d: launch" % cfg)
    o, lse = _attn(q, k, v, float(scale))
    torch.cuda.synchronize()
    rows = sample_rows(S, 192, seed=cfg)
    say("attn cfg%d: oracle on %d rows" % (cfg, len(rows)))
    o_ref, l_ref = oracle.attention(qv[:, :, :Hr], kv_[:, :, :Hr], vv[:, :, :Hr], scale, rows=rows)
    check_pair(host_f64(o[0, rows]), host_f64(lse[0, rows]), o_ref, l_ref, "bf16", "cfg%d" % cfg)


@pytest.mark.parametrize("split", [False, True], ids=["plain", "key_split"])
def test_qwen_ring_share_two_chunks_and_merge(split):
    """Qwen-Image Ring share: Q = tokens 0..3492, K/V in 2 chunks of 3493;
    with key_split each chunk's launch runs with a workspace (336 units on
    256 compute units: the last 80 are split)."""
    c = synth.CONFIGS[4]
    B, S, H, D = c["B"], c["S"], c["H"], c["D"]
    Sq = S // 2
    say("attn cfg4: generating inputs", "key split" if split else "plain")
    qb, qv = _load(4, 0, (B, S, H, D), "bf16", True)
    kb, kv_ = _load(4, 1, (B, S, H, D), "bf16", True)
    vb, vv = _load(4, 2, (B, S, H, D), "bf16", False)
    q = dev(np.ascontiguousarray(qb[:, :Sq]), "bf16")
    ks = [dev(np.ascontiguousarray(kb[:, a:a + Sq]), "bf16") for a in (0, Sq)]
    vs = [dev(np.ascontiguousarray(vb[:, a:a + Sq]), "bf16") for a in (0, Sq)]
    scale = float(np.float32(1.0 / math.sqrt(D)))
    if split:
        ws = uaa.attn_workspace(q, ks[0])
        assert ws is not None
        parts = []
        for n in range(2):
            o_n = torch.empty_like(q)
            l_n = torch.empty(q.shape[:3], device="cuda", dtype=torch.float32)
            uaa.usp_attn_fwd_lse(q, ks[n], vs[n], o_n, l_n, scale, workspace=ws)
            parts.append((o_n, l_n))
    else:
        parts = [_attn(q, ks[n], vs[n], scale) for n in range(2)]
    o = torch.empty_like(parts[0][0])
    lse = torch.empty_like(parts[0][1])
    uaa.usp_lse_merge([p[0] for p in parts], [p[1] for p in parts], o, lse)
    torch.cuda.synchronize()
    rows = sample_rows(Sq, 160, seed=4)
    say("attn cfg4: oracle on %d rows" % len(rows))
    o_ref, l_ref = oracle.attention(qv[:, :Sq], kv_, vv, np.float32(scale), rows=rows)
    check_pair(host_f64(o[0, rows]), host_f64(lse[0, rows]), o_ref, l_ref, "bf16", "cfg4 merged")
    # each partial too
    for n in range(2):
        o_p, l_p = oracle.attention(qv[:, :Sq], kv_[:, n * Sq:(n + 1) * Sq], vv[:, n * Sq:(n + 1) * Sq],
                                    np.float32(scale), rows=rows[:24])
        check_pair(host_f64(parts[n][0][0, rows[:24]]), host_f64(parts[n][1][0, rows[:24]]), o_p, l_p,
                   "bf16", "cfg4 partial %d" % n)


def test_long_context_zigzag_share():
    """Long-context causal share, zigzag layout: Q = global chunks {1, 6} of
    8 x 4096 tokens (rank 1 of a 4-rank zigzag ring), K/V iterated over all 8
    chunks with causal masking by global position, then an 8-way merge."""
    c = synth.CONFIGS[5]
    B, S, H, D = c["B"], c["S"], c["H"], c["D"]
    C = S // c["chunks"]
    say("attn cfg5: generating inputs")
    qb, qv = _load(5, 0, (B, S, H, D), "bf16", False)
    kb, kv_ = _load(5, 1, (B, S, H, D), "bf16", False)
    vb, vv = _load(5, 2, (B, S, H, D), "bf16", False)
    qpos = oracle.positions({"kind": "zigzag", "chunk": C, "ids": c["q_chunks"]}, 2 * C)
    q = dev(np.ascontiguousarray(qb[:, qpos]), "bf16")
    scale = float(np.float32(1.0 / math.sqrt(D)))
    parts = []
    for ch in range(c["chunks"]):
        kc = dev(np.ascontiguousarray(kb[:, ch * C:(ch + 1) * C]), "bf16")
        vc = dev(np.ascontiguousarray(vb[:, ch * C:(ch + 1) * C]), "bf16")
        m = uaa.mask_zigzag(C, c["q_chunks"], [ch])
        say("attn cfg5: chunk %d" % ch)
        parts.append(_attn(q, kc, vc, scale, m))
    torch.cuda.synchronize()
    # chunk 7 lies after every query position: exactly O = 0, LSE = -inf
    assert (parts[7][0].float() == 0).all() and torch.isneginf(parts[7][1]).all()
    o = torch.empty_like(parts[0][0])
    lse = torch.empty_like(parts[0][1])
    uaa.usp_lse_merge([p[0] for p in parts], [p[1] for p in parts], o, lse)
    torch.cuda.synchronize()
    rows = sample_rows(2 * C, 96, seed=5)
    say("attn cfg5: oracle on %d rows" % len(rows))
    pos = np.arange(S, dtype=np.int64)
    o_ref, l_ref = oracle.attention(qv[:, qpos], kv_, vv, np.float32(scale), qpos=qpos, kpos=pos, rows=rows)
    check_pair(host_f64(o[0, rows]), host_f64(lse[0, rows]), o_ref, l_ref, "bf16", "cfg5 merged")
