"""Parity of the Ring-step attention (usp_attn_fwd_lse_acc): a key/value
block's attention merged in place into the running (O, LSE) of the blocks
seen before -- the per-step update of a Ring pass (USP pull request, the
Ring attention loop; "Context parallelism", Ring Attention).  Two blocks
processed as (plain, accumulate) must equal the oracle's attention over the
concatenated keys; the accumulate call started from LSE = -inf must equal
the plain call bit for bit; rows with no allowed key in a block never read
that block's (possibly garbage) O."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import sequence_attention_dits_amd as uaa
from gpu_common import check_pair, dev, host_f64, sample_rows, say

pytestmark = pytest.mark.gpu


def _inputs(cfg, B, Sq, Sk, H, D, dtype):
    qb, qv = synth.tensor(cfg, 0, (B, Sq, H, D), dtype, rms_norm=True)
    kb, kv_ = synth.tensor(cfg, 1, (B, Sk, H, D), dtype, rms_norm=True)
    vb, vv = synth.tensor(cfg, 2, (B, Sk, H, D), dtype)
    return (dev(qb, dtype), dev(kb, dtype), dev(vb, dtype)), (qv, kv_, vv)


def _ring_two_blocks(q, k, v, split, scale, odt, masks=(None, None), ws=None, garbage=True):
    """Block 0 = keys [0, split), block 1 = keys [split, Sk): plain call, then
    the accumulate call, into one (o, lse)."""
    B, Sq, H, D = q.shape
    o = torch.full((B, Sq, H, D), float("nan") if garbage else 0.0, device="cuda", dtype=odt)
    lse = torch.full((B, Sq, H), float("nan"), device="cuda", dtype=torch.float32)
    k0, v0 = k[:, :split].contiguous(), v[:, :split].contiguous()
    k1, v1 = k[:, split:].contiguous(), v[:, split:].contiguous()
    uaa.usp_attn_fwd_lse(q, k0, v0, o, lse, scale, masks[0], workspace=ws)
    uaa.usp_attn_fwd_lse(q, k1, v1, o, lse, scale, masks[1], workspace=ws, accumulate=True)
    return o, lse


CASES = [
    # (name, B, Sq, Sk, split, H, D, dtype, out)
    ("bf16_d128", 1, 300, 329, 129, 2, 128, "bf16", "bf16"),
    ("bf16_d128_fp32out", 1, 300, 329, 129, 2, 128, "bf16", "fp32"),
    ("bf16_d64_ragged", 2, 257, 190, 64, 3, 64, "bf16", "bf16"),
    ("fp32_d128", 1, 130, 150, 70, 2, 128, "fp32", "fp32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_two_blocks_equal_attention_over_all_keys(case):
    name, B, Sq, Sk, split, H, D, dtype, out = case
    say("attn acc", name)
    (q, k, v), (qv, kv_, vv) = _inputs(970 + CASES.index(case), B, Sq, Sk, H, D, dtype)
    scale = 1.0 / math.sqrt(D)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    o, lse = _ring_two_blocks(q, k, v, split, scale, odt)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qv, kv_, vv, np.float32(scale))
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16" if "bf16" in (dtype, out) else "fp32", name)


def test_accumulate_matches_attention_then_merge():
    B, Sq, Sk, split, H, D = 1, 300, 329, 129, 2, 128
    (q, k, v), _ = _inputs(975, B, Sq, Sk, H, D, "bf16")
    scale = 1.0 / math.sqrt(D)
    o, lse = _ring_two_blocks(q, k, v, split, scale, torch.bfloat16)
    parts = []
    for a, b in ((0, split), (split, Sk)):
        op = torch.empty_like(q)
        lp = torch.empty(B, Sq, H, device="cuda")
        uaa.usp_attn_fwd_lse(q, k[:, a:b].contiguous(), v[:, a:b].contiguous(), op, lp, scale)
        parts.append((op, lp))
    om = torch.empty_like(q)
    lm = torch.empty(B, Sq, H, device="cuda")
    uaa.usp_lse_merge([p[0] for p in parts], [p[1] for p in parts], om, lm)
    torch.cuda.synchronize()
    # same inputs and roundings; the weights are taken in base 2 here and in
    # base e by the merge: a few bf16 ulps at most
    assert (o.float() - om.float()).abs().max().item() <= 4e-3
    assert (lse - lm).abs().max().item() <= 1e-5


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_accumulate_from_empty_equals_plain_call(out):
    B, Sq, Sk, H, D = 1, 200, 190, 2, 128
    (q, k, v), _ = _inputs(976, B, Sq, Sk, H, D, "bf16")
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    o0 = torch.empty(B, Sq, H, D, device="cuda", dtype=odt)
    l0 = torch.empty(B, Sq, H, device="cuda")
    uaa.usp_attn_fwd_lse(q, k, v, o0, l0, 0.09)
    o1 = torch.full((B, Sq, H, D), float("nan"), device="cuda", dtype=odt)   # never read: lse = -inf
    l1 = torch.full((B, Sq, H), float("-inf"), device="cuda")
    uaa.usp_attn_fwd_lse(q, k, v, o1, l1, 0.09, accumulate=True)
    torch.cuda.synchronize()
    iv = torch.int16 if out == "bf16" else torch.int32
    assert torch.equal(o0.view(iv), o1.view(iv)) and torch.equal(l0, l1)


def test_causal_blocks_with_empty_rows():
    """Causal by global position, Q = tokens 100..299, K/V = tokens 0..379 in
    two blocks (0..189, 190..379): early rows see nothing of block 1, and
    rows before 190 see block 0 only partly; rows with no key in a block keep
    (and never read) a NaN O."""
    B, Sq, Sk, split, H, D = 1, 200, 380, 190, 2, 128
    (q, k, v), (qv, kv_, vv) = _inputs(977, B, Sq, Sk, H, D, "bf16")
    scale = 1.0 / math.sqrt(D)
    masks = (uaa.mask_causal(100, 0), uaa.mask_causal(100, split))
    o, lse = _ring_two_blocks(q, k, v, split, scale, torch.bfloat16, masks)
    torch.cuda.synchronize()
    qpos = oracle.positions({"kind": "causal", "off": 100}, Sq)
    kpos = oracle.positions({"kind": "causal", "off": 0}, Sk)
    o_ref, l_ref = oracle.attention(qv, kv_, vv, np.float32(scale), qpos=qpos, kpos=kpos)
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "causal acc")


def test_accumulate_with_key_split():
    """272 units on 256 compute units (the last 16 split) for both blocks."""
    B, Sq, Sk, split, H, D = 1, 4096, 1200, 600, 17, 128
    say("attn acc: key split")
    (q, k, v), (qv, kv_, vv) = _inputs(978, B, Sq, Sk, H, D, "bf16")
    ws = uaa.attn_workspace(q, k[:, :split])
    assert ws is not None
    scale = 1.0 / math.sqrt(D)
    o, lse = _ring_two_blocks(q, k, v, split, scale, torch.bfloat16, ws=ws)
    torch.cuda.synchronize()
    rows = sample_rows(Sq, 96, seed=978)
    o_ref, l_ref = oracle.attention(qv, kv_, vv, np.float32(scale), rows=rows)
    check_pair(host_f64(o[0, rows]), host_f64(lse[0, rows]), o_ref, l_ref, "bf16", "acc + split")
