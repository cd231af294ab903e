"""Parity of the key-split attention (usp_attn_fwd_lse with a workspace).

When the (batch, head, 256-row) units of a problem do not fill the last
round of workgroups, the bf16 kernel cuts the keys of the units of that
round into pieces and combines the pieces' partial results -- the
online-softmax merge of key blocks that Ring attention performs across
ranks (USP paper, the Ring attention section), done inside one launch.  With
D = 64 the general kernel runs the pieces (partial states merged in fp32);
with D = 128 the pipelined kernel does (each piece's normalised O kept in
bf16 with its LSE).  The result is compared with the fp64 oracle under the
bf16 tolerance, with the plain call, and with itself on a repeated call (the
combine runs in piece order, so it is deterministic; the arrival counters
are reset by every call, which the repeated call also checks)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import sequence_attention_dits_amd as uaa
from gpu_common import check_pair, dev, host_f64, sample_rows, say

pytestmark = pytest.mark.gpu


def _run(q, k, v, scale, ws, out_dtype, mask=None):
    B, Sq, H, D = q.shape
    o = torch.full((B, Sq, H, D), float("nan"), device="cuda", dtype=out_dtype)
    lse = torch.full((B, Sq, H), float("nan"), device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale, mask, workspace=ws)
    return o, lse


def _inputs(cfg, B, Sq, Sk, H, D):
    qb, qv = synth.tensor(cfg, 0, (B, Sq, H, D), "bf16", rms_norm=True)
    kb, kv_ = synth.tensor(cfg, 1, (B, Sk, H, D), "bf16", rms_norm=True)
    vb, vv = synth.tensor(cfg, 2, (B, Sk, H, D), "bf16")
    return (dev(qb, "bf16"), dev(kb, "bf16"), dev(vb, "bf16")), (qv, kv_, vv)


SPLIT = [
    # (name, B, Sq, Sk, H, D): every unit split (fewer units than compute units)
    ("all_split_d128", 2, 1000, 777, 3, 128),
    ("all_split_d64", 2, 1000, 777, 3, 64),
    ("all_split_ragged", 1, 700, 531, 5, 128),
]


@pytest.mark.parametrize("out", ["bf16", "fp32"])
@pytest.mark.parametrize("case", SPLIT, ids=[c[0] for c in SPLIT])
def test_split_all_rows(case, out):
    name, B, Sq, Sk, H, D = case
    say("attn split", name, out)
    (q, k, v), (qv, kv_, vv) = _inputs(950 + SPLIT.index(case), B, Sq, Sk, H, D)
    ws = uaa.attn_workspace(q, k)
    assert ws is not None, "this shape is expected to split on a 256-CU device"
    scale = 1.0 / math.sqrt(D)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    assert uaa.usp_attn_kernel(q.shape, Sk, o_dtype=odt, workspace_bytes=ws.numel()) == \
        (uaa.USP_KERNEL_PIPELINED_SPLIT if D == 128 else uaa.USP_KERNEL_GENERAL_SPLIT)
    o, lse = _run(q, k, v, scale, ws, odt)
    o2, lse2 = _run(q, k, v, scale, ws, odt)   # same workspace, not re-zeroed
    o0, lse0 = _run(q, k, v, scale, None, odt)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qv, kv_, vv, np.float32(scale))
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", name)
    assert torch.equal(o.view(torch.int16) if out == "bf16" else o.view(torch.int32),
                       o2.view(torch.int16) if out == "bf16" else o2.view(torch.int32)), "repeat differs"
    assert torch.equal(lse, lse2)
    # Against the unsplit call: the LSE differs by fp32 rounding; O also by
    # the bf16 rounding of the probabilities, which each piece takes
    # relative to its own running maximum (a few 1e-4 here).
    assert (lse - lse0).abs().max().item() < 1e-5
    assert (o.float() - o0.float()).abs().max().item() <= 4e-3


def test_whole_units_and_split_units():
    """272 units on 256 compute units: 256 run whole, the last 16 (head 16)
    are split; sampled rows cover every head."""
    B, Sq, Sk, H, D = 1, 4096, 600, 17, 128
    say("attn split: whole + split units")
    (q, k, v), (qv, kv_, vv) = _inputs(960, B, Sq, Sk, H, D)
    ws = uaa.attn_workspace(q, k)
    assert ws is not None
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(q, k, v, scale, ws, torch.bfloat16)
    torch.cuda.synchronize()
    rows = sample_rows(Sq, 96, seed=960)
    o_ref, l_ref = oracle.attention(qv, kv_, vv, np.float32(scale), rows=rows)
    check_pair(host_f64(o[0, rows]), host_f64(lse[0, rows]), o_ref, l_ref, "bf16", "whole+split")


def test_small_workspace_and_masks_use_the_plain_path():
    B, Sq, Sk, H, D = 2, 1000, 777, 3, 128
    (q, k, v), (qv, kv_, vv) = _inputs(951, B, Sq, Sk, H, D)
    ws = uaa.attn_workspace(q, k)
    assert ws is not None
    scale = 1.0 / math.sqrt(D)
    o0, l0 = _run(q, k, v, scale, None, torch.bfloat16)
    o1, l1 = _run(q, k, v, scale, ws[: ws.numel() - 256], torch.bfloat16)   # one piece short
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)
    # a causal mask never splits: same bits as the plain masked call
    m = uaa.mask_causal(0, 0)
    assert uaa.attn_workspace(q, k, m) is None
    o2, l2 = _run(q, k, v, scale, None, torch.bfloat16, m)
    o3, l3 = _run(q, k, v, scale, ws, torch.bfloat16, m)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o3.view(torch.int16)) and torch.equal(l2, l3)


def test_misaligned_workspace_is_rejected():
    q = torch.zeros(1, 300, 2, 128, device="cuda", dtype=torch.bfloat16)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 300, 2, device="cuda")
    with pytest.raises(uaa.UaaError) as e:
        uaa.usp_attn_fwd_lse(q, q, q, o, lse, 0.1, workspace=ws[16:])
    assert e.value.status == uaa.UAA_ERR_INVALID_ARG
