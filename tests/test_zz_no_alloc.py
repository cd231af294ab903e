"""usp_attn_fwd_lse_static, the attention entry point that allocates
nothing (its key-split workspace is a device array inside the library),
against usp_attn_fwd_lse_ws given a workspace of its own: bit for bit.

Two calls in a row on the library's one scratch array, the second with a
smaller input (whose plan uses fewer pieces and puts its arrival counters
elsewhere in the array), then a shape that runs without a split, then the
small call captured in a HIP graph and replayed with eager work between the
replays.  The first two shapes are ones whose keys the library splits (the
Qwen-Image Ring chunk: 336 units on 256 compute units).
"""

import math

import numpy as np
import pytest
import torch

import synth
import sequence_attention_dits_amd as uaa
from gpu_common import dev_bf16, say

pytestmark = pytest.mark.gpu

SHAPES = [
    # name, B, Sq, Sk, H: the first two split their keys, the third does not
    ("qwen_chunk", 1, 3493, 3493, 24),
    ("smaller_split", 1, 2600, 1024, 24),
    ("one_full_round_unsplit", 1, 4096, 2048, 16),   # 256 units: one full round, no split
]


def _inputs(i, B, Sq, Sk, H, D=128):
    q = dev_bf16(synth.tensor(1300 + i, 0, (B, Sq, H, D), "bf16", rms_norm=True)[0])
    k = dev_bf16(synth.tensor(1300 + i, 1, (B, Sk, H, D), "bf16", rms_norm=True)[0])
    v = dev_bf16(synth.tensor(1300 + i, 2, (B, Sk, H, D), "bf16")[0])
    return q, k, v


def _with_workspace(q, k, v, scale):
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device="cuda", dtype=torch.float32)
    ws = uaa.attn_workspace(q, k)
    uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale, workspace=ws)
    return o, lse, ws


def _static(q, k, v, scale):
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse_static(q, k, v, o, lse, scale)
    return o, lse


def _same(a, b):
    return torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_static_scratch_equals_caller_workspace():
    scale = 1.0 / math.sqrt(128)
    results = []
    for i, (name, B, Sq, Sk, H) in enumerate(SHAPES):
        say("attn static scratch", name)
        q, k, v = _inputs(i, B, Sq, Sk, H)
        ref_o, ref_l, ws = _with_workspace(q, k, v, scale)
        assert (ws is not None) == (i < 2), name   # the first two shapes split their keys
        got = _static(q, k, v, scale)
        torch.cuda.synchronize()
        assert _same(got, (ref_o, ref_l)), name
        assert not torch.isnan(got[1]).any()
        results.append((q, k, v, ref_o, ref_l))
    # the big shape again after the smaller one: the array keeps the last
    # call's contents, and the call must not depend on them
    q, k, v, ref_o, ref_l = results[0]
    say("attn static scratch", "qwen_chunk again")
    got = _static(q, k, v, scale)
    torch.cuda.synchronize()
    assert _same(got, (ref_o, ref_l))


def test_static_scratch_under_graph_capture():
    scale = 1.0 / math.sqrt(128)
    name, B, Sq, Sk, H = SHAPES[1]
    say("attn static scratch graph", name)
    q, k, v = _inputs(1, B, Sq, Sk, H)
    ref_o, ref_l, _ = _with_workspace(q, k, v, scale)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device="cuda", dtype=torch.float32)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        uaa.usp_attn_fwd_lse_static(q, k, v, o, lse, scale)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        uaa.usp_attn_fwd_lse_static(q, k, v, o, lse, scale)
    torch.cuda.synchronize()
    big = _inputs(0, *SHAPES[0][1:])
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        if rep == 1:   # eager work between the replays that also uses the scratch array
            _static(*big, scale)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same((o, lse), (ref_o, ref_l)), "replay %d" % rep
