"""The hot path captured as a HIP graph (how a serving loop or the bench
runs it) must give the eager result on every replay, with eager work and
synchronisations between replays."""

import math

import numpy as np
import pytest
import torch

import sequence_attention_dits_amd as uaa
from gpu_common import say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_step():
    torch.manual_seed(0)
    B, S, H, D = 1, 700, 4, 128
    seq_off, head_off = [0, 351, 700], [0, 2, 4]
    shards = {n: [torch.randn(B, b - a, H, D, device="cuda").to(torch.bfloat16)
                  for a, b in ((0, 351), (351, 700))] for n in "qkv"}
    qh = {n: torch.empty(B, S, 2, D, device="cuda", dtype=torch.bfloat16) for n in "qkv"}
    o_p = [torch.empty(B, S, 2, D, device="cuda", dtype=torch.bfloat16) for _ in range(2)]
    l_p = [torch.empty(B, S, 2, device="cuda") for _ in range(2)]
    o = torch.empty(B, S, 2, D, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B, S, 2, device="cuda")
    other = torch.randn(B, S, 2, D, device="cuda").to(torch.bfloat16)
    o_tok = torch.empty(B, 351, H, D, device="cuda", dtype=torch.bfloat16)
    scale = 1.0 / math.sqrt(D)

    def step():
        for n in "qkv":
            uaa.uaa_seq2head_permute(uaa.UAA_SEQ2HEAD, 0, shards[n], qh[n], seq_off, head_off)
        for c, (a, b) in enumerate(((0, 300), (300, 700))):
            uaa.usp_attn_fwd_lse(qh["q"], qh["k"][:, a:b], qh["v"][:, a:b], o_p[c], l_p[c], scale,
                                 uaa.mask_causal(0, a))
        uaa.usp_lse_merge(o_p, l_p, o, lse)
        uaa.uaa_seq2head_permute(uaa.UAA_HEAD2SEQ, 0, [o, other], o_tok, seq_off, head_off)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l, ref_t = o.clone(), lse.clone(), o_tok.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        say("graph replay", r)
        # clobber the outputs eagerly between replays
        o.zero_()
        lse.fill_(7.0)
        o_tok.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(lse, ref_l)
        assert torch.equal(o_tok.view(torch.int16), ref_t.view(torch.int16))
    assert np.isfinite(ref_l.cpu().numpy()).all()
