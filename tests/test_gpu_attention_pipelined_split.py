"""GPU parity of the pipelined attention kernel's key split (usp_attn_fwd_lse
with a workspace, bf16, D = 128, every key allowed) against the fp64 oracle.

A launch whose 256-row units run a partial last round, or fill at most
half the compute units, cuts the keys of some units into pieces run by
their own workgroups; the last piece of a unit to finish merges the pieces'
(O, LSE) -- the LSE merge of key blocks that Ring attention performs across
ranks (USP paper, the Ring attention section), done inside one launch.  The
library plans the split from measured costs of a piece; two plans are
covered:

  * whole rounds plus equal pieces of the last partial round's units (the
    Qwen-Image Ring chunk: 336 units of 55 key tiles on 256 compute units);
  * equal pieces of every unit, when units are few.

Shapes where no split pays (the FLUX.1 share's 216 units, 40 compute units
idle) keep the plain kernel with or without a workspace.

Each case checks the kernel the library reports, compares with the oracle
(every row at small sizes, sampled rows at full size), with the unsplit
call (LSE to fp32 rounding; O to the bf16 rounding of a piece's O, which
is kept in bf16 between the piece and the merge) and with a repeated call
on the same workspace (the merge runs in piece order, so the result is
bit for bit the same, and every call resets its arrival counters).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import sequence_attention_dits_amd as uaa
from gpu_common import check_pair, dev_bf16, host_f64, sample_rows, say

pytestmark = pytest.mark.gpu

D = 128


def _inputs(cfg, B, Sq, Sk, H):
    qb, qv = synth.tensor(cfg, 0, (B, Sq, H, D), "bf16", rms_norm=True)
    kb, kv = synth.tensor(cfg, 1, (B, Sk, H, D), "bf16", rms_norm=True)
    vb, vv = synth.tensor(cfg, 2, (B, Sk, H, D), "bf16")
    return (dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)), (qv, kv, vv)


def _run(q, k, v, scale, ws, odt, o=None, lse=None, acc=False):
    B, Sq, H, _ = q.shape
    if o is None:
        o = torch.full((B, Sq, H, D), float("nan"), device="cuda", dtype=odt)
        lse = torch.full((B, Sq, H), float("nan"), device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale, workspace=ws, accumulate=acc)
    return o, lse


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [
    # name, B, Sq, Sk, H, every row checked
    ("qwen_chunk_whole_plus_pieces", 1, 3493, 3493, 24, False),
    ("whole_plus_pieces_b2_ragged", 2, 2600, 1500, 12, False),
    ("equal_pieces_b2", 2, 1000, 777, 3, True),
    ("equal_pieces_ragged", 1, 700, 531, 5, True),
    ("whole_rounds_plus_pieces", 1, 4096, 600, 17, False),
]


@pytest.mark.parametrize("sk", [2304, 4608])
def test_flux_share_stays_plain(sk):
    """216 units (40 compute units idle): no workspace and no split."""
    q = torch.empty(1, 4608, 12, D, device="cuda", dtype=torch.bfloat16)
    k = torch.empty(1, sk, 12, D, device="cuda", dtype=torch.bfloat16)
    assert uaa.attn_workspace(q, k) is None
    assert uaa.usp_attn_kernel(q.shape, sk, workspace_bytes=1 << 30) == uaa.USP_KERNEL_PIPELINED


@pytest.mark.parametrize("out", ["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_against_oracle_and_unsplit(case, out):
    name, B, Sq, Sk, H, all_rows = case
    say("attn pipelined split", name, out)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    (q, k, v), (qv, kv, vv) = _inputs(1500 + CASES.index(case), B, Sq, Sk, H)
    ws = uaa.attn_workspace(q, k)
    assert ws is not None, "this shape is expected to split on a 256-CU device"
    assert uaa.usp_attn_kernel(q.shape, Sk, o_dtype=odt, workspace_bytes=ws.numel()) == \
        uaa.USP_KERNEL_PIPELINED_SPLIT
    assert uaa.usp_attn_kernel(q.shape, Sk, o_dtype=odt) == uaa.USP_KERNEL_PIPELINED
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(q, k, v, scale, ws, odt)
    o2, lse2 = _run(q, k, v, scale, ws, odt)   # same workspace, not re-zeroed
    o0, lse0 = _run(q, k, v, scale, None, odt)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(o2)) and torch.equal(lse, lse2), "repeated call differs"
    assert (lse - lse0).abs().max().item() < 1e-5
    assert (o.float() - o0.float()).abs().max().item() <= 4e-3
    if all_rows:
        o_ref, l_ref = oracle.attention(qv, kv, vv, np.float32(scale))
        check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", name)
    else:
        # flat tokens b * Sq + i of every batch
        rows = np.concatenate([b * Sq + sample_rows(Sq, 48, seed=1500 + CASES.index(case), tile=256)
                               for b in range(B)])
        o_ref, l_ref = oracle.attention(qv, kv, vv, np.float32(scale), rows=rows)
        check_pair(host_f64(o.reshape(B * Sq, H, D)[rows]), host_f64(lse.reshape(B * Sq, H)[rows]), o_ref, l_ref,
                   "bf16", name)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_qwen_ring_pass_with_split(out):
    """The Qwen-Image share's Ring pass: chunk 0 written, chunk 1 merged into
    it (accumulate), both split; equals attention over all 6986 keys."""
    B, Sq, C, H = 1, 3493, 3493, 24
    say("attn pipelined split ring pass", out)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    (q, k, v), (qv, kv, vv) = _inputs(1540, B, Sq, 2 * C, H)
    ks = [k[:, :C].contiguous(), k[:, C:].contiguous()]
    vs = [v[:, :C].contiguous(), v[:, C:].contiguous()]
    ws = uaa.attn_workspace(q, ks[0])
    assert ws is not None
    assert uaa.usp_attn_kernel(q.shape, C, o_dtype=odt, workspace_bytes=ws.numel()) == \
        uaa.USP_KERNEL_PIPELINED_SPLIT
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(q, ks[0], vs[0], scale, ws, odt)
    _run(q, ks[1], vs[1], scale, ws, odt, o, lse, acc=True)
    o0, lse0 = _run(q, ks[0], vs[0], scale, None, odt)
    _run(q, ks[1], vs[1], scale, None, odt, o0, lse0, acc=True)
    torch.cuda.synchronize()
    assert (lse - lse0).abs().max().item() < 1e-5
    assert (o.float() - o0.float()).abs().max().item() <= 4e-3
    rows = sample_rows(Sq, 48, seed=1540, tile=256)
    o_ref, l_ref = oracle.attention(qv, kv, vv, np.float32(scale), rows=rows)
    check_pair(host_f64(o[0, rows]), host_f64(lse[0, rows]), o_ref, l_ref, "bf16", "qwen ring pass " + out)


def test_accumulate_from_empty_rows_with_split():
    """Accumulating into (0, -inf) rows equals the plain split call: the
    merge's weights give the new block everything."""
    B, Sq, Sk, H = 2, 1000, 777, 3
    say("attn pipelined split: accumulate from empty")
    (q, k, v), _ = _inputs(1541, B, Sq, Sk, H)
    ws = uaa.attn_workspace(q, k)
    scale = 1.0 / math.sqrt(D)
    o = torch.zeros(B, Sq, H, D, device="cuda", dtype=torch.bfloat16)
    lse = torch.full((B, Sq, H), float("-inf"), device="cuda", dtype=torch.float32)
    _run(q, k, v, scale, ws, torch.bfloat16, o, lse, acc=True)
    o1, lse1 = _run(q, k, v, scale, ws, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse1)
    assert torch.equal(_bits(o), _bits(o1))


def test_split_under_graph_replay():
    """The split launch captured in a HIP graph (its counters are reset by
    the kernel itself) and replayed with eager work between the replays:
    every replay equals the eager call."""
    B, Sq, Sk, H = 1, 3493, 3493, 24
    say("attn pipelined split: graph replays")
    (q, k, v), _ = _inputs(1542, B, Sq, Sk, H)
    ws = uaa.attn_workspace(q, k)
    scale = 1.0 / math.sqrt(D)
    o_e, l_e = _run(q, k, v, scale, ws, torch.bfloat16)
    torch.cuda.synchronize()
    o = torch.empty_like(o_e)
    lse = torch.empty_like(l_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        _run(q, k, v, scale, None, torch.bfloat16)   # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(_bits(o), _bits(o_e)) and torch.equal(lse, l_e)
