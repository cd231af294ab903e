"""GPU parity of the pipelined attention kernel's DIAG form against the fp64
oracle, every row: masked calls whose key positions form one increasing
piece (a basic ring block, a stripe block, a zigzag block of one chunk), so
that every query row may see a prefix of the keys and the 256-row units on
the mask's diagonal run only their live key tiles, masked row by row.

The USP / yunchang summary ("How It Works", "Highlighted Details") names the
zigzag layout as the load balance of causal Ring attention; the rank's own
chunks are where its units sit on the diagonal.  Shapes: square and ragged
causal blocks, rows with no allowed key, zigzag chunks of 768 (three units:
on the diagonal, seeing all, seeing none) and of 700 (units straddling the
two query chunks), a stripe block, a whole zigzag Ring pass over 8 chunks
with the Ring-step update, bf16 and fp32 output.  Each case also checks that
the library picked the DIAG form.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import sequence_attention_dits_amd as uaa
from gpu_common import check_pair, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _zz(C, ids, n):
    return np.concatenate([c * C + np.arange(C) for c in ids])[:n]


CASES = [
    # name, B, Sq, Sk, H, mask, qpos, kpos
    ("causal_square_768", 1, 768, 768, 2, lambda: uaa.mask_causal(0, 0), np.arange(768), np.arange(768)),
    ("causal_ragged_700_b2", 2, 700, 700, 3, lambda: uaa.mask_causal(0, 0), np.arange(700), np.arange(700)),
    ("causal_rows_without_keys", 1, 600, 768, 2, lambda: uaa.mask_causal(0, 100), np.arange(600),
     100 + np.arange(768)),
    ("causal_rows_after_block_start", 1, 1000, 384, 1, lambda: uaa.mask_causal(300, 0), 300 + np.arange(1000),
     np.arange(384)),
    ("zigzag_768_k1", 1, 1536, 768, 2, lambda: uaa.mask_zigzag(768, [1, 6], [1]), _zz(768, [1, 6], 1536),
     _zz(768, [1], 768)),
    ("zigzag_768_k6", 1, 1536, 768, 2, lambda: uaa.mask_zigzag(768, [1, 6], [6]), _zz(768, [1, 6], 1536),
     _zz(768, [6], 768)),
    ("zigzag_700_k6", 1, 1400, 700, 1, lambda: uaa.mask_zigzag(700, [1, 6], [6]), _zz(700, [1, 6], 1400),
     _zz(700, [6], 700)),
    ("stripe_w4", 1, 700, 700, 2, lambda: uaa.mask_stripe(4, 1, 2), 1 + 4 * np.arange(700), 2 + 4 * np.arange(700)),
]


def _inputs(cfg, B, Sq, Sk, H, D=128):
    qb, qv = synth.tensor(cfg, 0, (B, Sq, H, D), "bf16", rms_norm=True)
    kb, kv = synth.tensor(cfg, 1, (B, Sk, H, D), "bf16", rms_norm=True)
    vb, vv = synth.tensor(cfg, 2, (B, Sk, H, D), "bf16")
    return (qb, qv), (kb, kv), (vb, vv)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_diag_all_rows(case, out):
    name, B, Sq, Sk, H, mk, qpos, kpos = case
    say("attn pipelined diag", name, out)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    assert uaa.usp_attn_kernel((B, Sq, H, 128), Sk, o_dtype=odt, mask=mk()) == uaa.USP_KERNEL_PIPELINED_DIAG
    (qb, qv), (kb, kv), (vb, vv) = _inputs(1400 + CASES.index(case), B, Sq, Sk, H)
    scale = 1.0 / math.sqrt(128)
    o = torch.full((B, Sq, H, 128), 3.0, device="cuda", dtype=odt)
    lse = torch.full((B, Sq, H), 3.0, device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), o, lse, scale, mk())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qv, kv, vv, np.float32(scale), qpos=qpos, kpos=kpos)
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", name)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_zigzag_ring_pass_over_every_chunk(out):
    """Rank 1 of a 4-rank zigzag ring (chunks {1, 6} of 8 chunks of 768): its
    queries against every K/V chunk in turn, the first call plain and the
    rest merged in place -- chunk 0 unmasked, chunks 1 and 6 on the
    diagonal, the rest all-or-nothing, chunk 7 in every row's future -- must
    equal causal attention by global position over the whole sequence."""
    C, H, R = 768, 2, 4
    say("attn zigzag ring pass", out)
    S = 2 * R * C
    (qb_all, qv_all), (kb, kv), (vb, vv) = _inputs(1450, 1, S, S, H)
    rows = _zz(C, [1, 6], 2 * C)
    q = dev_bf16(np.ascontiguousarray(qb_all[:, rows]))
    k, v = dev_bf16(kb), dev_bf16(vb)
    scale = 1.0 / math.sqrt(128)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    o = torch.empty(1, 2 * C, H, 128, device="cuda", dtype=odt)
    lse = torch.empty(1, 2 * C, H, device="cuda", dtype=torch.float32)
    kinds = []
    for c in range(2 * R):
        m = uaa.mask_zigzag(C, [1, 6], [c])
        kinds.append(uaa.usp_attn_kernel((1, 2 * C, H, 128), C, o_dtype=odt, mask=m))
        uaa.usp_attn_fwd_lse(q, k[:, c * C:(c + 1) * C].contiguous(), v[:, c * C:(c + 1) * C].contiguous(), o, lse,
                             scale, m, accumulate=c > 0)
    torch.cuda.synchronize()
    assert kinds[1] == kinds[6] == uaa.USP_KERNEL_PIPELINED_DIAG
    assert all(k_ == uaa.USP_KERNEL_PIPELINED for i, k_ in enumerate(kinds) if i not in (1, 6))
    o_ref, l_ref = oracle.attention(qv_all[:, rows], kv, vv, np.float32(scale), qpos=rows, kpos=np.arange(S))
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "zigzag ring pass " + out)
