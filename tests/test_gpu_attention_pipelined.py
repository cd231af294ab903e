"""GPU parity of the software-pipelined attention kernel (unmasked, D = 128,
bf16 inputs, no key split) against the fp64 oracle, every row.

The kernel's loop body is six tile steps (two score parities x three LDS
stages) with an exit after each, so the key-tile counts here (64 keys a
tile) end the loop at every one of the six positions and after one and
two whole bodies: 1, 2, 3, 4, 5, 6, 7, 11, 12 and 13 tiles, with and without
a ragged last tile, ragged query rows (a partial last 256-row workgroup and
waves past the end), several heads and batches, bf16 and fp32 output, a
two-block Ring pass accumulated in place, and scores large enough to make
the running maximum rise mid-row (the rescale path).
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

CASES = [
    # name, B, Sq, Sk, H
    ("tiles1_tail", 1, 200, 50, 2),
    ("tiles2", 1, 300, 128, 1),
    ("tiles3_tail", 2, 260, 150, 2),
    ("tiles4", 1, 256, 256, 1),
    ("tiles5_tail", 1, 513, 300, 1),
    ("tiles6_exact", 1, 256, 384, 2),
    ("tiles6_ragged_keys_rows", 2, 300, 367, 3),
    ("tiles7_tail", 1, 300, 420, 1),
    ("tiles11", 1, 513, 700, 1),
    ("tiles12_tail63", 1, 100, 767, 2),
    ("tiles13", 1, 256, 832, 1),
]


def _inputs(cfg, B, Sq, Sk, H, D=128):
    qb, qv = synth.tensor(cfg, 0, (B, Sq, H, D), "bf16", rms_norm=True)
    kb, kv = synth.tensor(cfg, 1, (B, Sk, H, D), "bf16", rms_norm=True)
    vb, vv = synth.tensor(cfg, 2, (B, Sk, H, D), "bf16")
    return (qb, qv), (kb, kv), (vb, vv)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pipelined_all_rows(case, out):
    name, B, Sq, Sk, H = case
    say("attn pipelined", name, out)
    assert uaa.usp_attn_kernel((B, Sq, H, 128), Sk) == uaa.USP_KERNEL_PIPELINED
    (qb, qv), (kb, kv), (vb, vv) = _inputs(1100 + CASES.index(case), B, Sq, Sk, H)
    scale = 1.0 / math.sqrt(128)
    o = torch.empty(B, Sq, H, 128, device="cuda", dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    lse = torch.empty(B, Sq, H, device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), o, lse, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qv, kv, vv, np.float32(scale))
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", name)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_pipelined_ring_pass_accumulates(out):
    # two key blocks of 384 and 367 keys (6 tiles each), the second merged
    # into the first's (O, LSE) in place: equals attention over all keys
    B, Sq, H = 1, 300, 2
    say("attn pipelined ring pass", out)
    (qb, qv), (kb, kv), (vb, vv) = _inputs(1150, B, Sq, 751, H)
    scale = 1.0 / math.sqrt(128)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    assert uaa.usp_attn_kernel((B, Sq, H, 128), 384) == uaa.USP_KERNEL_PIPELINED
    assert uaa.usp_attn_kernel((B, Sq, H, 128), 367) == uaa.USP_KERNEL_PIPELINED
    o = torch.empty(B, Sq, H, 128, device="cuda", dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    lse = torch.empty(B, Sq, H, device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(q, k[:, :384].contiguous(), v[:, :384].contiguous(), o, lse, scale)
    uaa.usp_attn_fwd_lse(q, k[:, 384:].contiguous(), v[:, 384:].contiguous(), o, lse, scale, accumulate=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qv, kv, vv, np.float32(scale))
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "ring pass " + out)


def test_pipelined_rising_maximum():
    # large queries and a key block whose scores grow along the keys, so the
    # running maximum of a row rises by far more than the lazy-rescale
    # threshold several times along the row
    B, Sq, Sk, H = 1, 256, 384, 1
    say("attn pipelined rising maximum")
    rng = np.random.default_rng(11)
    q = 2.0 * rng.standard_normal((B, Sq, H, 128))
    k = 2.0 * rng.standard_normal((B, Sk, H, 128)) * np.linspace(0.2, 3.0, Sk)[None, :, None, None]
    v = rng.standard_normal((B, Sk, H, 128))
    bits = [synth.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v)]
    q, k, v = (synth.bf16_bits_to_f32(b) for b in bits)
    scale = 1.0 / math.sqrt(128)
    # the maximum of a row over all keys exceeds its maximum over the first
    # tile by far more than the lazy-rescale threshold (8 in log2 units)
    s = np.einsum("qd,kd->qk", q[0, :, 0].astype(np.float64), k[0, :, 0].astype(np.float64)) * scale / math.log(2)
    assert np.median(s.max(axis=1) - s[:, :64].max(axis=1)) > 16.0
    assert uaa.usp_attn_kernel((B, Sq, H, 128), Sk) == uaa.USP_KERNEL_PIPELINED
    o = torch.empty(B, Sq, H, 128, device="cuda", dtype=torch.float32)
    lse = torch.empty(B, Sq, H, device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(dev_bf16(bits[0]), dev_bf16(bits[1]), dev_bf16(bits[2]), o, lse, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, np.float32(scale))
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "rising maximum")


# A masked call whose keys all precede (or equal) every query in position
# allows every pair and runs as an unmasked call: bit-identical output.  With
# one key past the first query (or a plain causal block) the mask stays.
ALL_ALLOWED = [
    # name, mask builder, qpos, kpos (Sq = 300, Sk = 384), every pair allowed
    ("causal_past_block", lambda: uaa.mask_causal(1000, 616), 1000 + np.arange(300), 616 + np.arange(384), True),
    ("zigzag_past_chunks", lambda: uaa.mask_zigzag(192, [2, 5], [0, 1]),
     np.concatenate([2 * 192 + np.arange(192), 5 * 192 + np.arange(108)]), np.arange(384), True),
    ("causal_one_pair_out", lambda: uaa.mask_causal(1000, 618), 1000 + np.arange(300), 618 + np.arange(384), False),
    ("stripe_world1_causal", lambda: uaa.mask_stripe(1, 0, 0), np.arange(300), np.arange(384), False),
]


@pytest.mark.parametrize("case", ALL_ALLOWED, ids=[c[0] for c in ALL_ALLOWED])
def test_mask_allowing_every_pair_runs_unmasked(case):
    name, mk, qpos, kpos, every = case
    assert every == bool(kpos.max() <= qpos.min())
    say("attn every pair allowed", name)
    B, Sq, Sk, H = 1, 300, 384, 2
    (qb, qv), (kb, kv), (vb, vv) = _inputs(1170, B, Sq, Sk, H)
    scale = 1.0 / math.sqrt(128)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o = torch.empty(B, Sq, H, 128, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B, Sq, H, device="cuda", dtype=torch.float32)
    o_u, lse_u = torch.empty_like(o), torch.empty_like(lse)
    uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale, mask=mk())
    uaa.usp_attn_fwd_lse(q, k, v, o_u, lse_u, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qv, kv, vv, np.float32(scale), qpos=qpos, kpos=kpos)
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", name)
    assert (torch.equal(o, o_u) and torch.equal(lse, lse_u)) == every, name


def _zigzag_pos(C, ids, n):
    return np.concatenate([c * C + np.arange(C) for c in ids])[:n]


# Masked calls in which every 256-row unit sees every key of the block or
# none: zigzag chunks of 768 rows (three units each), K chunk 2 in the future
# of Q chunk 1 and in the past of Q chunk 4.  Units that see nothing give
# (0, -inf); a Ring pass continued over such a block keeps its rows.
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_units_all_or_nothing(out):
    C, H = 768, 2
    say("attn units all or nothing", out)
    (qb, qv), (kb, kv), (vb, vv) = _inputs(1180, 1, 2 * C, 2 * C, H)
    scale = 1.0 / math.sqrt(128)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    qpos = _zigzag_pos(C, [1, 4], 2 * C)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    o = torch.full((1, 2 * C, H, 128), 7.0, device="cuda", dtype=dt)
    lse = torch.full((1, 2 * C, H), 7.0, device="cuda", dtype=torch.float32)
    for kc in ([2], [0]):
        assert uaa.usp_attn_kernel((1, 2 * C, H, 128), C, mask=uaa.mask_zigzag(C, [1, 4], kc)) == \
            uaa.USP_KERNEL_PIPELINED
    # K chunk 2 alone: rows of Q chunk 1 see nothing, rows of Q chunk 4 all
    uaa.usp_attn_fwd_lse(q, k[:, :C].contiguous(), v[:, :C].contiguous(), o, lse, scale,
                         mask=uaa.mask_zigzag(C, [1, 4], [2]))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qv, kv[:, :C], vv[:, :C], np.float32(scale), qpos=qpos,
                                    kpos=_zigzag_pos(C, [2], C))
    assert np.isneginf(l_ref[0, :C]).all() and np.isfinite(l_ref[0, C:]).all()
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "chunk 2 " + out)
    # a Ring pass: K chunk 0 (every pair allowed), then K chunk 2 merged in
    uaa.usp_attn_fwd_lse(q, k[:, C:].contiguous(), v[:, C:].contiguous(), o, lse, scale,
                         mask=uaa.mask_zigzag(C, [1, 4], [0]))
    uaa.usp_attn_fwd_lse(q, k[:, :C].contiguous(), v[:, :C].contiguous(), o, lse, scale,
                         mask=uaa.mask_zigzag(C, [1, 4], [2]), accumulate=True)
    torch.cuda.synchronize()
    kpos = np.concatenate([_zigzag_pos(C, [2], C), _zigzag_pos(C, [0], C)])
    o_ref, l_ref = oracle.attention(qv, kv, vv, np.float32(scale), qpos=qpos, kpos=kpos)
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "ring pass " + out)
