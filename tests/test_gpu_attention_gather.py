"""Parity of the gathering attention (usp_attn_fwd_lse_gather): rank r's
Ulysses view of token-sharded Q, K, V read straight from the shards through
the length prefix sums ("Context parallelism", Ulysses Attention and Ulysses
Anything Attention), instead of from the SEQ2HEAD copy.  The call is defined
as that copy followed by usp_attn_fwd_lse(_acc) on it, so the two must agree
bit for bit: shard lengths that are and are not multiples of the row tiles
(a wave's 32 query rows then straddle two shards), an empty shard, uneven
heads, B = 2, every rank, the Ring-step accumulate, the key split and a
causal mask by global position.  One case is also checked against the
oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import sequence_attention_dits_amd as uaa
from gpu_common import check_pair, dev, host_f64, say

pytestmark = pytest.mark.gpu


def _shards(cfg, B, seq_off, H, D):
    """Seeded global Q, K, V [B, S, H, D] (bf16 bits), cut into token shards."""
    S = seq_off[-1]
    qb, qv = synth.tensor(cfg, 0, (B, S, H, D), "bf16", rms_norm=True)
    kb, kv_ = synth.tensor(cfg, 1, (B, S, H, D), "bf16", rms_norm=True)
    vb, vv = synth.tensor(cfg, 2, (B, S, H, D), "bf16")
    cut = lambda x: [dev(np.ascontiguousarray(x[:, a:b]), "bf16") for a, b in zip(seq_off[:-1], seq_off[1:])]
    return (cut(qb), cut(kb), cut(vb)), (qv, kv_, vv)


def _reference(rank, shards, k_shard, seq_off, head_off, scale, mask, acc_from=None, ws=None):
    """SEQ2HEAD copies, then usp_attn_fwd_lse(_acc) on them."""
    q_s, k_s, v_s = shards
    B, _, H, D = q_s[0].shape
    S = seq_off[-1]
    hoff = head_off if head_off is not None else oracle.split_offsets(H, len(seq_off) - 1)
    Hr = hoff[rank + 1] - hoff[rank]
    ys = []
    for sh in (q_s, k_s, v_s):
        y = torch.empty(B, S, Hr, D, device="cuda", dtype=torch.bfloat16)
        uaa.uaa_seq2head_permute(uaa.UAA_SEQ2HEAD, rank, sh, y, seq_off, head_off)
        ys.append(y)
    a, b = seq_off[k_shard], seq_off[k_shard + 1]
    o = torch.empty(B, S, Hr, D, device="cuda", dtype=torch.bfloat16) if acc_from is None else acc_from[0].clone()
    lse = torch.empty(B, S, Hr, device="cuda") if acc_from is None else acc_from[1].clone()
    uaa.usp_attn_fwd_lse(ys[0], ys[1][:, a:b].contiguous(), ys[2][:, a:b].contiguous(), o, lse, scale, mask,
                         workspace=ws, accumulate=acc_from is not None)
    return o, lse


CASES = [
    # (name, B, seq_off, H, head_off, D)
    ("aligned_2x256", 1, [0, 256, 512], 4, None, 128),
    ("ragged_129_128", 1, [0, 129, 257], 4, None, 128),
    ("ragged_2241_2240", 1, [0, 2241, 4481], 2, None, 128),
    ("three_with_empty", 1, [0, 100, 100, 161], 3, None, 64),
    ("uneven_heads_b2", 2, [0, 300, 333], 5, [0, 3, 5], 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gather_equals_permute_then_attention(case):
    name, B, seq_off, H, head_off, D = case
    world = len(seq_off) - 1
    shards, _ = _shards(990 + CASES.index(case), B, seq_off, H, D)
    scale = 1.0 / math.sqrt(D)
    hoff = head_off if head_off is not None else oracle.split_offsets(H, world)
    for rank in range(world):
        Hr = hoff[rank + 1] - hoff[rank]
        S = seq_off[-1]
        o = torch.full((B, S, Hr, D), float("nan"), device="cuda", dtype=torch.bfloat16)
        lse = torch.full((B, S, Hr), float("nan"), device="cuda")
        ref = None
        for ks in range(world):   # every shard's keys, plain then accumulating
            say("attn gather", name, "rank", rank, "k_shard", ks)
            uaa.usp_attn_fwd_lse_gather(rank, *shards, ks, o, lse, scale, seq_off, head_off, accumulate=ks > 0)
            ref = _reference(rank, shards, ks, seq_off, head_off, scale, None, acc_from=ref)
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16)), (name, rank, ks)
            assert torch.equal(torch.nan_to_num(lse), torch.nan_to_num(ref[1])), (name, rank, ks)


def test_gather_with_key_split_and_oracle():
    """B=2, 1000 tokens in two shards of 500, 6 heads (3 per rank): 24 units
    split over the keys; also checked against the oracle over all keys."""
    B, seq_off, H, D = 2, [0, 500, 1000], 6, 128
    shards, (qv, kv_, vv) = _shards(996, B, seq_off, H, D)
    scale = 1.0 / math.sqrt(D)
    rank = 1
    S, Hr = seq_off[-1], 3
    ws = uaa.attn_workspace(torch.empty(B, S, Hr, D, device="cuda", dtype=torch.bfloat16),
                            torch.empty(B, 500, Hr, D, device="cuda", dtype=torch.bfloat16))
    assert ws is not None
    o = torch.empty(B, S, Hr, D, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B, S, Hr, device="cuda")
    for ks in range(2):
        uaa.usp_attn_fwd_lse_gather(rank, *shards, ks, o, lse, scale, seq_off, workspace=ws, accumulate=ks > 0)
    ref = None
    for ks in range(2):
        ref = _reference(rank, shards, ks, seq_off, None, scale, None, acc_from=ref, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16))
    assert torch.equal(lse, ref[1])
    o_ref, l_ref = oracle.attention(qv[:, :, 3:6], kv_[:, :, 3:6], vv[:, :, 3:6], np.float32(scale))
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "gather + split")


def test_gather_causal_by_global_position():
    B, seq_off, H, D = 1, [0, 200, 390], 2, 128
    shards, _ = _shards(997, B, seq_off, H, D)
    scale = 1.0 / math.sqrt(D)
    o = torch.empty(B, 390, 1, D, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B, 390, 1, device="cuda")
    ref = None
    for ks in range(2):
        m = uaa.mask_causal(0, seq_off[ks])
        uaa.usp_attn_fwd_lse_gather(0, *shards, ks, o, lse, scale, seq_off, None, m, accumulate=ks > 0)
        ref = _reference(0, shards, ks, seq_off, None, scale, m, acc_from=ref)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16))
    assert torch.equal(lse, ref[1])


def test_gather_rejects_fp32_and_bad_shard_index():
    x = torch.zeros(1, 4, 2, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.empty(1, 8, 1, 64, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(1, 8, 1, device="cuda")
    with pytest.raises(uaa.UaaError) as e:
        uaa.usp_attn_fwd_lse_gather(0, [x, x], [x, x], [x, x], 2, o, lse, 0.1, [0, 4, 8])
    assert e.value.status == uaa.UAA_ERR_INVALID_ARG


@pytest.mark.parametrize("H,rank", [(5, 0), (5, 1)])
def test_gather_default_head_split_against_oracle(H, rank):
    """head_off = None goes to the library as NULL; the rank's heads are the
    oracle's own split (3 / 2 of 5), and the Ring pass over both token shards
    must equal the oracle's attention of those heads over every key."""
    B, seq_off, D = 1, [0, 197, 389], 128
    shards, (qv, kv_, vv) = _shards(998, B, seq_off, H, D)
    scale = 1.0 / math.sqrt(D)
    hoff = oracle.split_offsets(H, 2)
    h0, h1 = hoff[rank], hoff[rank + 1]
    o = torch.empty(B, 389, h1 - h0, D, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B, 389, h1 - h0, device="cuda")
    say("attn gather default head split H=%d rank %d" % (H, rank))
    for ks in range(2):
        uaa.usp_attn_fwd_lse_gather(rank, *shards, ks, o, lse, scale, seq_off, None, accumulate=ks > 0)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qv[:, :, h0:h1], kv_[:, :, h0:h1], vv[:, :, h0:h1], np.float32(scale))
    check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "gather, default head split")
