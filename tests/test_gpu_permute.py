"""GPU parity of uaa_seq2head_permute against the oracle: bit-exact.

Covers the tiny ragged fp32 share (129/128 tokens), the FLUX-shaped share
(2 x 2304 tokens, 24 heads) and the non-divisible FLUX share (2241/2240),
index-coded data with empty shards and uneven heads, every element width,
the LSE (D = 1) exchange, the round trip, and empty work.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import sequence_attention_dits_amd as uaa
from gpu_common import say

pytestmark = pytest.mark.gpu


def _run(direction, rank, src_np, seq_off, head_off, dtype_np, torch_dtype):
    src = [torch.from_numpy(np.ascontiguousarray(x).view(dtype_np)).cuda().view(torch_dtype) for x in src_np]
    B, D = src_np[0].shape[0], src_np[0].shape[3]
    world = len(src_np)
    if direction == uaa.UAA_SEQ2HEAD:
        shape = (B, seq_off[-1], head_off[rank + 1] - head_off[rank], D)
    else:
        shape = (B, seq_off[rank + 1] - seq_off[rank], head_off[-1], D)
    dst = torch.empty(shape, dtype=torch_dtype, device="cuda")
    uaa.uaa_seq2head_permute(direction, rank, src, dst, seq_off, head_off)
    torch.cuda.synchronize()
    return dst.view(torch.int8 if dst.element_size() == 1 else
                    {2: torch.int16, 4: torch.int32, 8: torch.int64}[dst.element_size()]).cpu().numpy()


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_config_shares_bit_exact(cfg):
    c = synth.CONFIGS[cfg]
    B, S, H, D = c["B"], c["S"], c["H"], c["D"]
    seq_off = [0, c["shards"][0], S]
    head_off = oracle.split_offsets(H, 2)
    bits, _ = synth.tensor(cfg, 0, (B, S, H, D), c["dtype"], rms_norm=c["rms"])
    raw = bits.view(np.uint16) if c["dtype"] == "bf16" else bits.view(np.uint32)
    shards = [raw[:, seq_off[p]:seq_off[p + 1]] for p in range(2)]
    tdt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    ndt = np.int16 if c["dtype"] == "bf16" else np.int32
    for rank in range(2):
        say("permute cfg%d SEQ2HEAD rank %d" % (cfg, rank))
        got = _run(uaa.UAA_SEQ2HEAD, rank, shards, seq_off, head_off, ndt, tdt)
        ref = oracle.seq2head(shards, rank, seq_off, head_off)
        assert got.tobytes() == ref.tobytes()
    heads = [oracle.seq2head(shards, r, seq_off, head_off) for r in range(2)]
    for p in range(2):
        say("permute cfg%d HEAD2SEQ rank %d" % (cfg, p))
        got = _run(uaa.UAA_HEAD2SEQ, p, heads, seq_off, head_off, ndt, tdt)
        assert got.tobytes() == np.ascontiguousarray(shards[p]).tobytes()


SPLITS = [
    ([0, 5, 5, 12, 20], [0, 2, 3, 5, 7]),
    ([0, 0, 9], [0, 3, 5]),
    ([0, 13, 26, 39], [0, 1, 2, 3]),
    ([0, 1], [0, 4]),
    ([0, 300, 301, 700], [0, 5, 10, 24]),
]


@pytest.mark.parametrize("seq_off,head_off", SPLITS)
@pytest.mark.parametrize("B,D", [(1, 128), (2, 64), (3, 1), (1, 3)])
def test_index_coded_matches_oracle_map(seq_off, head_off, B, D):
    world = len(seq_off) - 1
    H = head_off[-1]
    # element value = shard * 2^24 + flat index inside the shard (int32, 4-byte elements)
    shards = []
    for p in range(world):
        n = B * (seq_off[p + 1] - seq_off[p]) * H * D
        shards.append((np.arange(n, dtype=np.int64) + (p << 24)).astype(np.int32)
                      .reshape(B, seq_off[p + 1] - seq_off[p], H, D))
    for r in range(world):
        say("permute index-coded", seq_off, head_off, B, D, "rank", r)
        got = _run(uaa.UAA_SEQ2HEAD, r, shards, seq_off, head_off, np.int32, torch.int32)
        sh, el = oracle.seq2head_index(r, world, seq_off, head_off, B, H, D)
        np.testing.assert_array_equal(got.astype(np.int64), (sh << 24) + el)


@pytest.mark.parametrize("np_dt,t_dt", [(np.int8, torch.int8), (np.int16, torch.int16),
                                        (np.int32, torch.int32), (np.int64, torch.int64)])
def test_every_element_width_round_trip(np_dt, t_dt):
    seq_off, head_off = [0, 7, 7, 30], [0, 1, 3, 6]
    B, H, D = 2, 6, 5
    rng = np.random.default_rng(3)
    x = rng.integers(-100, 100, size=(B, 30, H, D)).astype(np_dt)
    shards = [x[:, seq_off[p]:seq_off[p + 1]] for p in range(3)]
    heads = []
    for r in range(3):
        got = _run(uaa.UAA_SEQ2HEAD, r, shards, seq_off, head_off, np_dt, t_dt)
        ref = oracle.seq2head(shards, r, seq_off, head_off)
        assert got.tobytes() == ref.tobytes()
        heads.append(ref)
    for p in range(3):
        got = _run(uaa.UAA_HEAD2SEQ, p, heads, seq_off, head_off, np_dt, t_dt)
        assert got.tobytes() == np.ascontiguousarray(shards[p]).tobytes()


def test_lse_exchange_d1():
    # The Unified path moves the LSE as (B, S, H_LOCAL, 1) fp32.
    seq_off, head_off = [0, 2241, 4481], [0, 12, 24]
    rng = np.random.default_rng(4)
    heads = [rng.standard_normal((1, 4481, 12, 1)).astype(np.float32) for _ in range(2)]
    for p in range(2):
        got = _run(uaa.UAA_HEAD2SEQ, p, heads, seq_off, head_off, np.int32, torch.float32)
        ref = oracle.head2seq(heads, p, seq_off, head_off)
        assert got.tobytes() == ref.tobytes()


def test_single_rank_is_copy_and_empty_shard_is_noop():
    x = torch.randn(2, 33, 4, 128, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(x)
    uaa.uaa_seq2head_permute(uaa.UAA_SEQ2HEAD, 0, [x], y, [0, 33], [0, 4])
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    # token rank 1 holds no tokens: HEAD2SEQ has nothing to write
    heads = [torch.randn(1, 9, 2, 64, device="cuda") for _ in range(2)]
    dst = torch.empty(1, 0, 4, 64, device="cuda")
    uaa.uaa_seq2head_permute(uaa.UAA_HEAD2SEQ, 1, heads, dst, [0, 9, 9], [0, 2, 4])
    torch.cuda.synchronize()


def test_misaligned_view_falls_back_to_narrow_access():
    # shards that start 2 bytes into an allocation cannot use 16-byte accesses
    n0 = 2 * 20 * 3 * 8
    buf = torch.arange(1 + 2 * n0, dtype=torch.int16, device="cuda")
    s0 = buf[1:1 + n0].view(2, 20, 3, 8)
    s1 = buf[1 + n0:1 + 2 * n0].view(2, 20, 3, 8)
    ybuf = torch.zeros(1 + 2 * 40 * 1 * 8, dtype=torch.int16, device="cuda")
    y = ybuf[1:].view(2, 40, 1, 8)
    uaa.uaa_seq2head_permute(uaa.UAA_SEQ2HEAD, 1, [s0, s1], y, [0, 20, 40], None)  # heads split 2/1
    torch.cuda.synchronize()
    ref = torch.cat([s0, s1], 1)[:, :, 2:3]
    assert torch.equal(ref, y)


def test_bad_arguments_are_rejected_before_launch():
    x = torch.zeros(1, 10, 4, 64, device="cuda", dtype=torch.bfloat16)
    y = torch.zeros(1, 20, 2, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ValueError):          # offsets disagree with the shapes
        uaa.uaa_seq2head_permute(uaa.UAA_SEQ2HEAD, 0, [x, x], y, [0, 10, 21], [0, 2, 4])
    y0 = torch.zeros(1, 20, 0, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(uaa.UaaError):        # a rank with no heads
        uaa.uaa_seq2head_permute(uaa.UAA_SEQ2HEAD, 0, [x, x], y0, [0, 10, 20], [0, 0, 4])


@pytest.mark.parametrize("direction", [uaa.UAA_SEQ2HEAD, uaa.UAA_HEAD2SEQ])
@pytest.mark.parametrize("n_t,seq_off,head_off,B,D", [
    (3, [0, 2304, 4608], [0, 12, 24], 1, 128),
    (3, [0, 2241, 4481], [0, 12, 24], 1, 128),
    (4, [0, 5, 5, 40], [0, 1, 3, 5], 2, 64),
    (2, [0, 100, 130, 131, 300], [0, 3, 4, 6, 9], 3, 128),
])
def test_multi_tensor_permute_equals_separate_calls(direction, n_t, seq_off, head_off, B, D):
    world = len(seq_off) - 1
    H = head_off[-1]
    S = seq_off[-1]
    gen = torch.Generator(device="cpu").manual_seed(n_t * 7 + B)
    srcs, dsts, refs = [], [], []
    for t in range(n_t):
        if direction == uaa.UAA_SEQ2HEAD:
            src = [torch.randn(B, seq_off[p + 1] - seq_off[p], H, D, generator=gen).to(torch.bfloat16).cuda()
                   for p in range(world)]
        else:
            src = [torch.randn(B, S, head_off[r + 1] - head_off[r], D, generator=gen).to(torch.bfloat16).cuda()
                   for r in range(world)]
        srcs.append(src)
    rank = 1
    for t in range(n_t):
        if direction == uaa.UAA_SEQ2HEAD:
            shape = (B, S, head_off[rank + 1] - head_off[rank], D)
        else:
            shape = (B, seq_off[rank + 1] - seq_off[rank], H, D)
        ref = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        uaa.uaa_seq2head_permute(direction, rank, srcs[t], ref, seq_off, head_off)
        refs.append(ref)
        dsts.append(torch.full(shape, 3.0, dtype=torch.bfloat16, device="cuda"))
    say("permute multi", direction, n_t, seq_off, head_off, B, D)
    uaa.uaa_seq2head_permute_multi(direction, rank, srcs, dsts, seq_off, head_off)
    torch.cuda.synchronize()
    for ref, got in zip(refs, dsts):
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


@pytest.mark.parametrize("direction", [uaa.UAA_SEQ2HEAD, uaa.UAA_HEAD2SEQ])
@pytest.mark.parametrize("seq_off,head_off", [([0, 129, 257], [0, 7, 13]), ([0, 2241, 4481], [0, 12, 24])])
def test_multi_tensor_mixed_row_sizes_equal_separate_calls(direction, seq_off, head_off):
    """O (bf16, D=128), its LSE (fp32, D=1) and an odd fp32 D=3 tensor in one
    launch (uaa_seq2head_permute_multi_ex) equal three separate calls."""
    world = len(seq_off) - 1
    H, S, B, rank = head_off[-1], seq_off[-1], 1, 1
    gen = torch.Generator(device="cpu").manual_seed(S)
    kinds = [(128, torch.bfloat16), (1, torch.float32), (3, torch.float32)]
    srcs, dsts, refs = [], [], []
    for D, dt in kinds:
        if direction == uaa.UAA_SEQ2HEAD:
            src = [torch.randn(B, seq_off[p + 1] - seq_off[p], H, D, generator=gen).to(dt).cuda() for p in range(world)]
            shape = (B, S, head_off[rank + 1] - head_off[rank], D)
        else:
            src = [torch.randn(B, S, head_off[r + 1] - head_off[r], D, generator=gen).to(dt).cuda() for r in range(world)]
            shape = (B, seq_off[rank + 1] - seq_off[rank], H, D)
        ref = torch.empty(shape, dtype=dt, device="cuda")
        uaa.uaa_seq2head_permute(direction, rank, src, ref, seq_off, head_off)
        srcs.append(src)
        refs.append(ref)
        dsts.append(torch.full(shape, 3.0, dtype=dt, device="cuda"))
    say("permute multi_ex", direction, seq_off, head_off)
    uaa.uaa_seq2head_permute_multi(direction, rank, srcs, dsts, seq_off, head_off)
    torch.cuda.synchronize()
    for ref, got in zip(refs, dsts):
        iv = torch.int16 if ref.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(ref.view(iv), got.view(iv))
    # and the O + LSE pair alone (the step's inverse gather)
    d2 = [torch.full_like(refs[0], 5.0), torch.full_like(refs[1], 5.0)]
    uaa.uaa_seq2head_permute_multi(direction, rank, srcs[:2], d2, seq_off, head_off)
    torch.cuda.synchronize()
    assert torch.equal(refs[0].view(torch.int16), d2[0].view(torch.int16))
    assert torch.equal(refs[1].view(torch.int32), d2[1].view(torch.int32))


@pytest.mark.parametrize("S,H,world,seq_split", [
    (389, 5, 2, None),               # uneven heads: 3 / 2
    (4481, 24, 2, [0, 2241, 4481]),  # the non-divisible FLUX share: 12 / 12 heads, 2241 / 2240 tokens
    (100, 7, 3, [0, 40, 40, 100]),   # 3 / 2 / 2 heads, an empty token shard
])
def test_default_head_split_inside_the_library(S, H, world, seq_split):
    """head_off = None is passed to the library as NULL: the heads are split
    there, and the result must equal the oracle's gather with the oracle's
    own split (first H mod world ranks take one extra head)."""
    B, D = 1, 64
    seq_off = seq_split or oracle.split_offsets(S, world)
    head_off = oracle.split_offsets(H, world)
    assert uaa.uaa_split_offsets(H, world) == head_off
    x = (np.arange(B * S * H * D, dtype=np.int64) * 2654435761 % (1 << 31)).astype(np.int32).reshape(B, S, H, D)
    shards = [x[:, seq_off[p]:seq_off[p + 1]] for p in range(world)]
    dev_shards = [torch.from_numpy(np.ascontiguousarray(s)).cuda() for s in shards]
    heads = []
    for r in range(world):
        say("permute default head split S=%d H=%d world=%d SEQ2HEAD rank %d" % (S, H, world, r))
        dst = torch.empty(B, S, head_off[r + 1] - head_off[r], D, dtype=torch.int32, device="cuda")
        uaa.uaa_seq2head_permute(uaa.UAA_SEQ2HEAD, r, dev_shards, dst, seq_off, None)
        torch.cuda.synchronize()
        ref = oracle.seq2head(shards, r, seq_off, head_off)
        assert dst.cpu().numpy().tobytes() == ref.tobytes()
        heads.append(dst)
    for p in range(world):
        say("permute default head split HEAD2SEQ rank %d" % p)
        out = torch.empty(B, seq_off[p + 1] - seq_off[p], H, D, dtype=torch.int32, device="cuda")
        uaa.uaa_seq2head_permute(uaa.UAA_HEAD2SEQ, p, heads, out, seq_off, None)
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == np.ascontiguousarray(shards[p]).tobytes()
    # the multi-tensor entry with its NULL head split: O and its LSE together
    lse_heads = [h[..., :1].contiguous() for h in heads]
    out_o = torch.empty(B, seq_off[1], H, D, dtype=torch.int32, device="cuda")
    out_l = torch.empty(B, seq_off[1], H, 1, dtype=torch.int32, device="cuda")
    uaa.uaa_seq2head_permute_multi(uaa.UAA_HEAD2SEQ, 0, [heads, lse_heads], [out_o, out_l], seq_off, None)
    torch.cuda.synchronize()
    assert out_o.cpu().numpy().tobytes() == np.ascontiguousarray(shards[0]).tobytes()
    assert out_l.cpu().numpy().tobytes() == np.ascontiguousarray(shards[0][..., :1]).tobytes()


def test_default_head_split_rejects_mismatched_destination():
    """With head_off None the binding checks the destination against the
    library's split, so a tensor sized for another split is refused before
    any launch."""
    src = [torch.zeros(1, 4, 5, 8, device="cuda"), torch.zeros(1, 4, 5, 8, device="cuda")]
    wrong = torch.empty(1, 8, 2, 8, device="cuda")    # rank 0 gets 3 of 5 heads
    with pytest.raises(ValueError):
        uaa.uaa_seq2head_permute(uaa.UAA_SEQ2HEAD, 0, src, wrong, [0, 4, 8], None)
