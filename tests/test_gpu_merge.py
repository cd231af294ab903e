"""GPU parity of usp_lse_merge against the oracle's max-shifted merge.

Shapes: the Qwen-Image Ring share (N = 2 at [1, 3493, 24, 128]), the
FLUX-shaped share (N = 2 at [1, 4608, 12, 128]), the long-context share
(N = 8 at [1, 8192, 32, 128], checked on sampled rows), the tiny fp32 share,
plus -inf partials, in-place aliasing, mixed dtypes and odd D.
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


def _partials(cfg, n, shape, dtype, neg_inf_frac=0.0):
    """Synthetic partials: O ~ N(0,1) in the storage dtype, LSE ~ 8 + 3 N(0,1)
    in fp32, optionally some LSE entries -inf (rows with no allowed key)."""
    o_bits, o_vals, l_vals = [], [], []
    for p in range(n):
        bits, vals = synth.tensor(cfg, 100 + p, shape, dtype)
        lse = (8.0 + 3.0 * synth.normal(cfg, 200 + p, shape[:3])).astype(np.float32)
        if neg_inf_frac > 0:
            kill = synth.rng(cfg, 300 + p).random(shape[:3]) < neg_inf_frac
            lse[kill] = -np.inf
        o_bits.append(bits)
        o_vals.append(vals)
        l_vals.append(lse)
    return o_bits, o_vals, l_vals


def _gpu_merge(o_bits, l_vals, dtype, out_dtype):
    o_parts = [dev(b, dtype) for b in o_bits]
    l_parts = [torch.from_numpy(l).cuda() for l in l_vals]
    shape = o_parts[0].shape
    o_out = torch.empty(shape, device="cuda", dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    l_out = torch.empty(shape[:3], device="cuda", dtype=torch.float32)
    uaa.usp_lse_merge(o_parts, l_parts, o_out, l_out)
    torch.cuda.synchronize()
    return o_out, l_out


@pytest.mark.parametrize("name,cfg,n,shape,dtype", [
    ("qwen_ring_share", 4, 2, (1, 3493, 24, 128), "bf16"),
    ("flux_share", 2, 2, (1, 4608, 12, 128), "bf16"),
    ("tiny_fp32", 1, 2, (1, 257, 1, 64), "fp32"),
    ("three_partials_fp32", 1, 3, (2, 33, 3, 64), "fp32"),
])
def test_merge_matches_oracle(name, cfg, n, shape, dtype):
    say("merge", name)
    o_bits, o_vals, l_vals = _partials(cfg, n, shape, dtype, neg_inf_frac=0.01)
    o_out, l_out = _gpu_merge(o_bits, l_vals, dtype, dtype)
    o_ref, l_ref = oracle.lse_merge(o_vals, [l.astype(np.float64) for l in l_vals])
    check_pair(host_f64(o_out), host_f64(l_out), o_ref, l_ref, dtype, name)


def test_merge_long_context_n8_sampled_rows():
    shape = (1, 8192, 32, 128)
    say("merge long-context N=8")
    o_bits, o_vals, l_vals = _partials(5, 8, shape, "bf16", neg_inf_frac=0.02)
    # one partial entirely empty (a key chunk after every query): drops out
    l_vals[7][:] = -np.inf
    o_out, l_out = _gpu_merge(o_bits, l_vals, "bf16", "bf16")
    rows = sample_rows(8192, 512, seed=5)
    o_ref, l_ref = oracle.lse_merge([v[:, rows] for v in o_vals],
                                    [l[:, rows].astype(np.float64) for l in l_vals])
    check_pair(host_f64(o_out[:, rows]), host_f64(l_out[:, rows]), o_ref, l_ref, "bf16", "long N=8")


def test_merge_neg_inf_rules():
    shape = (1, 4, 2, 16)
    o = [np.random.default_rng(i).standard_normal(shape).astype(np.float32) for i in range(3)]
    l = [np.zeros(shape[:3], np.float32) for _ in range(3)]
    l[0][0, 0, :] = -np.inf                     # one empty partial
    for x in l:
        x[0, 1, :] = -np.inf                    # every partial empty
    l[1][0, 2, 0] = 30.0                         # dominant partial
    o_out, l_out = _gpu_merge(o, l, "fp32", "fp32")
    o_ref, l_ref = oracle.lse_merge(o, l)
    check_pair(host_f64(o_out), host_f64(l_out), o_ref, l_ref, "fp32", "neg-inf rules")
    assert (host_f64(o_out)[0, 1] == 0).all() and np.isneginf(host_f64(l_out)[0, 1]).all()


@pytest.mark.parametrize("din,dout,D", [("bf16", "bf16", 128), ("fp32", "fp32", 64), ("bf16", "bf16", 33),
                                         ("bf16", "fp32", 128)])
def test_merge_does_not_read_empty_partials(din, dout, D):
    """Rows where a partial's LSE is -inf take nothing from its O, which is
    not read: NaN there gives the same bits as zeros (the zigzag layout's
    key blocks after half the queries), and both match the oracle with 0."""
    shape = (2, 300, 3, D)
    say("merge empty partials not read", din, dout, D)
    o_bits, o_vals, l_vals = _partials(7, 5, shape, din)
    # partial 1: the second half of the rows empty; partial 4: every row empty;
    # partial 2: scattered rows empty
    l_vals[1][:, 150:] = -np.inf
    l_vals[4][:] = -np.inf
    l_vals[2][synth.rng(7, 400).random(shape[:3]) < 0.3] = -np.inf
    nan_bits, zero_vals = [], []
    for b, v, l in zip(o_bits, o_vals, l_vals):
        empty = np.isneginf(l)
        nb = b.copy()
        nb[empty] = 0x7FC0 if din == "bf16" else np.nan   # a quiet NaN in the storage dtype
        zv = v.copy()
        zv[empty] = 0.0
        nan_bits.append(nb)
        zero_vals.append(zv)
    zero_bits = [b.copy() for b in o_bits]
    for zb, l in zip(zero_bits, l_vals):
        zb[np.isneginf(l)] = 0
    o_nan, l_nan = _gpu_merge(nan_bits, l_vals, din, dout)
    o_zero, l_zero = _gpu_merge(zero_bits, l_vals, din, dout)
    assert torch.equal(l_nan, l_zero)
    assert torch.equal(o_nan.view(torch.int16) if dout == "bf16" else o_nan.view(torch.int32),
                       o_zero.view(torch.int16) if dout == "bf16" else o_zero.view(torch.int32))
    o_ref, l_ref = oracle.lse_merge(zero_vals, [l.astype(np.float64) for l in l_vals])
    check_pair(host_f64(o_nan), host_f64(l_nan), o_ref, l_ref, "fp32" if din == "fp32" else "bf16",
               "empty partials")


def test_merge_single_partial_copies():
    o = [np.random.default_rng(1).standard_normal((1, 40, 3, 64)).astype(np.float32)]
    l = [np.random.default_rng(2).standard_normal((1, 40, 3)).astype(np.float32)]
    o_out, l_out = _gpu_merge(o, l, "fp32", "fp32")
    np.testing.assert_array_equal(o_out.cpu().numpy(), o[0])
    np.testing.assert_array_equal(l_out.cpu().numpy(), l[0])


def test_merge_in_place_into_first_partial():
    shape = (1, 300, 4, 128)
    o_bits, o_vals, l_vals = _partials(2, 2, shape, "bf16")
    o_parts = [dev(b, "bf16") for b in o_bits]
    l_parts = [torch.from_numpy(x).cuda() for x in l_vals]
    uaa.usp_lse_merge(o_parts, l_parts, o_parts[0], l_parts[0])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.lse_merge(o_vals, [x.astype(np.float64) for x in l_vals])
    check_pair(host_f64(o_parts[0]), host_f64(l_parts[0]), o_ref, l_ref, "bf16", "in place")


@pytest.mark.parametrize("din,dout,D,into", [
    ("bf16", "fp32", 128, 0),    # one element per lane: two passes over the row's 128 slices
    ("bf16", "bf16", 130, 1),    # D not a multiple of the vector: 130 slices, three passes
    ("fp32", "fp32", 301, 2),    # one element per lane: 301 slices, five passes
    ("bf16", "bf16", 1024, 0),   # 16-byte slices, two passes
])
def test_merge_lse_in_place_with_several_passes_per_row(din, dout, D, into):
    """lse_out aliasing one partial's LSE (allowed for any dtype pair) when a
    row's slices outnumber the 64 lanes, so the row is merged in several
    passes: the later passes must still see the partials' own LSEs."""
    say("merge in place, several passes", din, dout, D)
    shape = (1, 37, 3, D)
    o_bits, o_vals, l_vals = _partials(6, 3, shape, din, neg_inf_frac=0.05)
    o_parts = [dev(b, din) for b in o_bits]
    l_parts = [torch.from_numpy(x).cuda() for x in l_vals]
    same = din == dout
    o_out = o_parts[into] if same else torch.empty(shape, device="cuda",
                                                   dtype=torch.bfloat16 if dout == "bf16" else torch.float32)
    uaa.usp_lse_merge(o_parts, l_parts, o_out, l_parts[into])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.lse_merge(o_vals, [x.astype(np.float64) for x in l_vals])
    check_pair(host_f64(o_out), host_f64(l_parts[into]), o_ref, l_ref,
               "bf16" if "bf16" in (din, dout) else "fp32", "in place D=%d" % D)


@pytest.mark.parametrize("din,dout", [("bf16", "fp32"), ("fp32", "bf16")])
def test_merge_mixed_dtypes(din, dout):
    shape = (2, 70, 3, 128)
    o_bits, o_vals, l_vals = _partials(3, 3, shape, din)
    o_out, l_out = _gpu_merge(o_bits, l_vals, din, dout)
    o_ref, l_ref = oracle.lse_merge(o_vals, [x.astype(np.float64) for x in l_vals])
    check_pair(host_f64(o_out), host_f64(l_out), o_ref, l_ref, "bf16" if "bf16" in (din, dout) else "fp32",
               "mixed")


@pytest.mark.parametrize("D", [1, 5, 200])
def test_merge_odd_feature_width(D):
    shape = (1, 17, 2, D)
    o_bits, o_vals, l_vals = _partials(1, 4, shape, "fp32")
    o_out, l_out = _gpu_merge(o_bits, l_vals, "fp32", "fp32")
    o_ref, l_ref = oracle.lse_merge(o_vals, [x.astype(np.float64) for x in l_vals])
    check_pair(host_f64(o_out), host_f64(l_out), o_ref, l_ref, "fp32", "D=%d" % D)


def test_merge_sixteen_partials():
    shape = (1, 64, 2, 128)
    o_bits, o_vals, l_vals = _partials(2, 16, shape, "bf16", neg_inf_frac=0.1)
    o_out, l_out = _gpu_merge(o_bits, l_vals, "bf16", "bf16")
    o_ref, l_ref = oracle.lse_merge(o_vals, [x.astype(np.float64) for x in l_vals])
    check_pair(host_f64(o_out), host_f64(l_out), o_ref, l_ref, "bf16", "N=16")


def test_merge_rejects_bad_counts():
    x = torch.zeros(1, 2, 1, 8, device="cuda")
    l = torch.zeros(1, 2, 1, device="cuda")
    with pytest.raises(uaa.UaaError):
        uaa.usp_lse_merge([x] * 17, [l] * 17, x.clone(), l.clone())
    assert math.isinf(-math.inf)
