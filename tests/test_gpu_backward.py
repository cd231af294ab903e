"""GPU parity of the attention backward (usp_attn_bwd_delta + usp_attn_bwd)
against the fp64 oracle (oracle.attention_bwd).

Bound (bf16 inputs, fp32 accumulation): every product term of a gradient
carries at most two bf16 roundings (the P or dS operand, and dS from the
bf16 P), so |g - g_ref| <= 2^-8 * sum_terms |term| up to fp32 sums; the
test allows 2^-7 * that sum (computed by the oracle side from |P|, |dS| and
the inputs) plus 1e-3 * max|g_ref| for the delta and lse the kernels get
from the bf16 forward.  Cases:

* small shapes spanning several tiles with ragged tails, every mask kind,
  rows with no allowed key, fp32 and bf16 gradients, a non-zero LSE
  gradient; all elements checked;
* a Ring pass: keys in blocks, the forward accumulated over the blocks, the
  backward per block (dq accumulated, dk / dv per block) equals the
  gradient of attention over all keys;
* edge cases: no keys (dq = 0), no queries (dk = dv = 0), accumulation;
* the FLUX Ring-block shape at full size on sampled heads, and a
  long-context zigzag block on a diagonal at full size;
* usp_attn_bwd_ws (dq from the dS the dK/dV kernel stores): the cases it
  covers against the oracle with the workspace pre-filled with NaN bits,
  dK / dV unchanged by it, the calls it does not cover, accumulation, and
  graph replays against the eager call.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import sequence_attention_dits_amd as uaa
from gpu_common import dev, host_f64, say

pytestmark = pytest.mark.gpu

REL = 2.0 ** -7
ABS_FRAC = 1e-3


def _bounds(q, k, v, do, scale, qpos, kpos, dlse):
    """Sums of |terms| of each gradient element, in float64 (the oracle's
    P and dS, recomputed here only to size the error bound)."""
    B, Sq, H, D = q.shape
    allowed = np.ones((Sq, k.shape[1]), dtype=bool) if qpos is None else kpos[None, :] <= qpos[:, None]
    live = allowed.any(axis=1)
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    o, _ = oracle.attention(q, k, v, scale, qpos=qpos, kpos=kpos)
    for b in range(B):
        for h in range(H):
            S = np.where(allowed, scale * (q[b, :, h] @ k[b, :, h].T), -np.inf)
            m = np.where(live, S.max(axis=1, initial=-np.inf), 0.0)
            E = np.exp(S - m[:, None])
            P = E / np.where(live, E.sum(axis=1), 1.0)[:, None]
            dP = do[b, :, h] @ v[b, :, h].T
            delta = (do[b, :, h] * o[b, :, h]).sum(axis=1) - (0 if dlse is None else dlse[b, :, h])
            aS = np.abs(P * (dP - delta[:, None])) + P * np.abs(delta)[:, None]
            bq[b, :, h] = scale * (aS @ np.abs(k[b, :, h]))
            bk[b, :, h] = scale * (aS.T @ np.abs(q[b, :, h]))
            bv[b, :, h] = P.T @ np.abs(do[b, :, h])
    return bq, bk, bv


def _check(name, got, ref, bound):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), name + ": non-finite gradient"
    err = np.abs(got - ref)
    lim = REL * bound + ABS_FRAC * (np.max(np.abs(ref)) if ref.size else 0.0)
    worst = float(np.max(err / np.maximum(lim, 1e-30))) if err.size else 0.0
    say("  %s: max err %.3e, max |ref| %.3e, worst err/limit %.3f" % (
        name, float(err.max()) if err.size else 0.0, float(np.abs(ref).max()) if ref.size else 0.0, worst))
    assert (err <= lim).all(), "%s: error above the bound (worst ratio %.3f)" % (name, worst)


def _inputs(cfg, B, Sq, Sk, H, D, with_dlse=False, rms=False):
    qb, q = synth.tensor(cfg, 0, (B, Sq, H, D), "bf16", rms)
    kb, k = synth.tensor(cfg, 1, (B, Sk, H, D), "bf16", rms)
    vb, v = synth.tensor(cfg, 2, (B, Sk, H, D), "bf16")
    ob, do = synth.tensor(cfg, 5, (B, Sq, H, D), "bf16")
    dl = None
    if with_dlse:
        dl = synth.normal(cfg, 6, (B, Sq, H)).astype(np.float32).astype(np.float64)
    return (qb, kb, vb, ob), (q, k, v, do), dl


def _masks(kind, Sq, Sk, **kw):
    if kind == "full":
        return uaa.mask_full(), None, None
    if kind == "causal":
        return (uaa.mask_causal(kw["q_off"], kw["k_off"]), oracle.positions({"kind": "causal", "off": kw["q_off"]}, Sq),
                oracle.positions({"kind": "causal", "off": kw["k_off"]}, Sk))
    if kind == "zigzag":
        m = uaa.mask_zigzag(kw["chunk"], kw["q_chunks"], kw["k_chunks"])
        return (m, oracle.positions({"kind": "zigzag", "chunk": kw["chunk"], "ids": kw["q_chunks"]}, Sq),
                oracle.positions({"kind": "zigzag", "chunk": kw["chunk"], "ids": kw["k_chunks"]}, Sk))
    if kind == "stripe":
        m = uaa.mask_stripe(kw["world"], kw["q_rank"], kw["k_rank"])
        return (m, oracle.positions({"kind": "stripe", "rank": kw["q_rank"], "world": kw["world"]}, Sq),
                oracle.positions({"kind": "stripe", "rank": kw["k_rank"], "world": kw["world"]}, Sk))
    raise ValueError(kind)


def _nan_workspace(q, k, mask):
    """The dS workspace of this problem filled with NaN bits (every value the
    dq kernel reads must have been written by the dK/dV kernel), or None."""
    ws = uaa.attn_bwd_workspace(q, k, mask)
    if ws is not None:
        ws.fill_(255)
    return ws


def _run_hip(bits, shapes, scale, mask, grad_dtype, dlse=None, ws=False):
    """HIP forward (o bf16, lse), delta, backward; returns host float64 grads.
    ws: through usp_attn_bwd_ws (the workspace must apply)."""
    qb, kb, vb, ob = bits
    B, Sq, Sk, H, D = shapes
    q, k, v, do = dev(qb, "bf16"), dev(kb, "bf16"), dev(vb, "bf16"), dev(ob, "bf16")
    o = torch.empty((B, Sq, H, D), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, Sq, H), device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale, mask)
    delta = torch.empty_like(lse)
    dl = None if dlse is None else torch.from_numpy(dlse.astype(np.float32)).cuda()
    uaa.usp_attn_bwd_delta(o, do, delta, dl)
    dq = torch.full((B, Sq, H, D), float("nan"), device="cuda", dtype=grad_dtype)
    dk = torch.full((B, Sk, H, D), float("nan"), device="cuda", dtype=grad_dtype)
    dv = torch.full((B, Sk, H, D), float("nan"), device="cuda", dtype=grad_dtype)
    workspace = None
    if ws:
        workspace = _nan_workspace(q, k, mask)
        assert workspace is not None, "the dS workspace should apply to this call"
    uaa.usp_attn_bwd(q, k, v, do, lse, delta, dq, dk, dv, scale, mask, workspace=workspace)
    torch.cuda.synchronize()
    return host_f64(dq), host_f64(dk), host_f64(dv)


SMALL = [
    # (name, B, Sq, Sk, H, D, mask kind, mask kwargs)
    ("full_ragged", 1, 257, 129, 2, 128, "full", {}),
    ("full_tiles_d64", 2, 256, 192, 3, 64, "full", {}),
    ("full_one_query", 1, 1, 200, 1, 128, "full", {}),
    ("full_one_key", 1, 70, 1, 2, 128, "full", {}),
    ("full_long_keys", 1, 65, 700, 1, 128, "full", {}),
    ("causal_dead_rows", 1, 200, 300, 2, 128, "causal", dict(q_off=0, k_off=100)),
    ("causal_square_d64", 1, 333, 333, 2, 64, "causal", dict(q_off=0, k_off=0)),
    ("zigzag_mixed", 1, 192, 192, 2, 128, "zigzag", dict(chunk=96, q_chunks=[1, 2], k_chunks=[0, 3])),
    ("zigzag_dead_first", 1, 192, 192, 1, 128, "zigzag", dict(chunk=96, q_chunks=[0, 3], k_chunks=[1, 2])),
    ("zigzag_ragged_d64", 1, 150, 170, 2, 64, "zigzag", dict(chunk=85, q_chunks=[2, 5], k_chunks=[1, 6])),
    ("stripe", 1, 300, 280, 2, 128, "stripe", dict(world=3, q_rank=1, k_rank=2)),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("grad", ["fp32", "bf16"])
def test_small_against_oracle(case, grad):
    name, B, Sq, Sk, H, D, kind, kw = case
    say("backward %s grads=%s B=%d Sq=%d Sk=%d H=%d D=%d" % (name, grad, B, Sq, Sk, H, D))
    cfg = 700 + SMALL.index(case)
    bits, vals, _ = _inputs(cfg, B, Sq, Sk, H, D)
    q, k, v, do = vals
    scale = 1.0 / math.sqrt(D)
    mask, qpos, kpos = _masks(kind, Sq, Sk, **kw)
    gdt = torch.float32 if grad == "fp32" else torch.bfloat16
    got = _run_hip(bits, (B, Sq, Sk, H, D), scale, mask, gdt)
    ref = oracle.attention_bwd(q, k, v, do, scale, qpos, kpos)
    bnd = _bounds(q, k, v, do, scale, qpos, kpos, None)
    extra = 2.0 ** -8 if grad == "bf16" else 0.0   # the final rounding of bf16 gradients
    for nm, g, r, bd in zip(("dq", "dk", "dv"), got, ref, bnd):
        _check(nm, g, r, bd + extra / REL * np.abs(r))
    if qpos is not None:
        dead = ~(kpos[None, :] <= qpos[:, None]).any(axis=1)
        if dead.any():
            assert (got[0][:, dead] == 0).all(), "rows without keys must get dq = 0"


WS = [
    # (name, B, Sq, Sk, H, D, mask kind, mask kwargs): calls the dS workspace
    # covers (bf16, D = 128, every pair allowed)
    ("ragged", 1, 257, 129, 2, 128, "full", {}),
    ("three_panels_two_batches", 2, 300, 200, 2, 128, "full", {}),
    ("one_query", 1, 1, 200, 1, 128, "full", {}),
    ("one_key", 1, 70, 1, 2, 128, "full", {}),
    ("long_keys", 1, 65, 700, 1, 128, "full", {}),
    ("whole_tiles", 1, 512, 256, 3, 128, "full", {}),
    ("causal_all_allowed", 1, 160, 90, 2, 128, "causal", dict(q_off=100, k_off=0)),
]


@pytest.mark.parametrize("case", WS, ids=[c[0] for c in WS])
@pytest.mark.parametrize("grad", ["fp32", "bf16"])
def test_ds_workspace_against_oracle(case, grad):
    """usp_attn_bwd_ws: dQ formed from the dS the dK/dV kernel stores (the
    workspace starts as NaN bits, so a value read but never written shows),
    against the oracle at the same bound."""
    name, B, Sq, Sk, H, D, kind, kw = case
    say("backward dS workspace %s grads=%s B=%d Sq=%d Sk=%d H=%d" % (name, grad, B, Sq, Sk, H))
    bits, vals, _ = _inputs(780 + WS.index(case), B, Sq, Sk, H, D)
    q, k, v, do = vals
    scale = 1.0 / math.sqrt(D)
    mask, qpos, kpos = _masks(kind, Sq, Sk, **kw)
    gdt = torch.float32 if grad == "fp32" else torch.bfloat16
    got = _run_hip(bits, (B, Sq, Sk, H, D), scale, mask, gdt, ws=True)
    ref = oracle.attention_bwd(q, k, v, do, scale, qpos, kpos)
    bnd = _bounds(q, k, v, do, scale, qpos, kpos, None)
    extra = 2.0 ** -8 if grad == "bf16" else 0.0
    for nm, g, r, bd in zip(("dq", "dk", "dv"), got, ref, bnd):
        _check(nm, g, r, bd + extra / REL * np.abs(r))


def test_ds_workspace_scope_and_accumulate():
    """The workspace changes only dq (dK, dV bit for bit as without it); it
    is not used where it does not apply (D = 64, a mask that excludes a pair:
    size 0) or when too small (the plain call, bit for bit); dq accumulation
    through it adds exactly."""
    B, Sq, Sk, H, D = 1, 200, 150, 2, 128
    say("backward dS workspace scope / accumulate")
    bits, _, _ = _inputs(790, B, Sq, Sk, H, D)
    qb, kb, vb, ob = bits
    q, k, v, do = dev(qb, "bf16"), dev(kb, "bf16"), dev(vb, "bf16"), dev(ob, "bf16")
    scale = 1.0 / math.sqrt(D)
    o = torch.empty((B, Sq, H, D), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, Sq, H), device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale)
    delta = torch.empty_like(lse)
    uaa.usp_attn_bwd_delta(o, do, delta)
    grads = lambda: [torch.empty((B, S, H, D), device="cuda", dtype=torch.float32) for S in (Sq, Sk, Sk)]
    g0, g1, g2, g3 = grads(), grads(), grads(), grads()
    ws = _nan_workspace(q, k, None)
    assert ws is not None and ws.numel() == B * H * ((Sq + 31) // 32) * ((Sk + 15) // 16) * 1024
    uaa.usp_attn_bwd(q, k, v, do, lse, delta, *g0, scale)
    uaa.usp_attn_bwd(q, k, v, do, lse, delta, *g1, scale, workspace=ws)
    uaa.usp_attn_bwd(q, k, v, do, lse, delta, *g2, scale, workspace=ws[:-1])   # too small: plain call
    g3 = [torch.full_like(x, 0.5) for x in g1]
    uaa.usp_attn_bwd(q, k, v, do, lse, delta, *g3, scale, accumulate="dq", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(g0[1], g1[1]) and torch.equal(g0[2], g1[2])
    assert not torch.equal(g0[0], g1[0])   # dq from the stored dS (P rounded to bf16 first)
    assert all(torch.equal(a, b) for a, b in zip(g0, g2))
    assert torch.equal(g1[0] + 0.5, g3[0]) and torch.equal(g1[1], g3[1]) and torch.equal(g1[2], g3[2])
    q64 = torch.zeros((B, Sq, H, 64), device="cuda", dtype=torch.bfloat16)
    assert uaa.attn_bwd_workspace(q64, q64[:, :Sk]) is None
    assert uaa.attn_bwd_workspace(q, k, uaa.mask_causal(0, 0)) is None
    assert uaa.attn_bwd_workspace(q.float(), k.float()) is None


def test_ds_workspace_graph_replays():
    """usp_attn_bwd_ws captured in a HIP graph (delta, then the dK/dV and dQ
    kernels sharing the workspace): every replay, with eager work and
    synchronisation between replays, equals the eager call bit for bit."""
    B, Sq, Sk, H, D = 1, 300, 260, 2, 128
    say("backward dS workspace graph replays")
    bits, _, _ = _inputs(795, B, Sq, Sk, H, D)
    qb, kb, vb, ob = bits
    q, k, v, do = dev(qb, "bf16"), dev(kb, "bf16"), dev(vb, "bf16"), dev(ob, "bf16")
    scale = 1.0 / math.sqrt(D)
    o = torch.empty((B, Sq, H, D), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, Sq, H), device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale)
    delta = torch.empty_like(lse)
    ws = _nan_workspace(q, k, None)
    grads = [torch.empty((B, S, H, D), device="cuda", dtype=torch.bfloat16) for S in (Sq, Sk, Sk)]

    def run():
        uaa.usp_attn_bwd_delta(o, do, delta)
        uaa.usp_attn_bwd(q, k, v, do, lse, delta, *grads, scale, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = [g.clone() for g in grads]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()   # warm the side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for g in grads:
            g.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for g, r in zip(grads, ref):
            assert torch.equal(g.view(torch.int16), r.view(torch.int16)), "replay %d differs" % rep


def test_lse_gradient():
    B, Sq, Sk, H, D = 1, 190, 260, 2, 128
    say("backward with dlse")
    bits, vals, dl = _inputs(731, B, Sq, Sk, H, D, with_dlse=True)
    q, k, v, do = vals
    scale = 0.11
    mask, qpos, kpos = _masks("causal", Sq, Sk, q_off=100, k_off=0)
    got = _run_hip(bits, (B, Sq, Sk, H, D), scale, mask, torch.float32, dlse=dl)
    ref = oracle.attention_bwd(q, k, v, do, scale, qpos, kpos, dl)
    bnd = _bounds(q, k, v, do, scale, qpos, kpos, dl)
    for nm, g, r, bd in zip(("dq", "dk", "dv"), got, ref, bnd):
        _check(nm, g, r, bd)


@pytest.mark.parametrize("kind", ["full", "zigzag"])
def test_ring_pass_gradient(kind):
    """Keys in R blocks: forward accumulated block by block, backward per
    block with the final (o, lse); dq summed, each block's dk / dv its own
    -- together the gradient of attention over every key."""
    B, H, D, R = 1, 2, 128, 3
    C = 80
    say("backward ring pass %s" % kind)
    if kind == "full":
        Sq, Sks = 230, [150, 77, 201]
        qpos = kposs = None
        masks = [uaa.mask_full()] * R
    else:
        # zigzag ring of R ranks, queries of rank 1, key blocks of ranks 0, 1, 2
        Sq, Sks = 2 * C, [2 * C] * R
        qids = oracle.zigzag_chunks(1, R)
        qpos = oracle.positions({"kind": "zigzag", "chunk": C, "ids": qids}, Sq)
        kposs, masks = [], []
        for r in range(R):
            kids = oracle.zigzag_chunks(r, R)
            kposs.append(oracle.positions({"kind": "zigzag", "chunk": C, "ids": kids}, Sks[r]))
            masks.append(uaa.mask_zigzag(C, qids, kids))
    Sk = sum(Sks)
    bits, vals, _ = _inputs(740 + (kind == "zigzag"), B, Sq, Sk, H, D)
    q, k, v, do = vals
    scale = 1.0 / math.sqrt(D)
    qb, kb, vb, ob = bits
    tq, tk, tv, tdo = dev(qb, "bf16"), dev(kb, "bf16"), dev(vb, "bf16"), dev(ob, "bf16")
    offs = np.cumsum([0] + Sks)
    o = torch.empty((B, Sq, H, D), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, Sq, H), device="cuda", dtype=torch.float32)
    for r in range(R):
        kr = tk[:, offs[r]:offs[r + 1]].contiguous()
        vr = tv[:, offs[r]:offs[r + 1]].contiguous()
        uaa.usp_attn_fwd_lse(tq, kr, vr, o, lse, scale, masks[r], accumulate=r > 0)
    delta = torch.empty_like(lse)
    uaa.usp_attn_bwd_delta(o, tdo, delta)
    dq = torch.empty((B, Sq, H, D), device="cuda", dtype=torch.float32)
    dks, dvs = [], []
    for r in range(R):
        kr = tk[:, offs[r]:offs[r + 1]].contiguous()
        vr = tv[:, offs[r]:offs[r + 1]].contiguous()
        # block 0 writes dq, later blocks add into it; every block's dk / dv
        # are written fresh (uninitialised buffers)
        dk = torch.empty(kr.shape, device="cuda", dtype=torch.float32)
        dv = torch.empty(kr.shape, device="cuda", dtype=torch.float32)
        uaa.usp_attn_bwd(tq, kr, vr, tdo, lse, delta, dq, dk, dv, scale, masks[r],
                         accumulate="dq" if r > 0 else False)
        dks.append(dk)
        dvs.append(dv)
    torch.cuda.synchronize()
    kpos = None if kposs is None else np.concatenate(kposs)
    ref = oracle.attention_bwd(q, k, v, do, scale, qpos, kpos)
    bnd = _bounds(q, k, v, do, scale, qpos, kpos, None)
    _check("dq", host_f64(dq), ref[0], bnd[0])
    _check("dk", np.concatenate([host_f64(x) for x in dks], axis=1), ref[1], bnd[1])
    _check("dv", np.concatenate([host_f64(x) for x in dvs], axis=1), ref[2], bnd[2])


def test_accumulate_adds_and_edges():
    B, Sq, Sk, H, D = 1, 100, 90, 2, 64
    say("backward accumulate / empty sides")
    bits, vals, _ = _inputs(750, B, Sq, Sk, H, D)
    qb, kb, vb, ob = bits
    q, k, v, do = dev(qb, "bf16"), dev(kb, "bf16"), dev(vb, "bf16"), dev(ob, "bf16")
    scale = 0.125
    o = torch.empty((B, Sq, H, D), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, Sq, H), device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(q, k, v, o, lse, scale)
    delta = torch.empty_like(lse)
    uaa.usp_attn_bwd_delta(o, do, delta)
    g1 = [torch.empty((B, S, H, D), device="cuda", dtype=torch.float32) for S in (Sq, Sk, Sk)]
    uaa.usp_attn_bwd(q, k, v, do, lse, delta, *g1, scale)
    g2 = [torch.full_like(x, 0.5) for x in g1]
    uaa.usp_attn_bwd(q, k, v, do, lse, delta, *g2, scale, accumulate=True)
    g3 = [torch.full_like(x, 0.5) for x in g1]
    uaa.usp_attn_bwd(q, k, v, do, lse, delta, *g3, scale, accumulate="dq")
    g4 = [torch.full_like(x, 0.5) for x in g1]
    uaa.usp_attn_bwd(q, k, v, do, lse, delta, *g4, scale, accumulate="dkdv")
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a + 0.5, b)
    assert torch.equal(g1[0] + 0.5, g3[0]) and torch.equal(g1[1], g3[1]) and torch.equal(g1[2], g3[2])
    assert torch.equal(g1[0], g4[0]) and torch.equal(g1[1] + 0.5, g4[1]) and torch.equal(g1[2] + 0.5, g4[2])
    # no keys: dq = 0, dk / dv untouched (empty)
    k0 = torch.empty((B, 0, H, D), device="cuda", dtype=torch.bfloat16)
    e = torch.empty((B, 0, H, D), device="cuda", dtype=torch.float32)
    dq = torch.full((B, Sq, H, D), 3.0, device="cuda")
    lse_none = torch.full_like(lse, float("-inf"))
    uaa.usp_attn_bwd(q, k0, k0, do, lse_none, delta, dq, e, e, scale)
    # no queries: dk = dv = 0
    q0 = torch.empty((B, 0, H, D), device="cuda", dtype=torch.bfloat16)
    l0 = torch.empty((B, 0, H), device="cuda", dtype=torch.float32)
    dq0 = torch.empty((B, 0, H, D), device="cuda", dtype=torch.float32)
    dk = torch.full((B, Sk, H, D), 3.0, device="cuda")
    dv = torch.full((B, Sk, H, D), 3.0, device="cuda")
    uaa.usp_attn_bwd(q0, k, v, q0, l0, l0, dq0, dk, dv, scale)
    torch.cuda.synchronize()
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()


def test_delta_matches_definition():
    B, S, H, D = 2, 77, 3, 128
    say("backward delta")
    ob, o64 = synth.tensor(760, 0, (B, S, H, D), "bf16")
    gb, g64 = synth.tensor(760, 1, (B, S, H, D), "bf16")
    dl = synth.normal(760, 2, (B, S, H)).astype(np.float32)
    delta = torch.empty((B, S, H), device="cuda", dtype=torch.float32)
    uaa.usp_attn_bwd_delta(dev(ob, "bf16"), dev(gb, "bf16"), delta, torch.from_numpy(dl).cuda())
    torch.cuda.synchronize()
    ref = (o64 * g64).sum(axis=-1) - dl.astype(np.float64)
    bound = 2.0 ** -18 * (np.abs(o64 * g64).sum(axis=-1) + np.abs(dl))
    assert (np.abs(host_f64(delta) - ref) <= bound + 1e-6).all()


@pytest.mark.parametrize("ws", [False, True], ids=["recompute", "ds_workspace"])
def test_flux_block_full_size_sampled_heads(ws):
    """The FLUX Ring-block shape (Sq = 4608 queries of 12 heads against a
    2304-key block, D = 128), in both launches the bench may time (dq
    recomputing the scores, or from the dS workspace); heads 0 and 11
    checked against the oracle element by element."""
    B, Sq, Sk, H, D = 1, 4608, 2304, 12, 128
    say("backward FLUX block full size", "ds workspace" if ws else "recompute")
    bits, vals, _ = _inputs(770, B, Sq, Sk, H, D, rms=True)
    q, k, v, do = vals
    scale = 1.0 / math.sqrt(D)
    got = _run_hip(bits, (B, Sq, Sk, H, D), scale, uaa.mask_full(), torch.float32, ws=ws)
    for h in (0, 11):
        sl = slice(h, h + 1)
        ref = oracle.attention_bwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], scale)
        bnd = _bounds(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], scale, None, None, None)
        for nm, g, r, bd in zip(("dq", "dk", "dv"), got, ref, bnd):
            _check("%s head %d" % (nm, h), g[:, :, sl], r, bd)


def test_longctx_diagonal_block_full_size_sampled_head():
    """A long-context zigzag Ring block at full size: queries = chunks {1, 6}
    of 4096 tokens, keys = chunk 1 (the first query chunk's rows see a causal
    diagonal, the second's every key), 4 heads, D = 128; head 2 checked
    against the oracle element by element."""
    chunk = 4096
    B, Sq, Sk, H, D = 1, 2 * chunk, chunk, 4, 128
    say("backward long-context diagonal block full size")
    bits, vals, _ = _inputs(775, B, Sq, Sk, H, D)
    q, k, v, do = vals
    scale = 1.0 / math.sqrt(D)
    mask, qpos, kpos = _masks("zigzag", Sq, Sk, chunk=chunk, q_chunks=[1, 6], k_chunks=[1])
    got = _run_hip(bits, (B, Sq, Sk, H, D), scale, mask, torch.float32)
    sl = slice(2, 3)
    ref = oracle.attention_bwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], scale, qpos, kpos)
    bnd = _bounds(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], scale, qpos, kpos, None)
    for nm, g, r, bd in zip(("dq", "dk", "dv"), got, ref, bnd):
        _check("%s head 2" % nm, g[:, :, sl], r, bd)


FP32 = [
    ("full_ragged_d64", 1, 257, 129, 2, 64, "full", {}),
    ("causal_dead_rows", 1, 100, 150, 2, 128, "causal", dict(q_off=0, k_off=40)),
    ("zigzag_mixed", 2, 96, 96, 1, 64, "zigzag", dict(chunk=48, q_chunks=[1, 2], k_chunks=[0, 3])),
]


def _fp32_inputs(cfg, B, Sq, Sk, H, D):
    vals = [synth.tensor(cfg, t, shp, "fp32")[1] for t, shp in
            ((0, (B, Sq, H, D)), (1, (B, Sk, H, D)), (2, (B, Sk, H, D)), (5, (B, Sq, H, D)))]
    return vals


def _check_fp32(name, got, ref, bound):
    assert np.isfinite(got).all(), name + ": non-finite gradient"
    err = np.abs(got - ref)
    lim = 1e-5 * bound + 1e-6 * (np.max(np.abs(ref)) if ref.size else 0.0)
    worst = float(np.max(err / np.maximum(lim, 1e-30))) if err.size else 0.0
    say("  %s: max err %.3e, worst err/limit %.3f" % (name, float(err.max()) if err.size else 0.0, worst))
    assert (err <= lim).all(), "%s: fp32 error above the bound (worst ratio %.3f)" % (name, worst)


@pytest.mark.parametrize("case", FP32, ids=[c[0] for c in FP32])
def test_fp32_against_oracle(case):
    """fp32 inputs: the full-precision kernels, within 1e-5 of the sum of
    |terms| of each gradient element (plus 1e-6 of its largest value)."""
    name, B, Sq, Sk, H, D, kind, kw = case
    say("backward fp32 %s" % name)
    q, k, v, do = _fp32_inputs(780 + FP32.index(case), B, Sq, Sk, H, D)
    scale = 1.0 / math.sqrt(D)
    mask, qpos, kpos = _masks(kind, Sq, Sk, **kw)
    tq, tk, tv, tdo = (dev(x, "fp32") for x in (q, k, v, do))
    o = torch.empty_like(tq)
    lse = torch.empty((B, Sq, H), device="cuda", dtype=torch.float32)
    uaa.usp_attn_fwd_lse(tq, tk, tv, o, lse, scale, mask)
    delta = torch.empty_like(lse)
    uaa.usp_attn_bwd_delta(o, tdo, delta)
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
    uaa.usp_attn_bwd(tq, tk, tv, tdo, lse, delta, dq, dk, dv, scale, mask)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(q, k, v, do, scale, qpos, kpos)
    bnd = _bounds(q, k, v, do, scale, qpos, kpos, None)
    for nm, g, r, bd in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, bnd):
        _check_fp32(nm, host_f64(g), r, bd)


def test_fp32_ring_share_shape():
    """The small fp32 share (257 tokens, 2 heads, D = 64) as a two-block
    Ring pass: forward accumulated over key blocks of 129 and 128 tokens,
    backward per block against the final (o, lse)."""
    B, S, H, D = 1, 257, 2, 64
    say("backward fp32 ring share")
    q, k, v, do = _fp32_inputs(790, B, S, S, H, D)
    scale = 1.0 / math.sqrt(D)
    tq, tk, tv, tdo = (dev(x, "fp32") for x in (q, k, v, do))
    o = torch.empty_like(tq)
    lse = torch.empty((B, S, H), device="cuda", dtype=torch.float32)
    blocks = [(0, 129), (129, 257)]
    for n, (a, b) in enumerate(blocks):
        uaa.usp_attn_fwd_lse(tq, tk[:, a:b].contiguous(), tv[:, a:b].contiguous(), o, lse, scale, accumulate=n > 0)
    delta = torch.empty_like(lse)
    uaa.usp_attn_bwd_delta(o, tdo, delta)
    dq = torch.empty_like(tq)
    dks, dvs = [], []
    for n, (a, b) in enumerate(blocks):
        kb, vb = tk[:, a:b].contiguous(), tv[:, a:b].contiguous()
        dk, dv = torch.empty_like(kb), torch.empty_like(vb)
        uaa.usp_attn_bwd(tq, kb, vb, tdo, lse, delta, dq, dk, dv, scale, accumulate="dq" if n else False)
        dks.append(dk)
        dvs.append(dv)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(q, k, v, do, scale)
    bnd = _bounds(q, k, v, do, scale, None, None, None)
    _check_fp32("dq", host_f64(dq), ref[0], bnd[0])
    _check_fp32("dk", np.concatenate([host_f64(x) for x in dks], axis=1), ref[1], bnd[1])
    _check_fp32("dv", np.concatenate([host_f64(x) for x in dvs], axis=1), ref[2], bnd[2])
