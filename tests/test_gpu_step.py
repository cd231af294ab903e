"""The step that bench.py times, at full size, against the fp64 oracle.

Each workload's step is built by ``bench.make_share`` exactly as the bench
builds it (the same launches, kernels, streams, workspaces and Ring-step
update), run once eagerly, then captured as a HIP graph and replayed (the
form the bench times; every replay must equal the eager step bit for bit),
and compared with the oracle's composition of the same pass:

* FLUX.1-dev 1024x1024 and 1008x1008 rank shares (Ulysses / Ulysses
  Anything, "Context parallelism" docs, sections "Ulysses Attention" and
  "Ulysses Anything Attention"): SEQ2HEAD of Q, K and V from the two token
  shards, attention of the 12 heads over two Ring chunks of keys with the
  second merged into the first's (O, LSE) in its epilogue ("Add Unified
  Sequence Parallel attention", review thread: the Ring loop's merge of
  (out, lse)), then HEAD2SEQ of O and of the LSE into token shard 0.  Every
  row of the head-sharded (O, LSE) [1, S, 12, 128] is compared with the
  oracle's gather + Ring pass; the token shard the step returns must equal
  the oracle's inverse gather of the GPU's head shard and of the stand-in
  shard of the other head rank bit for bit, and its attention heads match
  the oracle's rows within the tolerance.
* Qwen-Image 1328x1328 Ring share ("Ring Attention"): the 3493 queries
  against both K/V chunks, merged by one usp_lse_merge launch; every row.
* long-context zigzag share (USP / yunchang summary, "How It Works": the
  zigzag layout): queries = chunks {1, 6} of 8, against all 8 K/V chunks
  masked by global position on two streams, merged by the Ring-step update
  (one running result per stream, then their 2-way merge) as the bench times
  it, and as 8 partials with one 8-way merge; 1024 rows sampled across both
  query chunks (the first and last rows of every 256-row unit included),
  since the oracle takes ~45 s for all 8192.

Tolerances: bf16 outputs, max-abs 2e-2 on O and 1e-3 on the LSE; rows the
oracle leaves without a key must come back exactly (0, -inf).
"""

import numpy as np
import pytest
import torch

import bench
import oracle
import sequence_attention_dits_amd as uaa
from gpu_common import check_pair, host_f64, say

pytestmark = pytest.mark.gpu


def _run_eager_and_graph(share):
    """One eager step, then the captured step replayed twice; returns the
    eager outputs (device tensors, cloned) after checking that each replay
    reproduces them bit for bit: the step's result, and for the Ulysses
    shares also the head-sharded (O, LSE) before the inverse gather."""
    outs = list(share.result())
    if share.result()[0] is not share.o:
        outs += [share.o, share.lse]
    share.step(0)
    torch.cuda.synchronize()
    res = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        share.step(0)
    torch.cuda.synchronize()
    for rep in range(2):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(res, outs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "graph replay %d differs" % rep
    del g
    return res


@pytest.mark.parametrize("workload", ["flux1024", "flux1008"])
def test_flux_step_every_row(workload):
    say("step", workload, "build")
    share = bench.make_share(workload, 1)
    assert share.ring_acc
    for a, b in share.ring:
        assert uaa.usp_attn_kernel((share.B, share.S, share.Hr, share.D), b - a) == uaa.USP_KERNEL_PIPELINED
    say("step", workload, "run")
    o_tok, l_tok, o_heads, l_heads = _run_eager_and_graph(share)

    say("step", workload, "oracle")
    h = share.host
    heads = {}
    for name in "qkv":
        shards = [h[name][:, a:b] for a, b in zip(share.seq_off[:-1], share.seq_off[1:])]
        heads[name] = oracle.seq2head(shards, 0, share.seq_off, share.head_off)
    o_ref, l_ref = oracle.ring_pass(heads["q"], [heads["k"][:, a:b] for a, b in share.ring],
                                    [heads["v"][:, a:b] for a, b in share.ring], share.scale)
    err = check_pair(host_f64(o_heads), host_f64(l_heads), o_ref, l_ref, "bf16", workload + " head shard")
    say("step", workload, "head shard, every row: O err %.3e, LSE err %.3e" % (err["o_err"], err["lse_err"]))

    # the inverse gather, bit for bit, of the GPU's head shard and the
    # stand-in shard of the other head rank
    d = share.sets[0]
    bits = lambda t: t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
    o_exp = oracle.head2seq([bits(o_heads), bits(d["o_other"])], 0, share.seq_off, share.head_off)
    l_exp = oracle.head2seq([l_heads.unsqueeze(-1).cpu().numpy(), d["l_other"].cpu().numpy()], 0,
                            share.seq_off, share.head_off)
    assert bits(o_tok).tobytes() == o_exp.tobytes()
    assert l_tok.cpu().numpy().tobytes() == l_exp.tobytes()
    S0, Hr = share.seq_off[1], share.Hr
    check_pair(host_f64(o_tok[:, :, :Hr]), host_f64(l_tok[:, :, :Hr, 0]), o_ref[:, :S0], l_ref[:, :S0], "bf16",
               workload + " token shard")


def _ring_reference(share, rows=None):
    h = share.host
    qpos = h["q_rows"] if share.masks[0] is not None else None
    kpos = [np.arange(a, b) for a, b in share.kv] if qpos is not None else None
    return oracle.ring_pass(h["q"], [h["k"][:, a:b] for a, b in share.kv], [h["v"][:, a:b] for a, b in share.kv],
                            share.scale, qpos=qpos, kpos_chunks=kpos, rows=rows)


def test_qwen_ring_step_every_row():
    say("step qwen1328 build")
    share = bench.make_share("qwen1328", 1)
    say("step qwen1328 run")
    o, lse = _run_eager_and_graph(share)
    say("step qwen1328 oracle")
    o_ref, l_ref = _ring_reference(share)
    err = check_pair(host_f64(o), host_f64(lse), o_ref, l_ref, "bf16", "qwen1328 step")
    say("step qwen1328 every row: O err %.3e, LSE err %.3e" % (err["o_err"], err["lse_err"]))


@pytest.mark.parametrize("ring_update", ["auto", "merge"])
def test_longctx_zigzag_step_sampled_rows(ring_update):
    say("step longctx build", ring_update)
    share = bench.make_share("longctx", 1, ring_update=ring_update)
    assert share.overlap_chunks and share.ring_acc == (ring_update == "auto")
    say("step longctx run")
    o, lse = _run_eager_and_graph(share)
    # the first and last row of every 256-row unit, the rest drawn at random
    edges = np.unique(np.concatenate([np.arange(0, share.Sq, 256), np.arange(255, share.Sq, 256)]))
    rest = np.setdiff1d(np.arange(share.Sq), edges)
    rows = np.sort(np.concatenate([edges, np.random.default_rng(55).choice(rest, 1024 - len(edges),
                                                                           replace=False)]))
    assert len(rows) == 1024 and (rows < 4096).any() and (rows >= 4096).any()
    say("step longctx oracle on %d rows" % len(rows))
    o_ref, l_ref = _ring_reference(share, rows=rows)
    err = check_pair(host_f64(o[0, rows]), host_f64(lse[0, rows]), o_ref, l_ref, "bf16", "longctx step")
    say("step longctx %d rows: O err %.3e, LSE err %.3e" % (len(rows), err["o_err"], err["lse_err"]))
