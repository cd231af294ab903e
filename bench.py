"""Throughput of one rank's share of context-parallel attention on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
resident in HBM, for the FLUX.1-dev 1024x1024 rank share (B=1, S=4608 =
512 text + 4096 image tokens, 24 heads of 128, bf16, Ulysses degree 2, this
rank = head rank 0 / token rank 0):

  1. Ulysses gather (SEQ2HEAD) of Q, K and V from the 2 token shards of 2304
     tokens into this rank's 12 heads over all 4608 tokens, the three
     tensors in one multi-tensor launch                          (1 launch)
  2. attention with LSE of the 4608 queries against the keys/values, taken
     as 2 Ring chunks of 2304                                   (2 launches)
  3. LSE merge of the 2 partial (O, LSE) pairs: by default the Ring-step
     update inside the second chunk's launch (usp_attn_fwd_lse_acc);
     --ring-update merge runs it as its own usp_lse_merge launch
  4. inverse gather (HEAD2SEQ) of O and of the LSE into this rank's token
     shard, both in one launch; the other head rank's shard stands in for
     what the exchange would deliver                            (1 launch)
  (4 launches per step; 5 with --ring-update merge)

value = attention FLOPs of the step (4*D*H*Sq*Sk = 130.46 GFLOP) / step time.
Input sets rotate over more than 4x the 256 MB Infinity Cache so every
step starts from cold HBM.  Each step is captured once per input set as a
HIP graph and replayed (a replay is checked bit for bit against the eager
step first).  Per-kernel times come from HIP events around K back-to-back
launches of each kernel of the step, on the stream the kernels run on; the
HBM-bound ones (permute, merge, inverse gather) read and write buffers of
their own per rotating set, so that neither side stays in the Infinity
Cache.

Other workloads (--workload): flux1008 (the same step on the non-divisible
4481-token UAA share), and two Ring-only shares whose step is one attention
launch per K/V chunk plus the merge: qwen1328 (Qwen-Image 1328x1328, 2
chunks of 3493, then usp_lse_merge) and longctx (32768-token causal zigzag
layout, Q = chunks {1, 6}, 8 chunks of 4096 masked by global position, on
two streams, then one 8-way merge launch).  There `value` counts only the
allowed (query, key) pairs.  The per-kernel figures include the standalone
merge and permute launches whether or not the step uses them.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_BF16_TFLOPS = 2516.6   # dense bf16 matrix (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBPS = 8000.0      # HBM3E

METRIC = "attention TFLOP/s + % bf16 MFMA peak on FLUX-shaped rank share; permute GB/s"

WORKLOADS = {
    # name: (synth config id, description)
    "flux1024": (2, "FLUX.1-dev 1024x1024 Ulysses rank share: S=4608, 12 of 24 heads, D=128, bf16, "
                    "K/V as 2 Ring chunks of 2304, LSE merge, inverse gather"),
    "flux1008": (3, "FLUX.1-dev 1008x1008 UAA rank share: S=4481 (2241/2240), 12 of 24 heads, D=128, bf16, "
                    "K/V as 2 Ring chunks of 2241/2240, LSE merge, inverse gather"),
    "qwen1328": (4, "Qwen-Image 1328x1328 Ring rank share: Q = 3493 of 6986 tokens, 24 heads, D=128, bf16, "
                    "K/V as 2 Ring chunks of 3493, LSE merge"),
    "longctx": (5, "long-context causal zigzag Ring share: S=32768 in 8 chunks of 4096, Q = chunks {1,6}, "
                   "32 heads, D=128, bf16, K/V over all 8 chunks masked by global position, LSE merge of the "
                   "chunks' results (Ring-step update on two streams, 2-way merge of the two running results)"),
}
RING_WORKLOADS = ("qwen1328", "longctx")
# Workloads whose chunk launches run on two streams by default.  Measured:
# the 8 masked long-context launches gain ~5 % (their skipped tiles leave
# compute units idle); the FLUX and Qwen chunks lose 3-6 % (two chunks' K/V
# no longer fit the per-XCD L2 together).
OVERLAP_WORKLOADS = ("longctx",)
# Workloads whose chunk partials are merged by the Ring-step update inside
# the attention launches (usp_attn_fwd_lse_acc) rather than by one N-way
# merge launch: the FLUX shares, where it saves the merge pass, and the
# long-context share (two running results on two streams, merged at the end:
# 1.5-2 % faster than its 8 partials and an 8-way merge on the same box,
# since a partial is written for every query row while the update leaves a
# chunk's rows without an allowed key untouched).  The Qwen share is defined
# with a usp_lse_merge of its 2 partials and keeps it (within ~3 % of the
# accumulating form).
ACC_WORKLOADS = ("flux1024", "flux1008", "longctx")


def make_share(workload: str, n_sets: int, overlap_chunks: str = "auto", ring_update: str = "auto"):
    """The device buffers and launches of one workload's step, in the launch
    configuration the bench times by default ("auto": the per-workload
    stream overlap and Ring-step update above)."""
    cfg_id, _ = WORKLOADS[workload]
    overlap = {"on": True, "off": False}.get(overlap_chunks, workload in OVERLAP_WORKLOADS)
    ring_acc = {"acc": True, "merge": False}.get(ring_update, workload in ACC_WORKLOADS)
    return (RingShare if workload in RING_WORKLOADS else Share)(cfg_id, n_sets, overlap, ring_acc)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="flux1024", choices=sorted(WORKLOADS))
    p.add_argument("--overlap-chunks", choices=["auto", "on", "off"], default="auto",
                   help="run the Ring chunks' attention launches on two streams (auto: per workload)")
    p.add_argument("--ring-update", choices=["auto", "acc", "merge"], default="auto",
                   help="merge the chunk partials inside the attention launches (acc) or with one N-way "
                        "merge launch (auto: per workload)")
    p.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = enough for 1 GiB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernels-only", metavar="NAMES",
                   help="only time the named launch kinds of the step (comma-separated, e.g. attn,attn_acc), "
                        "as the per-kernel figures of the line are timed; for kernel traces")
    p.add_argument("--no-workloads", action="store_true",
                   help="with the default workload, skip the other three workloads' figures")
    p.add_argument("--no-backward", action="store_true", help="skip the backward variant")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--pmc-probe", nargs="?", const="attn", choices=["attn", "hbm", "bwd"],
                   help="only enqueue the dispatches that the counters are read on: a plain device copy of known "
                        "size, then --steps attention launch pairs (attn), or --steps rounds of the HBM-bound "
                        "launches and of plain copies of the same sizes, every one on cold buffers (hbm), or "
                        "--steps backward passes of the step's attention with the dS workspace (bwd)")
    p.add_argument("--hbm-summary", nargs="+", metavar="DIR",
                   help="print the HBM-bound kernels' counter summary from rocprofv3 runs of --pmc-probe hbm: "
                        "--pmc runs (FETCH_SIZE, WRITE_SIZE, ...) and one --kernel-trace --stats run")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="print the traffic summary of two rocprofv3 --pmc runs of --pmc-probe")
    p.add_argument("--stats-summary", metavar="DIR", help="print the summary of a rocprofv3 --stats run")
    p.add_argument("--last", type=int, default=0,
                   help="with --stats-summary: also average each kernel's last N dispatches (the timed launches "
                        "a --kernels-only run reports)")
    p.add_argument("--counter-summary", nargs="+", metavar="DIR",
                   help="print the attention kernel's shader counters from rocprofv3 --pmc runs of --pmc-probe "
                        "(MFMA busy cycles against the active cycles, instruction mix, waits)")
    p.add_argument("--counter-kernels", choices=["attn", "bwd"], default="attn",
                   help="with --counter-summary: the forward attention kernel (attn) or each backward kernel (bwd)")
    return p.parse_args()


class Share:
    """Device buffers of one workload and the launches of one step."""

    def __init__(self, cfg_id: int, n_sets: int, overlap_chunks: bool = False, ring_acc: bool = False):
        import numpy as np
        import torch

        import synth
        import sequence_attention_dits_amd as uaa
        self.uaa = uaa
        self.torch = torch
        self.overlap_chunks = overlap_chunks
        self.ring_acc = ring_acc
        c = synth.CONFIGS[cfg_id]
        self.B, self.S, self.H, self.D = c["B"], c["S"], c["H"], c["D"]
        self.P = 2
        self.seq_off = [0, c["shards"][0], self.S]
        base, extra = divmod(self.H, self.P)
        self.head_off = [0, base + (1 if extra else 0), self.H]
        self.Hr = self.head_off[1]
        self.scale = float(np.float32(1.0 / math.sqrt(self.D)))
        self.ring = [(0, self.seq_off[1]), (self.seq_off[1], self.S)]   # K/V chunks
        self.host = {}
        dev0 = {}
        for t, name in enumerate("qkv"):
            bits, vals = synth.tensor(cfg_id, t, (self.B, self.S, self.H, self.D), "bf16", rms_norm=(name != "v"))
            self.host[name] = vals
            dev0[name] = [torch.from_numpy(np.ascontiguousarray(bits[:, a:b]).view(np.int16)).cuda()
                          .view(torch.bfloat16) for a, b in zip(self.seq_off[:-1], self.seq_off[1:])]
        ob, _ = synth.tensor(cfg_id, 9, (self.B, self.S, self.H - self.Hr, self.D), "bf16")
        dev0["o_other"] = torch.from_numpy(ob.view(np.int16)).cuda().view(torch.bfloat16)
        dev0["l_other"] = torch.from_numpy(
            (8 + synth.normal(cfg_id, 10, (self.B, self.S, self.H - self.Hr, 1))).astype(np.float32)).cuda()
        # rotating copies of the inputs, each in its own allocation
        self.sets = [dev0] + [{k: ([x.clone() for x in v] if isinstance(v, list) else v.clone())
                               for k, v in dev0.items()} for _ in range(n_sets - 1)]
        bf = torch.bfloat16
        B, S, Hr, D, H = self.B, self.S, self.Hr, self.D, self.H
        self.qh = {n: torch.empty(B, S, Hr, D, device="cuda", dtype=bf) for n in "qkv"}
        self.kc = [(self.qh["k"][:, a:b], self.qh["v"][:, a:b]) for a, b in self.ring]
        self.o_part = [torch.empty(B, S, Hr, D, device="cuda", dtype=bf) for _ in self.ring]
        self.l_part = [torch.empty(B, S, Hr, device="cuda", dtype=torch.float32) for _ in self.ring]
        self.o = torch.empty(B, S, Hr, D, device="cuda", dtype=bf)
        self.lse = torch.empty(B, S, Hr, device="cuda", dtype=torch.float32)
        # the chunk launches alternate between two streams (below); each
        # stream has its own split workspace, if the shape asks for one
        self.ws = [_workspace(self.uaa, self.qh["q"], [kc for kc, _ in self.kc], [None] * len(self.kc))
                   for _ in range(2)]
        self.side = torch.cuda.Stream()   # default priority
        S0 = self.seq_off[1]
        self.o_tok = torch.empty(B, S0, H, D, device="cuda", dtype=bf)
        self.l_tok = torch.empty(B, S0, H, 1, device="cuda", dtype=torch.float32)

    def timing_bufs(self, s):
        """Buffers of set s for the per-kernel timing of the HBM-bound
        launches (permute, merge, inverse gather): inputs and outputs both
        rotate with the set, so that those timings read and write HBM and not
        the Infinity Cache.  Allocated on first use; partials hold finite
        values."""
        if not hasattr(self, "_tbufs"):
            self._tbufs = {}
        if s not in self._tbufs:
            torch, bf = self.torch, self.torch.bfloat16
            B, S, Hr, D, H = self.B, self.S, self.Hr, self.D, self.H
            S0 = self.seq_off[1]
            qh = {n: torch.empty(B, S, Hr, D, device="cuda", dtype=bf) for n in "qkv"}
            # the set's gathered Q, K, V hold the real gathered inputs: the
            # attention timing reads them (cold, like the HBM-bound timings)
            d = self.sets[s]
            self.uaa.uaa_seq2head_permute_multi(self.uaa.UAA_SEQ2HEAD, 0, [d[n] for n in "qkv"],
                                                [qh[n] for n in "qkv"], self.seq_off, self.head_off)
            self._tbufs[s] = {
                "qh": qh,
                "o_part": [torch.randn(B, S, Hr, D, device="cuda").to(bf) for _ in self.ring],
                "l_part": [8 + torch.randn(B, S, Hr, device="cuda") for _ in self.ring],
                "o": torch.randn(B, S, Hr, D, device="cuda").to(bf),
                "lse": 8 + torch.randn(B, S, Hr, device="cuda"),
                "o_tok": torch.empty(B, S0, H, D, device="cuda", dtype=bf),
                "l_tok": torch.empty(B, S0, H, 1, device="cuda", dtype=torch.float32),
                "copy": _copy_bufs(torch, {"copy_permute": self.permute_bytes(), "copy_qkv": 3 * self.permute_bytes(),
                                           "copy_merge": self.merge_bytes()}),
            }
        return self._tbufs[s]

    # algorithmic work per launch
    def attn_flops(self, chunk):
        a, b = self.ring[chunk]
        return 4.0 * self.D * self.Hr * self.B * self.S * (b - a)

    def permute_bytes(self):
        return 2.0 * 2 * self.B * self.S * self.Hr * self.D          # read + write, bf16

    def merge_bytes(self):
        rows = self.B * self.S * self.Hr
        per = rows * self.D * 2 + rows * 4                             # bf16 O + fp32 LSE
        return 2 * per + per                                           # N=2 in, 1 out

    def head2seq_lse_bytes(self):
        return 2.0 * 4 * self.B * self.seq_off[1] * self.H

    def head2seq_bytes(self):
        return 2.0 * 2 * self.B * self.seq_off[1] * self.H * self.D

    def launch_one(self, name, s, timing=False):
        """Enqueue the launch(es) of one kind that a step makes on set s;
        returns how many launches were enqueued.  With timing, the HBM-bound
        launches use the set's own buffers (timing_bufs) instead of the
        step's shared intermediates."""
        uaa = self.uaa
        d = self.sets[s]
        t = self.timing_bufs(s) if timing else None
        qh = t["qh"] if timing else self.qh
        o_part, l_part = (t["o_part"], t["l_part"]) if timing else (self.o_part, self.l_part)
        o, lse = (t["o"], t["lse"]) if timing else (self.o, self.lse)
        o_tok, l_tok = (t["o_tok"], t["l_tok"]) if timing else (self.o_tok, self.l_tok)
        if name == "permute":
            uaa.uaa_seq2head_permute(uaa.UAA_SEQ2HEAD, 0, d["q"], qh["q"], self.seq_off, self.head_off)
            return 1
        if name == "permute_qkv":
            uaa.uaa_seq2head_permute_multi(uaa.UAA_SEQ2HEAD, 0, [d[n] for n in "qkv"], [qh[n] for n in "qkv"],
                                           self.seq_off, self.head_off)
            return 1
        if name == "attn":
            for c in range(len(self.kc)):
                self.attn_chunk(s, c, self.ws[0], bufs=t)
            return len(self.kc)
        if name == "attn_acc":   # the accumulating launches of a Ring-step-update pass
            for c in range(1, len(self.kc)):
                self.attn_chunk(s, c, self.ws[0], acc=True, bufs=t)
            return len(self.kc) - 1
        if name == "merge":
            uaa.usp_lse_merge(o_part, l_part, o, lse)
            return 1
        if name == "head2seq":
            uaa.uaa_seq2head_permute(uaa.UAA_HEAD2SEQ, 0, [o, d["o_other"]], o_tok, self.seq_off, self.head_off)
            return 1
        if name == "head2seq_o_lse":
            # O and its LSE back to the token layout in one launch
            uaa.uaa_seq2head_permute_multi(uaa.UAA_HEAD2SEQ, 0, [[o, d["o_other"]], [lse.unsqueeze(-1), d["l_other"]]],
                                           [o_tok, l_tok], self.seq_off, self.head_off)
            return 1
        if name.startswith("copy_"):
            src, dst = t["copy"][name]
            dst.copy_(src)
            return 1
        if name == "copy2d_permute":
            # the runtime's own 2-D copy with the SEQ2HEAD geometry: per source
            # shard, rows of this rank's heads (strided reads) to contiguous rows
            a, b = self.head_off[0], self.head_off[1]
            for p, src in enumerate(d["q"]):
                r0, r1 = self.seq_off[p], self.seq_off[p + 1]
                _memcpy2d(qh["q"][:, r0:r1], src[:, :, a:b], r1 - r0)
            return 1   # one transfer of the permute's bytes
        if name == "copy2d_head2seq":
            # and with the HEAD2SEQ geometry: each rank's head rows (contiguous
            # reads) into their columns of this shard's token rows
            S0 = self.seq_off[1]
            for r, src in enumerate((o, d["o_other"])):
                a, b = self.head_off[r], self.head_off[r + 1]
                _memcpy2d(o_tok[:, :, a:b], src[:, :S0], S0)
            return 1   # one transfer of the inverse gather's bytes
        if name == "head2seq_lse":
            uaa.uaa_seq2head_permute(uaa.UAA_HEAD2SEQ, 0, [lse.unsqueeze(-1), d["l_other"]], l_tok, self.seq_off,
                                     self.head_off)
            return 1
        raise ValueError(name)

    kernel_names = ("permute", "permute_qkv", "attn", "attn_acc", "merge", "head2seq", "head2seq_lse",
                    "head2seq_o_lse")
    # plain device copies of the HBM-bound launches' byte counts (read + write),
    # timed the same way: the reference those launches are measured against
    copy_names = ("copy_permute", "copy_qkv", "copy_merge", "copy2d_permute", "copy2d_head2seq")

    def attn_chunk(self, s, c, ws, acc=False, bufs=None):
        """Chunk c's attention into its partial buffers, or with acc into the
        running (o, lse): chunk 0 writes it, later chunks merge into it.
        With bufs (timing_bufs of set s) every tensor is the set's own."""
        if bufs is None:
            qh, (kc, vc) = self.qh, self.kc[c]
            o, l = (self.o, self.lse) if acc else (self.o_part[c], self.l_part[c])
        else:
            a, b = self.ring[c]
            qh = bufs["qh"]
            kc, vc = qh["k"][:, a:b], qh["v"][:, a:b]
            o, l = (bufs["o"], bufs["lse"]) if acc else (bufs["o_part"][c], bufs["l_part"][c])
        self.uaa.usp_attn_fwd_lse(qh["q"], _contig(kc), _contig(vc), o, l, self.scale, workspace=ws,
                                  accumulate=acc and c > 0)

    def result(self):
        return self.o_tok, self.l_tok

    def step(self, s):
        """Enqueue one step on input set s: the Q/K/V gather, the attention
        of every Ring chunk with the LSE merge of the partials -- with
        ring_acc as the Ring-step update (chunk 0 writes the running (O,
        LSE), each later chunk's launch merges itself into it), otherwise as
        independent launches (alternating between two streams with
        overlap_chunks) followed by one N-way merge launch -- then the
        inverse gather of O and its LSE in one launch."""
        torch = self.torch
        main = torch.cuda.current_stream()
        self._seq2head_qkv(s)
        if self.ring_acc:
            # each chunk merged into the running result as it is computed
            for c in range(len(self.kc)):
                self.attn_chunk(s, c, self.ws[0], acc=True)
        else:
            chunks = [lambda w, c=c: self.attn_chunk(s, c, w) for c in range(len(self.kc))]
            if self.overlap_chunks:
                _two_streams(torch, main, self.side, chunks, self.ws)
            else:
                for fn in chunks:
                    fn(self.ws[0])
            self.launch_one("merge", s)
        self.launch_one("head2seq_o_lse", s)

    def step_fused(self, s):
        """The same step with the Q/K/V gather done inside the attention's
        loads (usp_attn_fwd_lse_gather: queries from both token shards, the
        keys of chunk c = token shard c), the chunks merged by the Ring-step
        update, then the inverse gather: 3 launches."""
        d = self.sets[s]
        for c in range(len(self.ring)):
            self.uaa.usp_attn_fwd_lse_gather(0, d["q"], d["k"], d["v"], c, self.o, self.lse, self.scale,
                                             self.seq_off, self.head_off, workspace=self.ws[0], accumulate=c > 0)
        self.launch_one("head2seq_o_lse", s)

    def _seq2head_qkv(self, s):
        uaa = self.uaa
        d = self.sets[s]
        uaa.uaa_seq2head_permute_multi(uaa.UAA_SEQ2HEAD, 0, [d[n] for n in "qkv"], [self.qh[n] for n in "qkv"],
                                       self.seq_off, self.head_off)


def _two_streams(torch, main, side, launches, ws):
    """Enqueue independent launches alternately on `main` and `side` (fork
    after the work already on `main`, join before anything later on it);
    launch i gets workspace ws[i % 2].  Under graph capture the fork and join
    become graph edges."""
    side.wait_stream(main)
    for i, fn in enumerate(launches):
        if i % 2 == 0:
            fn(ws[0])
        else:
            with torch.cuda.stream(side):
                fn(ws[1])
    main.wait_stream(side)


def _workspace(uaa, q, ks, masks):
    """One attention workspace for every launch of a step (the launches run
    in stream order, so they may share it): the largest any of them asks
    for, or None when none splits its keys."""
    best = None
    for k, m in zip(ks, masks):
        w = uaa.attn_workspace(q, k, m)
        if w is not None and (best is None or w.numel() > best.numel()):
            best = w
    return best


class RingShare:
    """Device buffers and launches of a Ring-only share: the rank's queries
    against every K/V chunk of the ring (one attention launch per chunk, with
    the causal zigzag mask by global position where the layout has one), then
    the N-way LSE merge of the partials."""

    def __init__(self, cfg_id: int, n_sets: int, overlap_chunks: bool = False, ring_acc: bool = False):
        import numpy as np
        import torch

        import synth
        import sequence_attention_dits_amd as uaa
        self.uaa = uaa
        self.torch = torch
        self.overlap_chunks = overlap_chunks
        self.ring_acc = ring_acc
        c = synth.CONFIGS[cfg_id]
        self.B, self.H, self.D = c["B"], c["H"], c["D"]
        self.scale = float(np.float32(1.0 / math.sqrt(self.D)))
        if "chunks" in c:        # zigzag: Q = this rank's two chunks, K/V = every chunk
            n, self.qc = c["chunks"], list(c["q_chunks"])
            self.chunk = c["S"] // n
            self.Sq = self.chunk * len(self.qc)
            self.kv = [(i * self.chunk, (i + 1) * self.chunk) for i in range(n)]
            self.masks = [uaa.mask_zigzag(self.chunk, self.qc, [i]) for i in range(n)]
            q_rows = np.concatenate([np.arange(i * self.chunk, (i + 1) * self.chunk) for i in self.qc])
        else:                    # basic ring: Q = shard 0, K/V = both shards
            sh = c["shards"]
            self.chunk = None
            self.Sq = sh[0]
            self.kv = [(0, sh[0]), (sh[0], sh[0] + sh[1])]
            self.masks = [None, None]
            q_rows = np.arange(sh[0])
        S = c["S"]
        qb, qv = synth.tensor(cfg_id, 0, (self.B, S, self.H, self.D), "bf16", rms_norm=c["rms"])
        kb, kv_ = synth.tensor(cfg_id, 1, (self.B, S, self.H, self.D), "bf16", rms_norm=c["rms"])
        vb, vv = synth.tensor(cfg_id, 2, (self.B, S, self.H, self.D), "bf16", rms_norm=False)
        self.host = {"q": qv[:, q_rows], "k": kv_, "v": vv, "q_rows": q_rows}
        dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).cuda().view(torch.bfloat16)
        d0 = {"q": dev(qb[:, q_rows]), "k": dev(kb), "v": dev(vb)}
        self.sets = [d0] + [{k: v.clone() for k, v in d0.items()} for _ in range(n_sets - 1)]
        bf = torch.bfloat16
        self.o_part = [torch.empty(self.B, self.Sq, self.H, self.D, device="cuda", dtype=bf) for _ in self.kv]
        self.l_part = [torch.empty(self.B, self.Sq, self.H, device="cuda", dtype=torch.float32) for _ in self.kv]
        self.o = torch.empty(self.B, self.Sq, self.H, self.D, device="cuda", dtype=bf)
        self.lse = torch.empty(self.B, self.Sq, self.H, device="cuda", dtype=torch.float32)
        self.ws = [_workspace(uaa, d0["q"], [d0["k"][:, a:b] for a, b in self.kv], self.masks) for _ in range(2)]
        self.side = torch.cuda.Stream()   # default priority
        # allowed (query, key) pairs of each launch, from the position maps,
        # and the query rows with at least one allowed key in each chunk (the
        # others come out of the launch as (0, -inf) and the merge does not
        # read their O)
        self.pairs, self.live = [], []
        for (a, b), m in zip(self.kv, self.masks):
            if m is None:
                self.pairs.append(float(self.Sq) * (b - a))
                self.live.append(np.ones(self.Sq, dtype=bool))
            else:
                cnt = np.searchsorted(np.arange(a, b), q_rows, side="right")
                self.pairs.append(float(cnt.sum()))
                self.live.append(cnt > 0)

    kernel_names = ("attn", "attn_acc", "merge")
    copy_names = ("copy_merge",)

    def attn_flops(self, chunk):
        return 4.0 * self.D * self.H * self.B * self.pairs[chunk]

    def merge_bytes(self):
        """The N-way merge's algorithmic bytes: every partial LSE, the O rows
        of the partials whose chunk has an allowed key for the row (a row
        without one has LSE -inf and weight 0, so its O is not read), and the
        merged (O, LSE)."""
        rows = self.B * self.Sq * self.H
        live_rows = sum(int(l.sum()) for l in self.live) * self.B * self.H
        return live_rows * self.D * 2 + len(self.kv) * rows * 4 + rows * (self.D * 2 + 4)

    def timing_bufs(self, s):
        """Per-set partials and result for the merge timing (see Share); the
        partial LSEs are -inf on the rows a chunk's mask leaves empty, as the
        attention launches leave them."""
        if not hasattr(self, "_tbufs"):
            self._tbufs = {}
        if s not in self._tbufs:
            torch, bf = self.torch, self.torch.bfloat16
            shp = (self.B, self.Sq, self.H)
            dead = [torch.from_numpy(~l).cuda().view(1, -1, 1).expand(*shp) for l in self.live]
            self._tbufs[s] = {
                "o_part": [torch.randn(*shp, self.D, device="cuda").to(bf) for _ in self.kv],
                "l_part": [(8 + torch.randn(*shp, device="cuda")).masked_fill(d, float("-inf")) for d in dead],
                # the running (O, LSE) the accumulating launches merge into: finite
                "o": torch.randn(*shp, self.D, device="cuda").to(bf),
                "lse": 8 + torch.randn(*shp, device="cuda"),
                "copy": _copy_bufs(torch, {"copy_merge": self.merge_bytes()}),
            }
        return self._tbufs[s]

    def launch_one(self, name, s, timing=False):
        uaa = self.uaa
        t = self.timing_bufs(s) if timing else None
        if name == "attn":
            for c in range(len(self.kv)):
                self.attn_chunk(s, c, self.ws[0], into=(t["o_part"][c], t["l_part"][c]) if timing else None)
            return len(self.kv)
        if name == "attn_acc":
            for c in range(1, len(self.kv)):
                self.attn_chunk(s, c, self.ws[0], acc=True, into=(t["o"], t["lse"]) if timing else None)
            return len(self.kv) - 1
        if name.startswith("copy_"):
            src, dst = self.timing_bufs(s)["copy"][name]
            dst.copy_(src)
            return 1
        if name == "merge":
            if timing:
                t = self.timing_bufs(s)
                uaa.usp_lse_merge(t["o_part"], t["l_part"], t["o"], t["lse"])
            else:
                uaa.usp_lse_merge(self.o_part, self.l_part, self.o, self.lse)
            return 1
        raise ValueError(name)

    def attn_chunk(self, s, c, ws, acc=False, into=None, first=None):
        """Chunk c's attention into (O, LSE) `into` (default: its partial
        buffers, or with acc the result); with acc it is merged into what
        `into` holds unless this is the first chunk accumulated there (first;
        default: c == 0)."""
        d = self.sets[s]
        a, b = self.kv[c]
        if into is not None:
            o, l = into
        else:
            o, l = (self.o, self.lse) if acc else (self.o_part[c], self.l_part[c])
        if first is None:
            first = c == 0
        self.uaa.usp_attn_fwd_lse(d["q"], d["k"][:, a:b], d["v"][:, a:b], o, l, self.scale, self.masks[c],
                                  workspace=ws, accumulate=acc and not first)

    def step(self, s):
        """The attention of every chunk with the merge of the partials (see
        Share.step)."""
        torch = self.torch
        if self.ring_acc and self.overlap_chunks:
            # two running results, one per stream (chunks alternate), then
            # the 2-way merge of the two
            runs = [(self.o_part[0], self.l_part[0]), (self.o_part[1], self.l_part[1])]
            chunks = [lambda w, c=c: self.attn_chunk(s, c, w, acc=True, into=runs[c % 2], first=c < 2)
                      for c in range(len(self.kv))]
            _two_streams(torch, torch.cuda.current_stream(), self.side, chunks, self.ws)
            self.uaa.usp_lse_merge([r[0] for r in runs], [r[1] for r in runs], self.o, self.lse)
            return
        if self.ring_acc:
            for c in range(len(self.kv)):
                self.attn_chunk(s, c, self.ws[0], acc=True)
            return
        chunks = [lambda w, c=c: self.attn_chunk(s, c, w) for c in range(len(self.kv))]
        if self.overlap_chunks:
            _two_streams(torch, torch.cuda.current_stream(), self.side, chunks, self.ws)
        else:
            for fn in chunks:
                fn(self.ws[0])
        self.launch_one("merge", s)

    def result(self):
        return self.o, self.lse


def ring_cpu_baseline(share: "RingShare", target_s: float):
    """The fp64 oracle on a sample of query rows of a Ring share: attention
    against every chunk (with the positions of the mask) and the merge."""
    import numpy as np

    import oracle
    oracle.build(force=False)
    h = share.host

    res = {}

    def run(rows):
        t = time.perf_counter()
        parts = []
        for (a, b), m in zip(share.kv, share.masks):
            qpos = kpos = None
            if m is not None:
                qpos, kpos = h["q_rows"], np.arange(a, b)
            parts.append(oracle.attention(h["q"], h["k"][:, a:b], h["v"][:, a:b], share.scale, qpos=qpos,
                                          kpos=kpos, rows=rows))
        res["o"], res["lse"] = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
        return time.perf_counter() - t

    n = 8
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(share.Sq, n, replace=False))
    elapsed = run(rows)
    while elapsed < target_s / 4 and n < share.Sq:
        n = min(share.Sq, int(n * max(2.0, min(8.0, target_s / max(elapsed, 1e-3) / 2))))
        rows = np.sort(rng.choice(share.Sq, n, replace=False))
        elapsed = run(rows)
    o_gpu, l_gpu = _step_result_rows(share, share.o, share.lse, rows)
    # the sample's share of the allowed pairs
    if share.masks[0] is None:
        pairs = float(n) * sum(b - a for a, b in share.kv)
    else:
        qpos = h["q_rows"][rows]
        pairs = float(sum(np.searchsorted(np.arange(a, b), qpos, side="right").sum() for a, b in share.kv))
    flops = 4.0 * share.D * share.H * pairs
    out = {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": "%d of %d query rows x %d heads against all %d K/V chunks + %d-way merge, fp64; %.1f s"
                     % (n, share.Sq, share.H, len(share.kv), len(share.kv), elapsed)}
    out.update(_parity(o_gpu, l_gpu, res["o"], res["lse"], n))
    return out


def _step_result_rows(share, o, lse, rows):
    """Rows `rows` (flat tokens of batch 0) of one fresh eager step's (O, LSE)
    on input set 0, as float64 host arrays [n, H, D] and [n, H]."""
    torch = share.torch
    share.step(0)
    torch.cuda.synchronize()
    idx = torch.as_tensor(rows, device=o.device)
    return (o[0].index_select(0, idx).float().cpu().numpy().astype("float64"),
            lse[0].index_select(0, idx).cpu().numpy().astype("float64"))


def _parity(o_gpu, l_gpu, o_ref, l_ref, n_rows):
    """Largest errors of the GPU step's rows against the oracle's, and
    whether they are inside the bf16 tolerances (O 2e-2, LSE 1e-3 max-abs;
    rows without a key exactly (0, -inf))."""
    import numpy as np
    empty = np.isneginf(l_ref)
    same_empty = bool(np.array_equal(np.isneginf(l_gpu), empty) and (o_gpu[empty] == 0).all())
    o_err = float(np.abs(o_gpu - o_ref).max())
    l_err = float(np.abs(l_gpu[~empty] - l_ref[~empty]).max()) if (~empty).any() else 0.0
    return {"parity_rows": int(n_rows), "max_abs_err_o": o_err, "max_abs_err_lse": l_err,
            "parity_ok": bool(same_empty and o_err <= 2e-2 and l_err <= 1e-3)}


def _backward_setup(share, cfg_id: int):
    """The backward of one step's attention, ready to enqueue: a seeded output
    gradient dO of the step's (O, LSE), delta, dQ and per-chunk dK, dV
    buffers (fp32), one dS workspace for the chunks (their calls run in
    stream order), the largest any of them uses; returns (run, sizes, chunks)
    with run(use_ws) enqueueing delta and usp_attn_bwd per Ring chunk -- the
    first chunk writes dQ, later chunks add into it -- with the workspace
    where use_ws and it applies."""
    import numpy as np

    import synth
    torch, uaa = share.torch, share.uaa
    share.step(0)
    if isinstance(share, RingShare):
        d = share.sets[0]
        q = d["q"]
        chunks = [(d["k"][:, a:b], d["v"][:, a:b], m) for (a, b), m in zip(share.kv, share.masks)]
    else:
        q = share.qh["q"]
        chunks = [(_contig(kc), _contig(vc), None) for kc, vc in share.kc]
    B, Sq, H, D = q.shape
    bits, _ = synth.tensor(cfg_id, 11, (B, Sq, H, D), "bf16")
    dout = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    delta = torch.empty_like(share.lse)
    dq = torch.empty(B, Sq, H, D, device="cuda", dtype=torch.float32)
    dkv = [(torch.empty(k.shape, device="cuda", dtype=torch.float32),
            torch.empty(k.shape, device="cuda", dtype=torch.float32)) for k, _, _ in chunks]
    sizes = [uaa.attn_bwd_workspace_bytes(q, k, m) for k, _, m in chunks]
    ws = torch.empty(max(sizes), dtype=torch.uint8, device="cuda") if max(sizes) > 0 else None

    def run(use_ws):
        uaa.usp_attn_bwd_delta(share.o, dout, delta)
        for c, ((k, v, m), (dk, dv)) in enumerate(zip(chunks, dkv)):
            uaa.usp_attn_bwd(q, k, v, dout, share.lse, delta, dq, dk, dv, share.scale, m,
                             accumulate="dq" if c else False, workspace=ws if use_ws and sizes[c] else None)

    return run, sizes, chunks


def backward_variant(share, cfg_id: int, steps: int, warmup: int) -> dict:
    """The backward of one step's attention (_backward_setup), with the dS
    workspace where it applies (dQ formed from the dS the dK/dV kernel
    stores), and for comparison without it (dQ recomputing the scores).
    Algorithmic FLOPs: 2.5x the forward's (the five products S, dP, dV, dK,
    dQ over the allowed pairs)."""
    torch = share.torch
    run, sizes, chunks = _backward_setup(share, cfg_id)
    ws = max(sizes) > 0

    def timed(use_ws):
        for _ in range(max(warmup, 1)):
            run(use_ws)
        torch.cuda.synchronize()
        # untimed steps right before the timed ones: the GPU is at its working
        # clock when timing starts (an idle GPU lowers it), and the host is
        # ahead of the GPU by their run time
        for _ in range(max(warmup, 1)):
            run(use_ws)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run(use_ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_re = timed(False)
    ms = timed(True) if ws else ms_re
    flops = 2.5 * sum(share.attn_flops(c) for c in range(len(chunks)))
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms, 4), "value": round(tf, 2), "unit": "TFLOP/s",
            "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_step": flops,
            "launches_per_step": 1 + 2 * len(chunks), "grad_dtype": "fp32",
            "dq_from_ds_chunks": sum(1 for n in sizes if n > 0), "ds_workspace_bytes": max(sizes),
            "recompute_ms_per_step": round(ms_re, 4)}


_HIP = None


def _memcpy2d(dst, src, rows):
    """hipMemcpy2DAsync of `rows` rows (B = 1) from the strided view src to
    the strided view dst on the current stream: each row is src.shape[2] x
    src.shape[3] contiguous elements, the pitches are the views' row strides."""
    global _HIP
    import ctypes

    import torch
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipMemcpy2DAsync.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    assert src.shape[0] == 1 and dst.shape[0] == 1 and src.shape[2:] == dst.shape[2:]
    es = src.element_size()
    width = src.shape[2] * src.shape[3] * es
    assert src.stride(3) == 1 and src.stride(2) == src.shape[3] and dst.stride(3) == 1 and dst.stride(2) == dst.shape[3]
    r = _HIP.hipMemcpy2DAsync(ctypes.c_void_p(dst.data_ptr()), dst.stride(1) * es, ctypes.c_void_p(src.data_ptr()),
                              src.stride(1) * es, width, rows, 3,   # hipMemcpyDeviceToDevice
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if r != 0:
        raise RuntimeError("hipMemcpy2DAsync failed: %d" % r)


def _copy_bufs(torch, sizes):
    """Source and destination of a plain device copy per entry, each moving
    `bytes` (half read, half written)."""
    return {k: (torch.ones(int(n) // 8, device="cuda"), torch.empty(int(n) // 8, device="cuda"))
            for k, n in sizes.items()}


def _contig(t):
    # a K/V chunk of the head-sharded tensor is a slice along S: with B = 1 it
    # is already contiguous, so no copy is made here
    return t if t.is_contiguous() else t.contiguous()


def cpu_baseline(share: "Share", target_s: float):
    """The fp64 oracle (as it stands) on a bounded sample of the same step:
    the Ulysses gather of Q, K, V, the two Ring-chunk attentions and the merge
    for a sample of query rows of all 12 heads, and the inverse gather.
    Returns TFLOP/s of attention work on the sample."""
    import numpy as np

    import oracle
    oracle.build(force=False)
    S, H, Hr, D = share.S, share.H, share.Hr, share.D
    t0 = time.perf_counter()
    heads = {}
    for name in "qkv":
        x = share.host[name]
        shards = [x[:, a:b] for a, b in zip(share.seq_off[:-1], share.seq_off[1:])]
        heads[name] = oracle.seq2head(shards, 0, share.seq_off, share.head_off)
    t_perm = time.perf_counter() - t0

    res = {}

    def run(rows):
        t = time.perf_counter()
        parts = [oracle.attention(heads["q"], heads["k"][:, a:b], heads["v"][:, a:b], share.scale, rows=rows)
                 for a, b in share.ring]
        res["o"], res["lse"] = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
        return time.perf_counter() - t

    n = 16
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(S, n, replace=False))
    elapsed = run(rows)
    while elapsed < target_s / 4 and n < S:
        n = min(S, int(n * max(2.0, min(8.0, target_s / max(elapsed, 1e-3) / 2))))
        rows = np.sort(rng.choice(S, n, replace=False))
        elapsed = run(rows)
    # the gather of the whole tensors is pro-rated to the sampled rows
    t_total = elapsed + t_perm * (n / S)
    flops = 4.0 * D * Hr * n * S
    o_gpu, l_gpu = _step_result_rows(share, share.o, share.lse, rows)
    out = {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": "%d of %d query rows x %d heads over all %d keys (2 Ring chunks + merge), fp64, "
                     "plus the Ulysses gather of Q/K/V pro-rated; %.1f s" % (n, S, Hr, S, t_total)}
    out.update(_parity(o_gpu, l_gpu, res["o"], res["lse"], n))
    return out


# ---- HBM traffic of the attention kernel (rocprofv3 counters) ---------------
PMC_COPY_BYTES = 1 << 30              # calibration copy: a plain device-to-device copy of 1 GiB
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_p32_flux1024_hbm_traffic.txt")
ATTN_SOURCES = ["attn_bf16.hip", "attn_p32.hip", "attn_common.h", "internal.h"]


def attn_source_hash():
    """sha256 over the sources the bf16 attention kernel is built from, so that
    counters taken on an older kernel are not reported for a newer one."""
    import hashlib
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "sequence_attention_dits_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _is_attn_fwd(kernel_name):
    """A bf16 attention forward kernel: the pipelined one or the general one."""
    return "attn_p32_kernel" in kernel_name or "attn_bf16_kernel" in kernel_name


# forward kernels by the library's USP_KERNEL_* code (usp_attn_kernel), as
# the kernel traces name them
KERNEL_NAMES = {
    2: "attn_bf16_kernel<128, false, true, false>",
    3: "attn_bf16_kernel<128, true, true, false>",
    4: "attn_bf16_kernel<128, false, true, true>",
    5: "attn_p32_kernel<true, false, false>",
    6: "attn_p32_kernel<true, true, false>",
    7: "attn_p32_kernel<true, false, true>",
}


def attn_kernel_label(share, ring):
    """The forward kernel(s) the timed attention launches run, from the
    library's own choice (usp_attn_kernel); with several, each with its
    launch count."""
    uaa = share.uaa
    names = []
    if ring:
        q = share.sets[0]["q"]
        for (a, b), m in zip(share.kv, share.masks):
            ws = share.ws[0].numel() if share.ws[0] is not None else 0
            names.append(KERNEL_NAMES.get(uaa.usp_attn_kernel(q.shape, b - a, mask=m, workspace_bytes=ws), "?"))
    else:
        ws = share.ws[0].numel() if share.ws[0] is not None else 0
        for a, b in share.ring:
            names.append(KERNEL_NAMES.get(uaa.usp_attn_kernel(share.qh["q"].shape, b - a, workspace_bytes=ws), "?"))
    if len(set(names)) == 1:
        return names[0]
    return " + ".join("%s x%d" % (n, names.count(n)) for n in sorted(set(names), key=names.index))


def pmc_probe(args):
    import torch
    torch.cuda.set_device(0)
    cfg_id, _ = WORKLOADS[args.workload]
    src = torch.ones(PMC_COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    if args.pmc_probe == "hbm":
        hbm_probe(args, cfg_id, src, dst)
        return
    if args.pmc_probe == "bwd":
        run, _, _ = _backward_setup(make_share(args.workload, 1), cfg_id)
        for _ in range(args.steps):
            run(True)
        torch.cuda.synchronize()
        return
    for _ in range(3):
        dst.copy_(src)
    share = Share(cfg_id, 4)
    for i in range(args.steps):
        share.launch_one("attn", i % 4)
    torch.cuda.synchronize()


# The HBM-bound launches of the FLUX-type step whose counters --pmc-probe hbm
# collects, in the order each round enqueues them, then the plain device
# copies of the same byte counts measured beside them.
HBM_PROBE_ORDER = ("permute", "permute_qkv", "head2seq_o_lse", "merge", "copy_1x", "copy_3x", "copy_merge")


def hbm_probe(args, cfg_id, big_src, big_dst):
    """Everything allocated and initialised first; then the calibration
    copies (3 x 1 GiB); then --steps rounds of HBM_PROBE_ORDER: each
    HBM-bound launch of the step on its rotating set's own buffers, and
    plain device copies that read and write the byte counts of one tensor,
    of Q/K/V and of the merge, also rotating -- every dispatch on buffers
    that rotate over more than 1 GiB, so nothing is served from the
    Infinity Cache."""
    import torch
    n_sets = 11
    share = Share(cfg_id, n_sets)
    for s_ in range(n_sets):
        share.timing_bufs(s_)
    sizes = {"copy_1x": share.permute_bytes() / 2, "copy_3x": 3 * share.permute_bytes() / 2,
             "copy_merge": share.merge_bytes() / 2}
    copies = {k: [(torch.ones(int(v) // 4, device="cuda"), torch.empty(int(v) // 4, device="cuda"))
                  for _ in range(n_sets)] for k, v in sizes.items()}
    torch.cuda.synchronize()
    for _ in range(3):
        big_dst.copy_(big_src)
    for i in range(args.steps):
        s_ = i % n_sets
        for name in HBM_PROBE_ORDER:
            if name.startswith("copy"):
                a, b = copies[name][s_]
                b.copy_(a)
            else:
                share.launch_one(name, s_, timing=True)
    torch.cuda.synchronize()


def _hbm_dispatches(d):
    """[(label, {counter: value}, duration_ns)] of the probe rounds in one
    rocprofv3 output directory (counter collection or kernel trace): the
    dispatches after the last calibration copy, labelled by their place in
    the round."""
    import csv
    import glob
    recs = {}
    for pat in ("*counter_collection.csv", "*kernel_trace.csv"):
        for f in glob.glob(os.path.join(d, "**", pat), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    did = int(r["Dispatch_Id"])
                    e = recs.setdefault(did, {"name": r["Kernel_Name"], "c": {},
                                              "ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
                    if "Counter_Name" in r:
                        e["c"][r["Counter_Name"]] = float(r["Counter_Value"])
    order = sorted(recs)
    # the first round: the first two SEQ2HEAD launches followed by a HEAD2SEQ
    # and a merge (the set initialisation before it has no such run)
    sig = ("permute_kernel<0>", "permute_kernel<0>", "permute_kernel<1>", "merge_kernel")
    first = None
    for i in range(len(order) - len(sig)):
        if all(k in recs[order[i + j]]["name"] for j, k in enumerate(sig)):
            first = i
            break
    if first is None:
        return []
    out = []
    for j, did in enumerate(order[first:]):
        e = recs[did]
        out.append((HBM_PROBE_ORDER[j % len(HBM_PROBE_ORDER)], e["c"], e["ns"], e["name"]))
    return out


def hbm_summary(dirs, workload):
    """Per HBM-bound kernel of --pmc-probe hbm and per plain copy of the same
    size: HBM bytes from FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for the 1 GiB calibration copy, against the algorithmic
    bytes; the kernel-trace duration and rate; and the means of every other
    counter the runs hold."""
    import numpy as np
    import synth
    cfg_id, _ = WORKLOADS[workload]
    c = synth.CONFIGS[cfg_id]
    B, S, H, D = c["B"], c["S"], c["H"], c["D"]
    Hr, S0 = (H + 1) // 2, c["shards"][0]
    perm = 2.0 * 2 * B * S * Hr * D
    rows = B * S * Hr
    merge = 3.0 * (rows * D * 2 + rows * 4)
    algo = {"permute": perm, "permute_qkv": 3 * perm,
            "head2seq_o_lse": 2.0 * 2 * B * S0 * H * D + 2.0 * 4 * B * S0 * H, "merge": merge,
            "copy_1x": perm, "copy_3x": 3 * perm, "copy_merge": merge}
    per = {}       # label -> counter -> [values]
    scale = {}
    for d in dirs:
        # calibration: the 1 GiB copies' FETCH_SIZE / WRITE_SIZE (KiB)
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            big = [v for k, vv in _pmc_values(d, counter).items() if "copy" in k.lower() for v in vv
                   if v * 1024 > PMC_COPY_BYTES / 4]
            if big:
                scale[counter] = PMC_COPY_BYTES / (1024 * float(np.mean(big)))
        for label, cs, ns, name in _hbm_dispatches(d):
            for k, v in cs.items():
                per.setdefault(label, {}).setdefault(k, []).append(v)
            if not cs:
                per.setdefault(label, {}).setdefault("duration_ns", []).append(ns)
    cmd = "python3 bench.py --pmc-probe hbm --steps 40"
    lines = [
        "rocprofv3 counter summary: the HBM-bound kernels of the %s step (the single-tensor and Q/K/V" % workload,
        "SEQ2HEAD permutes, the O+LSE HEAD2SEQ, the N=2 LSE merge) and plain device copies of the same byte",
        "counts (hipMemcpy device to device), every dispatch on buffers that rotate over more than 1 GiB",
        "",
        "commands (run from the repository root on one MI355X; one counter group per run):",
        "  rocprofv3 --kernel-trace --stats -d gpurun_out/hbm_trace -o hbm --output-format csv -- " + cmd,
        "  rocprofv3 --pmc FETCH_SIZE -d gpurun_out/hbm_fetch -o pmc --output-format csv -- " + cmd,
        "  rocprofv3 --pmc WRITE_SIZE GRBM_GUI_ACTIVE -d gpurun_out/hbm_write -o pmc --output-format csv -- " + cmd,
        "  (further --pmc groups as listed below)",
        "  python3 bench.py --hbm-summary " + " ".join(dirs),
        "",
        "calibration (1 GiB copy): FETCH_SIZE scale %s, WRITE_SIZE scale %s" % (
            "%.4f" % scale["FETCH_SIZE"] if "FETCH_SIZE" in scale else "n/a",
            "%.4f" % scale["WRITE_SIZE"] if "WRITE_SIZE" in scale else "n/a"),
        "",
        "%-16s %9s %9s %9s %10s %8s %8s %6s" % ("dispatch", "algo_MB", "fetch_MB", "write_MB", "traffic/x",
                                               "avg_us", "GB/s", "n"),
    ]
    for label in HBM_PROBE_ORDER:
        g = per.get(label, {})
        f = float(np.mean(g["FETCH_SIZE"])) * 1024 * scale["FETCH_SIZE"] if "FETCH_SIZE" in g and \
            "FETCH_SIZE" in scale else float("nan")
        w = float(np.mean(g["WRITE_SIZE"])) * 1024 * scale["WRITE_SIZE"] if "WRITE_SIZE" in g and \
            "WRITE_SIZE" in scale else float("nan")
        us = float(np.mean(g["duration_ns"])) / 1e3 if "duration_ns" in g else float("nan")
        n = len(g.get("duration_ns", g.get("FETCH_SIZE", [])))
        lines.append("%-16s %9.2f %9.2f %9.2f %10.3f %8.2f %8.1f %6d" % (
            label, algo[label] / 1e6, f / 1e6, w / 1e6, (f + w) / algo[label], us, algo[label] / (us * 1e3), n))
    others = sorted({k for g in per.values() for k in g} - {"FETCH_SIZE", "WRITE_SIZE", "duration_ns"})
    if others:
        lines += ["", "other counters, mean per dispatch (columns in the order above):"]
        for k in others:
            lines.append("  %-40s %s" % (k, " ".join("%10.4g" % float(np.mean(per.get(lb, {}).get(k, [float("nan")])))
                                                     for lb in HBM_PROBE_ORDER)))
    print("\n".join(lines))


def _pmc_values(d, counter):
    """{kernel name: [per-dispatch values]} of one counter from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out



def pmc_summary(fetch_dir, write_dir, workload):
    """Per-dispatch HBM bytes of the attention kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for the calibration copy of PMC_COPY_BYTES."""
    res = {}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        vals = _pmc_values(d, counter)
        copy = sorted(v for k, vs in vals.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs)
        copy = [v for v in copy if v * 1024 > PMC_COPY_BYTES / 4]
        attn = [v for k, vs in vals.items() if _is_attn_fwd(k) for v in vs]
        if not copy or not attn:
            raise SystemExit("no calibration copy or attention dispatch in " + d)
        scale = PMC_COPY_BYTES / (1024 * sum(copy) / len(copy))
        res[key] = (sum(copy) / len(copy), scale, sum(attn) / len(attn), len(attn))
    cfg_id, desc = WORKLOADS[workload]
    import synth
    c = synth.CONFIGS[cfg_id]
    Hr = (c["H"] + 1) // 2
    sq, sk = c["S"], c["shards"][0]
    algo = 2 * c["B"] * Hr * c["D"] * (2 * sq + 2 * sk) + 4 * c["B"] * sq * Hr
    traffic = res["fetch"][1] * res["fetch"][2] * 1024 + res["write"][1] * res["write"][2] * 1024
    lines = [
        "rocprofv3 counter summary: HBM traffic of the bf16 attention kernel, one Ring-chunk launch of the",
        "%s step (Sq=%d, Sk=%d, %d heads, D=%d)" % (workload, sq, sk, Hr, c["D"]),
        "",
        "commands (run from the repository root on one MI355X):",
        "  rocprofv3 --pmc FETCH_SIZE -d %s -o pmc --output-format csv -- python3 bench.py --pmc-probe" % fetch_dir,
        "  rocprofv3 --pmc WRITE_SIZE -d %s -o pmc --output-format csv -- python3 bench.py --pmc-probe" % write_dir,
        "  python3 bench.py --pmc-summary %s %s" % (fetch_dir, write_dir),
        "",
        "calibration: plain device copy of %d bytes" % PMC_COPY_BYTES,
        "  FETCH_SIZE %.1f KiB per copy -> scale %.4f;  WRITE_SIZE %.1f KiB per copy -> scale %.4f"
        % (res["fetch"][0], res["fetch"][1], res["write"][0], res["write"][1]),
        "attention (%d dispatches): FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB per dispatch"
        % (res["fetch"][3], res["fetch"][2], res["write"][2]),
        "algorithmic_bytes_per_launch: %d   (Q, K, V read once, O and LSE written once)" % algo,
        "traffic_bytes_per_launch: %d" % round(traffic),
        "traffic_over_algorithmic: %.3f" % (traffic / algo),
        "source_sha256: %s" % attn_source_hash(),
    ]
    print("\n".join(lines))


def measured_traffic():
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(": ", 1) for line in f.read().splitlines() if ": " in line)
        if kv.get("source_sha256", "").strip() != attn_source_hash():
            return None
        return int(kv["traffic_bytes_per_launch"].split()[0])
    except (OSError, KeyError, ValueError):
        return None


SIMDS = 256 * 4   # MI355X: 256 compute units of 4 SIMDs, in 8 XCDs


def counter_summary(dirs, which: str = "attn"):
    """Means per dispatch of every counter in the given rocprofv3 --pmc runs,
    for the bf16 attention forward kernel (which="attn") or for each
    backward kernel (which="bwd"), and the matrix-core utilisation they
    imply: busy cycles of the matrix units over (active cycles of one XCD x
    all SIMDs), where GRBM_GUI_ACTIVE is summed over the 8 XCDs."""
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for counter in ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                        "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES",
                        "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT"):
            for k, vs in _pmc_values(d, counter).items():
                if which == "attn" and _is_attn_fwd(k):
                    vals["attention forward"][counter].extend(vs)
                elif which == "bwd" and "attn_bwd_" in k and "delta" not in k:
                    vals[k.replace("void ", "").split("(")[0]][counter].extend(vs)
    if not vals:
        raise SystemExit("no %s dispatch in %s" % (which, " ".join(dirs)))
    for name in sorted(vals):
        mean = {k: sum(v) / len(v) for k, v in vals[name].items()}
        if which == "bwd":
            print("\n%s" % name)
        print("%-28s %10s %16s" % ("counter", "dispatches", "mean per dispatch"))
        for k in sorted(mean):
            print("%-28s %10d %16.4g" % (k, len(vals[name][k]), mean[k]))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "GRBM_GUI_ACTIVE" in mean:
            cyc = mean["GRBM_GUI_ACTIVE"] / 8
            print("active cycles per XCD: %.4g" % cyc)
            print("matrix-core busy / (active cycles x %d SIMDs): %.3f" %
                  (SIMDS, mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS)))
            if "SQ_INSTS_MFMA" in mean:
                print("busy cycles per matrix instruction: %.2f" % (mean["SQ_VALU_MFMA_BUSY_CYCLES"] / mean["SQ_INSTS_MFMA"]))
        if "SQ_WAIT_INST_ANY" in mean and "SQ_WAVE_CYCLES" in mean:
            print("wave time waiting on a dependency: %.3f" % (mean["SQ_WAIT_INST_ANY"] / mean["SQ_WAVE_CYCLES"]))
        if "SQ_INSTS_LDS" in mean and "SQ_INSTS_MFMA" in mean:
            print("LDS instructions per matrix instruction: %.2f" % (mean["SQ_INSTS_LDS"] / mean["SQ_INSTS_MFMA"]))


def stats_summary(d, last: int = 0):
    """Kernel table of a rocprofv3 --kernel-trace --stats run (its
    *_kernel_stats.csv); with last > 0 also the average of each kernel's
    last `last` dispatches (its *_kernel_trace.csv): the timed launches of a
    --kernels-only run of one launch kind."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_stats.csv under " + d)
    rows = list(csv.DictReader(open(files[0])))
    print("%-70s %6s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us"))
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"] if len(r["Name"]) <= 70 else r["Name"][:67] + "..."
        print("%-70s %6d %12.2f %12.2f %12.2f" % (name, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                                                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if last > 0 and traces:
        by = {}
        for r in csv.DictReader(open(traces[0])):
            by.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        print("\nlast %d dispatches of each kernel (the timed launches of --kernels-only):" % last)
        print("%-70s %6s %12s" % ("kernel", "calls", "avg_us"))
        for name, ts in sorted(by.items(), key=lambda kv: -sum(e - b for b, e in kv[1])):
            if len(ts) < last:
                continue
            ts.sort()
            tail = ts[-last:]
            nm = name if len(name) <= 70 else name[:67] + "..."
            print("%-70s %6d %12.2f" % (nm, len(tail), sum(e - b for b, e in tail) / len(tail) / 1e3))
        # a launch kind that runs several attention kernels (the masked Ring
        # pass: plain and DIAG forms): its last N attention dispatches together
        att = sorted(t for name, ts in by.items() if _is_attn_fwd(name) for t in ts)
        if len(att) >= last and len([n for n in by if _is_attn_fwd(n)]) > 1:
            tail = att[-last:]
            print("%-70s %6d %12.2f" % ("(every attention-forward kernel together)", len(tail),
                                        sum(e - b for b, e in tail) / len(tail) / 1e3))


TIMED_MS = 20.0   # least GPU time of one launch kind's timed region


def time_launches(share, names, steps: int, n_sets: int, counts: dict = None) -> dict:
    """Per-launch microseconds of each named launch kind of the step: `steps`
    rounds back to back over the rotating sets, every launch on its set's own
    buffers (timing_bufs: inputs and outputs cold).  The rounds of one kind
    are captured in a HIP graph, replayed once untimed and then, between two
    HIP events, as many times as fill TIMED_MS: no launch waits on the host
    (the short HBM-bound kernels take less time than a host-side launch), the
    GPU is busy at its working clock when timing starts (an idle GPU, or one
    running a spin kernel, lowers it), and the average spans the swings of
    its power management (a few milliseconds each).  counts, if given,
    receives each kind's (untimed, timed) launch counts."""
    torch = share.torch
    for s_ in range(n_sets):   # allocated before capture
        share.timing_bufs(s_)
    torch.cuda.synchronize()
    log = {}
    for name in names:
        g = torch.cuda.CUDAGraph()
        n = 0
        with torch.cuda.graph(g):
            for i in range(steps):
                n += share.launch_one(name, i % n_sets, timing=True)
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        a_ev = torch.cuda.Event(enable_timing=True)
        b_ev = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0.record()
        g.replay()
        w1.record()
        torch.cuda.synchronize()
        reps = max(1, int(math.ceil(TIMED_MS / max(w0.elapsed_time(w1), 1e-3))))
        g.replay()   # keeps the GPU busy while the timed replays are queued
        a_ev.record()
        for _ in range(reps):
            g.replay()
        b_ev.record()
        torch.cuda.synchronize()
        log[name] = 1e3 * a_ev.elapsed_time(b_ev) / (n * reps)
        if counts is not None:
            counts[name] = (2 * n, n * reps)
        del g
    return log


def n_sets_for(workload: str) -> int:
    """Rotating input sets whose inputs exceed 1 GiB (over 4x the 256 MB
    Infinity Cache), at least 2."""
    import synth
    c = synth.CONFIGS[WORKLOADS[workload][0]]
    if workload in RING_WORKLOADS:
        sq = c["S"] // c["chunks"] * len(c["q_chunks"]) if "chunks" in c else c["shards"][0]
        per_set = (sq + 2 * c["S"]) * c["B"] * c["H"] * c["D"] * 2
    else:
        per_set = 3 * c["B"] * c["S"] * c["H"] * c["D"] * 2 + c["B"] * c["S"] * (c["H"] // 2) * c["D"] * 2
    return max(2, int(math.ceil((1 << 30) / per_set)))


def kernels_only(args):
    """--kernels-only: only the per-launch timing of the named launch kinds
    (the same loop that gives the bench line's per-kernel figures), so that a
    kernel trace of this command averages exactly those launches."""
    share = make_share(args.workload, args.sets or n_sets_for(args.workload))
    names = [n for n in args.kernels_only.split(",") if n]
    kinds = share.kernel_names + share.copy_names
    for n in names:
        if n not in kinds:
            raise SystemExit("unknown launch kind %r (one of %s)" % (n, ", ".join(kinds)))
    share.step(0)
    counts = {}
    log = time_launches(share, names, args.steps, len(share.sets), counts)
    print(json.dumps({"workload": args.workload, "steps": args.steps, "us_per_launch": log,
                      "launches_untimed_timed": counts}), flush=True)


def measure(args, workload: str, steps: int, warmup: int, full: bool) -> dict:
    """Build one workload's step, time it (graph replays) and its launches
    (back to back, cold), run the oracle baseline on a sample and compare
    its rows with the GPU step; the variants (fused gather, backward) and
    the command-line overrides of the launch configuration only with full."""
    import torch
    cfg_id, desc = WORKLOADS[workload]
    import synth
    c = synth.CONFIGS[cfg_id]
    ring = workload in RING_WORKLOADS
    n_sets = (args.sets if full else 0) or n_sets_for(workload)
    share = make_share(workload, n_sets, args.overlap_chunks if full else "auto", args.ring_update if full else "auto")

    for i in range(max(warmup, 1)):
        share.step(i % n_sets)
    torch.cuda.synchronize()

    # One HIP graph per input set: replaying a captured step keeps host launch
    # overhead out of the step time.
    graphs = []
    for s_ in range(n_sets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            share.step(s_)
        graphs.append(g)
    torch.cuda.synchronize()
    # replay check: a replay must reproduce the eager step bit for bit
    share.step(0)
    torch.cuda.synchronize()
    ref_o, ref_l = (t.clone() for t in share.result())
    graphs[1 % n_sets].replay()
    graphs[0].replay()
    torch.cuda.synchronize()
    out_o, out_l = share.result()
    replay_ok = bool(torch.equal(ref_o.view(torch.int16), out_o.view(torch.int16)) and torch.equal(ref_l, out_l))
    if not replay_ok:
        print("graph replay differs from the eager step", file=sys.stderr)
        sys.exit(1)

    # W warm-up replays right before the timed region (only the
    # synchronisation between them): the GPU is at its working clock when
    # timing starts
    for i in range(warmup):
        graphs[i % n_sets].replay()
    torch.cuda.synchronize()

    # timed region 1: K graph replays (ms_per_step, value)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        graphs[i % n_sets].replay()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps

    # the fused-gather variant of the FLUX-type step (SEQ2HEAD inside the
    # attention's loads), checked bit for bit against the step above
    variants = {}
    if full and not ring:
        share.step(0)
        torch.cuda.synchronize()
        ref_o, ref_l = (t.clone() for t in share.result())
        share.step_fused(0)
        torch.cuda.synchronize()
        out_o, out_l = share.result()
        same = bool(torch.equal(ref_o.view(torch.int16), out_o.view(torch.int16)) and torch.equal(ref_l, out_l))
        fgraphs = []
        for s_ in range(n_sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                share.step_fused(s_)
            fgraphs.append(g)
        for i in range(warmup):
            fgraphs[i % n_sets].replay()
        torch.cuda.synchronize()
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        f0.record()
        for i in range(steps):
            fgraphs[i % n_sets].replay()
        f1.record()
        torch.cuda.synchronize()
        ms_fused = f0.elapsed_time(f1) / steps
        variants["fused_gather"] = {
            "ms_per_step": round(ms_fused, 4),
            "value": round(sum(share.attn_flops(c_) for c_ in range(len(share.ring))) / (ms_fused * 1e-3) / 1e12, 2),
            "launches_per_step": 3,
            "equals_default_step_bitwise": same,
        }
        del fgraphs

    # the backward of the step's attention (usp_attn_bwd_delta + usp_attn_bwd)
    if full and not args.no_backward:
        variants["backward"] = backward_variant(share, cfg_id, steps, warmup)

    # timed region 2: per-kernel durations.  Each launch of the step is
    # repeated back to back over the rotating input sets, captured in a HIP
    # graph replayed untimed and then between two HIP events (time_launches).
    log = time_launches(share, share.kernel_names + share.copy_names, steps, n_sets)

    n_attn = len(share.kv) if ring else len(share.ring)
    attn_flops = sum(share.attn_flops(c_) for c_ in range(n_attn))
    value = attn_flops / (ms_step * 1e-3) / 1e12
    attn_us = log["attn"]
    attn_flops_launch = attn_flops / n_attn
    attn_tf = attn_flops_launch / (attn_us * 1e-6) / 1e12
    merge_us = log["merge"]
    merge_gbps = share.merge_bytes() / (merge_us * 1e-6) / 1e9
    def vs_copy(us, name):
        # the same bytes moved by a plain device copy, timed the same way
        c = log[name]
        return {"copy_us": round(c, 2), "frac_of_copy": round(c / us, 4)}

    def vs_copy2d(us, name):
        # the same transfer, same geometry, by the runtime's 2-D copy
        c = log[name]
        return {"copy2d_us": round(c, 2), "frac_of_copy2d": round(c / us, 4)}

    kernels = {
        "lse_merge": {"us": round(merge_us, 2), "GB/s": round(merge_gbps, 1),
                      "hbm_frac": round(merge_gbps / PEAK_HBM_GBPS, 4), "bytes": share.merge_bytes(),
                      **vs_copy(merge_us, "copy_merge")},
        "attention": {"us": round(attn_us, 2), "TFLOP/s": round(attn_tf, 2),
                      "mfma_frac": round(attn_tf / PEAK_BF16_TFLOPS, 4)},
        "attention_acc": {"us": round(log["attn_acc"], 2)},
    }
    if ring:
        config = {"workload": desc, "B": share.B, "Sq": share.Sq, "heads": share.H, "D": share.D,
                  "ring_chunks": n_attn, "attn_flops_per_step": attn_flops}
    else:
        perm_us = log["permute"]
        perm_gbps = share.permute_bytes() / (perm_us * 1e-6) / 1e9
        h2s_us = log["head2seq"]
        qkv_us = log["permute_qkv"]
        qkv_gbps = 3 * share.permute_bytes() / (qkv_us * 1e-6) / 1e9
        h2s_gbps = share.head2seq_bytes() / (h2s_us * 1e-6) / 1e9
        kernels.update({
            "seq2head_permute": {"us": round(perm_us, 2), "GB/s": round(perm_gbps, 1),
                                 "hbm_frac": round(perm_gbps / PEAK_HBM_GBPS, 4), "bytes": share.permute_bytes(),
                                 **vs_copy(perm_us, "copy_permute"), **vs_copy2d(perm_us, "copy2d_permute")},
            "seq2head_permute_qkv": {"us": round(qkv_us, 2), "GB/s": round(qkv_gbps, 1),
                                     "hbm_frac": round(qkv_gbps / PEAK_HBM_GBPS, 4),
                                     "bytes": 3 * share.permute_bytes(), **vs_copy(qkv_us, "copy_qkv")},
            "head2seq_permute": {"us": round(h2s_us, 2), "GB/s": round(h2s_gbps, 1),
                                 "hbm_frac": round(h2s_gbps / PEAK_HBM_GBPS, 4), "bytes": share.head2seq_bytes(),
                                 **vs_copy(h2s_us, "copy_permute"), **vs_copy2d(h2s_us, "copy2d_head2seq")},
            "head2seq_permute_o_lse": {"us": round(log["head2seq_o_lse"], 2),
                                       "bytes": share.head2seq_bytes() + share.head2seq_lse_bytes()},
        })
        config = {"workload": desc, "B": share.B, "S": share.S, "heads_total": share.H, "heads_rank": share.Hr,
                  "D": share.D, "ulysses": share.P, "ring_chunks": n_attn, "attn_flops_per_step": attn_flops}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), Q/K RMS-normalised per head where the workload says so; inputs "
                "resident in HBM, %d rotating sets)" % n_sets,
        "config": config,
        "roofline": {"bound": "mfma", "achieved": round(attn_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic() if workload == "flux1024" else None,
                     "kernel": attn_kernel_label(share, ring),
                     "launch_us": round(attn_us, 2), "flops_per_launch": attn_flops_launch},
        "kernels": kernels,
    }
    if variants:
        out["variants"] = variants
    if not ring:
        out["permute_GBps"] = kernels["seq2head_permute"]["GB/s"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (ring_cpu_baseline if ring else cpu_baseline)(
            share, args.cpu_seconds if full else args.cpu_seconds / 3)
    del graphs, share
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload)
        return
    if args.hbm_summary:
        hbm_summary(args.hbm_summary, args.workload)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary, args.last)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.counter_kernels)
        return
    if args.gpus != 1:
        print("bench.py measures one rank's share on one GPU; --gpus %d is not supported "
              "(the library has no collective or multi-GPU path)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.pmc_probe:
        pmc_probe(args)
        return
    if args.kernels_only:
        kernels_only(args)
        return
    out = measure(args, args.workload, args.steps, args.warmup, True)
    if args.workload == "flux1024" and not args.no_workloads:
        # the other workloads in their default launch configuration, each
        # with its own oracle sample (the driver's one line carries all five)
        out["workloads"] = {}
        for w in ("flux1008", "qwen1328", "longctx"):
            r = measure(args, w, min(args.steps, 20), args.warmup, False)
            out["workloads"][w] = {k: r[k] for k in ("value", "unit", "ms_per_step", "steps", "config", "roofline",
                                                      "kernels", "cpu_baseline") if k in r}
        out["workloads_note"] = ("the tiny ragged fp32 share (257 tokens, 129/128) is a correctness case: every "
                                 "row is checked in the GPU tests, it is not timed")
    out["library"] = library_record()
    print(json.dumps(out), flush=True)


def library_record() -> dict:
    """Which native library this run called: its file and the build id
    compiled into it (sha256 of the csrc sources and build flags; the binding
    refuses a library whose id differs from the sources beside it)."""
    from sequence_attention_dits_amd import binding, build
    lib = binding.lib()
    return {"file": os.path.relpath(lib._name, os.path.dirname(os.path.abspath(__file__))),
            "build_id": lib.uaa_build_id().decode(), "sources_id": build.source_id(),
            "kernel_arch": build.ARCH}


if __name__ == "__main__":
    main()
