"""fp64 CPU oracle: Python side.

TEST INFRASTRUCTURE.  Imported only by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  Shares no code with the HIP
library.

The heavy steps (permute, attention, merge) are plain loops in ``oracle.c``;
this module builds and loads that file, writes out the split and position
definitions, and composes the steps into the Ring, Ulysses-Anything and
Unified passes exactly as the pages describe them.  The attention backward
is written here with numpy float64 matrix products as its steps.

Pages cited (title, then section):
  [CP]  "Context parallelism" (diffusers documentation): "Ring Attention",
        "Ulysses Attention", "Unified Attention", "Ulysses Anything
        Attention", "Ring Anything Attention".
  [USP] "Add Unified Sequence Parallel attention" (diffusers pull request
        #12693), review thread: Ring loop merge of (out, lse); LSE exchanged
        as (B, S, H_LOCAL) in the Unified path.
  [UAA] "UAA: Ulysses Anything Attention" (diffusers issue #12706).
  [YC]  USP / yunchang project summary (sourcepulse): "How It Works",
        "Highlighted Details", "Limitations & Caveats" -- zigzag, stripe and
        basic ring layouts, named but not defined there.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib_handle = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        for name in ("orc_seq2head", "orc_head2seq"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_int, ctypes.c_int, _P, _P, _I64, _I64, _I64,
                           ctypes.c_int, _P, _P]
        lib.orc_seq2head_index.restype = ctypes.c_int
        lib.orc_seq2head_index.argtypes = [ctypes.c_int, ctypes.c_int, _P, _P,
                                           _I64, _I64, _I64, _P, _P]
        lib.orc_attention.restype = ctypes.c_int
        lib.orc_attention.argtypes = [_I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P,
                                      ctypes.c_int, ctypes.c_double, _P, _I64, _P, _P]
        lib.orc_lse_merge.restype = ctypes.c_int
        lib.orc_lse_merge.argtypes = [ctypes.c_int, _I64, _I64, _P, _P, _P, _P]
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_num_threads.argtypes = []
        _lib_handle = lib
    return _lib_handle


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_lib().orc_num_threads())


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ptr_array(arrays: Sequence[np.ndarray]):
    arr = (ctypes.c_void_p * len(arrays))(*[_ptr(a) for a in arrays])
    return arr


# --------------------------------------------------------------------------
# Split of a length over ranks ([UAA]; [CP] "Ulysses Anything Attention").
# The pages only say the length may be anything and that no padding is
# added.  Reading: the first (total mod parts) ranks take one extra element,
# which gives 257 -> 129/128 and 4481 -> 2241/2240; heads split the same way.
# --------------------------------------------------------------------------
def split_offsets(total: int, parts: int) -> list:
    """Exclusive prefix sums [0, n_0, n_0+n_1, ..., total] of the split."""
    if parts < 1 or total < 0:
        raise ValueError("bad split")
    base, extra = divmod(total, parts)
    off = [0]
    for p in range(parts):
        off.append(off[-1] + base + (1 if p < extra else 0))
    return off


# --------------------------------------------------------------------------
# Global token positions of the rows a rank holds ([YC] names the zigzag,
# stripe and basic ring layouts without defining them).  Readings:
#   basic  ("causal"): pos = off + idx  (a contiguous block)
#   zigzag: 2R chunks of length C, rank r holds chunks r and 2R-1-r in that
#           row order, pos = ids[idx // C] * C + idx % C
#   stripe: pos = rank + R * idx
# Causal masking keeps key j for query i iff kpos[j] <= qpos[i].
# --------------------------------------------------------------------------
def positions(desc: Optional[dict], n: int) -> Optional[np.ndarray]:
    if desc is None or desc.get("kind", "full") == "full":
        return None
    kind = desc["kind"]
    idx = np.arange(n, dtype=np.int64)
    if kind == "causal":
        return int(desc.get("off", 0)) + idx
    if kind == "zigzag":
        c = int(desc["chunk"])
        ids = [int(x) for x in desc["ids"]]
        if n > c * len(ids):
            raise ValueError("zigzag side longer than its chunks")
        return np.array([ids[i // c] * c + i % c for i in range(n)], dtype=np.int64)
    if kind == "stripe":
        return int(desc["rank"]) + int(desc["world"]) * idx
    raise ValueError("unknown position kind %r" % kind)


def zigzag_chunks(rank: int, world: int) -> list:
    """Chunk ids held by `rank` of a `world`-rank zigzag ring: r and 2R-1-r."""
    return [rank, 2 * world - 1 - rank]


# --------------------------------------------------------------------------
# Permute (Ulysses all-to-all seen from one rank, run as a local gather).
# --------------------------------------------------------------------------
def _check_offsets(world, seq_off, head_off, H):
    seq_off = np.ascontiguousarray(np.asarray(seq_off, dtype=np.int64))
    head_off = np.ascontiguousarray(np.asarray(head_off, dtype=np.int64))
    if seq_off.shape != (world + 1,) or head_off.shape != (world + 1,):
        raise ValueError("offsets must have world+1 entries")
    if head_off[-1] != H:
        raise ValueError("head offsets must end at H")
    return seq_off, head_off


def seq2head(shards: Sequence[np.ndarray], rank: int, seq_off, head_off) -> np.ndarray:
    """[CP] "Ulysses Attention" first all-to-all, for head-rank `rank`:
    seq shards X_p [B,S_p,H,D] -> Y_r [B,S,H_r,D] (any element dtype)."""
    world = len(shards)
    B, _, H, D = shards[0].shape
    seq_off, head_off = _check_offsets(world, seq_off, head_off, H)
    dt = shards[0].dtype
    shards = [np.ascontiguousarray(s) for s in shards]
    for p, s in enumerate(shards):
        if s.dtype != dt or s.shape != (B, seq_off[p + 1] - seq_off[p], H, D):
            raise ValueError("shard %d has shape %s" % (p, s.shape))
    Hr = int(head_off[rank + 1] - head_off[rank])
    out = np.empty((B, int(seq_off[-1]), Hr, D), dtype=dt)
    rc = _lib().orc_seq2head(rank, world, _ptr(seq_off), _ptr(head_off), B, H, D,
                             dt.itemsize, _ptr_array(shards), _ptr(out))
    if rc != 0:
        raise ValueError("orc_seq2head rejected its arguments")
    return out


def head2seq(heads: Sequence[np.ndarray], rank: int, seq_off, head_off) -> np.ndarray:
    """[CP] "Ulysses Attention" second all-to-all, for seq-rank `rank`:
    head shards Y_r [B,S,H_r,D] -> Z_p [B,S_p,H,D]."""
    world = len(heads)
    B, S, _, D = heads[0].shape
    H = int(np.asarray(head_off)[-1])
    seq_off, head_off = _check_offsets(world, seq_off, head_off, H)
    dt = heads[0].dtype
    heads = [np.ascontiguousarray(x) for x in heads]
    for r, x in enumerate(heads):
        if x.dtype != dt or x.shape != (B, S, head_off[r + 1] - head_off[r], D):
            raise ValueError("head shard %d has shape %s" % (r, x.shape))
    Sp = int(seq_off[rank + 1] - seq_off[rank])
    out = np.empty((B, Sp, H, D), dtype=dt)
    rc = _lib().orc_head2seq(rank, world, _ptr(seq_off), _ptr(head_off), B, H, D,
                             dt.itemsize, _ptr_array(heads), _ptr(out))
    if rc != 0:
        raise ValueError("orc_head2seq rejected its arguments")
    return out


def seq2head_index(rank: int, world: int, seq_off, head_off, B: int, H: int, D: int):
    """Source (shard, flat element) of every element of Y_r, in Y_r's order."""
    seq_off, head_off = _check_offsets(world, seq_off, head_off, H)
    S = int(seq_off[-1])
    Hr = int(head_off[rank + 1] - head_off[rank])
    shard = np.empty((B, S, Hr, D), dtype=np.int64)
    elem = np.empty((B, S, Hr, D), dtype=np.int64)
    rc = _lib().orc_seq2head_index(rank, world, _ptr(seq_off), _ptr(head_off), B, H, D,
                                   _ptr(shard), _ptr(elem))
    if rc != 0:
        raise ValueError("orc_seq2head_index rejected its arguments")
    return shard, elem


# --------------------------------------------------------------------------
# Attention with LSE, by definition (oracle.c orc_attention).
# --------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              qpos: Optional[np.ndarray] = None, kpos: Optional[np.ndarray] = None,
              rows: Optional[Sequence[int]] = None):
    """(O, LSE) of softmax attention; causal by position when qpos/kpos given.

    q [B,Sq,H,D], k/v [B,Sk,H,D], any float dtype (widened to float64).
    rows=None evaluates every query token and returns O [B,Sq,H,D],
    LSE [B,Sq,H]; otherwise rows lists flat tokens b*Sq+i and the result is
    O [n,H,D], LSE [n,H].
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape != (B, Sk, H, D) or v.shape != (B, Sk, H, D):
        raise ValueError("k/v shape mismatch")
    causal = qpos is not None or kpos is not None
    if causal:
        if qpos is None or kpos is None:
            raise ValueError("causal masking needs both position maps")
        qpos = np.ascontiguousarray(qpos, dtype=np.int64)
        kpos = np.ascontiguousarray(kpos, dtype=np.int64)
        if qpos.shape != (Sq,) or kpos.shape != (Sk,):
            raise ValueError("position map length mismatch")
    full = rows is None
    rows_a = np.arange(B * Sq, dtype=np.int64) if full else np.ascontiguousarray(rows, dtype=np.int64)
    n = rows_a.shape[0]
    o = np.empty((n, H, D), dtype=np.float64)
    lse = np.empty((n, H), dtype=np.float64)
    dummy = np.zeros(1, dtype=np.int64)
    rc = _lib().orc_attention(B, Sq, Sk, H, D, _ptr(q), _ptr(k), _ptr(v),
                              _ptr(qpos) if causal else _ptr(dummy),
                              _ptr(kpos) if causal else _ptr(dummy),
                              1 if causal else 0, float(scale), _ptr(rows_a), n, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("orc_attention rejected its arguments")
    if full:
        return o.reshape(B, Sq, H, D), lse.reshape(B, Sq, H)
    return o, lse


def lse_merge(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """Max-shifted N-way LSE merge (oracle.c orc_lse_merge).

    o_parts[n] [..., D], lse_parts[n] [...] with matching leading shapes.
    """
    if len(o_parts) != len(lse_parts) or not o_parts:
        raise ValueError("need matching, non-empty part lists")
    shape = o_parts[0].shape
    D = shape[-1]
    rows = int(np.prod(shape[:-1]))
    os_ = [np.ascontiguousarray(x, dtype=np.float64).reshape(rows, D) for x in o_parts]
    ls_ = [np.ascontiguousarray(x, dtype=np.float64).reshape(rows) for x in lse_parts]
    for x, l in zip(os_, ls_):
        if x.shape != (rows, D) or l.shape != (rows,):
            raise ValueError("part shape mismatch")
    o = np.empty((rows, D), dtype=np.float64)
    lse = np.empty(rows, dtype=np.float64)
    rc = _lib().orc_lse_merge(len(os_), rows, D, _ptr_array(os_), _ptr_array(ls_), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("orc_lse_merge rejected its arguments")
    return o.reshape(shape), lse.reshape(shape[:-1])


# --------------------------------------------------------------------------
# Backward of attention with LSE.  [USP] (pull request conversation): the
# Unified / Ring attention carries a backward (a forward + backward test
# script; the gradient count of the templated Unified attention's backward)
# without writing it out.  Reading: the gradient of the forward above, by
# the chain rule -- what any backward of the same forward must return.
# --------------------------------------------------------------------------
def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, scale: float,
                  qpos: Optional[np.ndarray] = None, kpos: Optional[np.ndarray] = None,
                  dlse: Optional[np.ndarray] = None):
    """Gradients (dQ, dK, dV) of  L = sum(dout * O) + sum(dlse * LSE)  where
    (O, LSE) = attention(q, k, v, scale, qpos, kpos).

    q/dout [B,Sq,H,D], k/v [B,Sk,H,D], dlse [B,Sq,H] or None (zero); all
    widened to float64.  Per (batch, head), with S = scale Q K^T (entries with
    kpos > qpos removed), P = softmax(S) row by row and O = P V:
        dV  = P^T dO
        dP  = dO V^T
        dS  = P * (dP - Delta + dlse),   Delta_i = sum_d dO_id O_id
        dQ  = scale dS K,   dK = scale dS^T Q
    (the softmax Jacobian is diag(P_i) - P_i P_i^T, and d LSE_i / d S_ij =
    P_ij).  Rows with no allowed key have P = 0 and a constant LSE (-inf):
    they add nothing, whatever their dout or dlse.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    do = np.ascontiguousarray(dout, dtype=np.float64)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape != (B, Sk, H, D) or v.shape != (B, Sk, H, D) or do.shape != q.shape:
        raise ValueError("q/k/v/dout shape mismatch")
    if (qpos is None) != (kpos is None):
        raise ValueError("causal masking needs both position maps")
    allowed = np.ones((Sq, Sk), dtype=bool)
    if qpos is not None:
        qpos = np.asarray(qpos, dtype=np.int64)
        kpos = np.asarray(kpos, dtype=np.int64)
        if qpos.shape != (Sq,) or kpos.shape != (Sk,):
            raise ValueError("position map length mismatch")
        allowed = kpos[None, :] <= qpos[:, None]
    dl = np.zeros((B, Sq, H)) if dlse is None else np.asarray(dlse, dtype=np.float64)
    if dl.shape != (B, Sq, H):
        raise ValueError("dlse shape mismatch")
    live = allowed.any(axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h]
            S = np.where(allowed, scale * (Q @ K.T), -np.inf)
            m = np.where(live, S.max(axis=1, initial=-np.inf), 0.0)
            E = np.exp(S - m[:, None])               # exp(-inf) = 0 for removed entries
            P = E / np.where(live, E.sum(axis=1), 1.0)[:, None]
            O = P @ V
            dV = P.T @ dO
            dP = dO @ V.T
            delta = (dO * O).sum(axis=1)
            dS = P * (dP - delta[:, None] + np.where(live, dl[b, :, h], 0.0)[:, None])
            dq[b, :, h] = scale * (dS @ K)
            dk[b, :, h] = scale * (dS.T @ Q)
            dv[b, :, h] = dV
    return dq, dk, dv


# --------------------------------------------------------------------------
# Compositions.
# --------------------------------------------------------------------------
def ring_pass(q, k_chunks, v_chunks, scale, qpos=None, kpos_chunks=None, rows=None):
    """[CP] "Ring Attention": attention of the local queries against each K/V
    block in turn, each block's (O, LSE) folded in with the LSE merge
    ([USP] review thread).  k_chunks/v_chunks: lists of [B,S_c,H,D]."""
    parts_o, parts_l = [], []
    for c, (kc, vc) in enumerate(zip(k_chunks, v_chunks)):
        kp = None if kpos_chunks is None else kpos_chunks[c]
        o, l = attention(q, kc, vc, scale, qpos=qpos if kp is not None else None, kpos=kp, rows=rows)
        parts_o.append(o)
        parts_l.append(l)
    return lse_merge(parts_o, parts_l)


def ring_layout_tokens(S: int, R: int, layout: str) -> list:
    """Global token ids each ring rank holds, in its row order."""
    if layout == "basic":
        off = split_offsets(S, R)
        return [np.arange(off[r], off[r + 1], dtype=np.int64) for r in range(R)]
    if layout == "zigzag":
        if S % (2 * R):
            raise ValueError("zigzag needs S divisible by 2R")
        c = S // (2 * R)
        return [positions({"kind": "zigzag", "chunk": c, "ids": zigzag_chunks(r, R)}, 2 * c)
                for r in range(R)]
    if layout == "stripe":
        if S % R:
            raise ValueError("stripe needs S divisible by R")
        return [positions({"kind": "stripe", "rank": r, "world": R}, S // R) for r in range(R)]
    raise ValueError("unknown layout %r" % layout)


def usp_pass(q, k, v, scale, ulysses: int, ring: int, layout: str = "basic",
             causal: bool = False, seq_splits=None, head_off=None):
    """[CP] "Unified Attention": all-to-all to head-sharded layout, Ring
    attention on the result, then the reverse all-to-all; Ulysses is ring=1
    and Ring is ulysses=1.  With uneven splits this is the Ulysses Anything
    pass ([CP] "Ulysses Anything Attention").

    q, k, v: global [B,S,H,D].  Every rank of the ulysses x ring grid is
    simulated; returns the reassembled global (O [B,S,H,D], LSE [B,S,H]).
    seq_splits: optional per-ring-rank list of Ulysses seq offsets (default
    O1 split of the ring rank's local length); head_off: Ulysses head offsets
    (default O1 split of H).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, H, D = q.shape
    P, R = ulysses, ring
    tokens = ring_layout_tokens(S, R, layout)
    hoff = split_offsets(H, P) if head_off is None else list(head_off)

    # Ulysses gather inside each ring group: [B, S_rho, H_u, D] per (rho, u).
    local = {}
    for rho in range(R):
        t = tokens[rho]
        S_rho = t.shape[0]
        soff = split_offsets(S_rho, P) if seq_splits is None else list(seq_splits[rho])
        for name, x in (("q", q), ("k", k), ("v", v)):
            xl = x[:, t]
            shards = [xl[:, soff[p]:soff[p + 1]] for p in range(P)]
            for u in range(P):
                local[(name, rho, u)] = seq2head(shards, u, soff, hoff)
        local[("soff", rho)] = soff

    o_glob = np.empty((B, S, H, D), dtype=np.float64)
    l_glob = np.empty((B, S, H), dtype=np.float64)
    for rho in range(R):
        o_heads, l_heads = [], []
        for u in range(P):
            kcs = [local[("k", rr, u)] for rr in range(R)]
            vcs = [local[("v", rr, u)] for rr in range(R)]
            qpos = tokens[rho] if causal else None
            kpos = [tokens[rr] for rr in range(R)] if causal else None
            o, l = ring_pass(local[("q", rho, u)], kcs, vcs, scale, qpos=qpos, kpos_chunks=kpos)
            o_heads.append(o)
            l_heads.append(l[..., None])
        soff = local[("soff", rho)]
        o_rows = np.concatenate([head2seq(o_heads, p, soff, hoff) for p in range(P)], axis=1)
        l_rows = np.concatenate([head2seq(l_heads, p, soff, hoff) for p in range(P)], axis=1)
        o_glob[:, tokens[rho]] = o_rows
        l_glob[:, tokens[rho]] = l_rows[..., 0]
    return o_glob, l_glob


def uaa_pass(q, k, v, scale, ulysses: int, causal: bool = False, seq_off=None, head_off=None):
    """[CP] "Ulysses Anything Attention" / [UAA]: the Unified pass with a
    single ring rank and arbitrary (uneven, possibly empty) shards."""
    splits = None if seq_off is None else [seq_off]
    return usp_pass(q, k, v, scale, ulysses, 1, "basic", causal, splits, head_off)
