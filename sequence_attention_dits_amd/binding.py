"""Python binding of libuaa.so: the three calls of include/uaa.h under the
same names, taking torch tensors.

Argument marshalling only: shapes, dtypes and device placement are checked
so that the raw pointers handed to the library always cover what the call
will touch, then the C entry point is called with ``data_ptr()`` values and
the current HIP stream.  Every step of the computation runs in the HIP
kernels; there is no fallback of any kind, and a missing library is an
error.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuaa.so")

UAA_OK = 0
UAA_ERR_INVALID_ARG = -1
UAA_ERR_UNSUPPORTED = -2
UAA_ERR_HIP = -3
UAA_BF16 = 0
UAA_FP32 = 1
UAA_SEQ2HEAD = 0
UAA_HEAD2SEQ = 1
UAA_MAX_WORLD = 64
USP_MAX_PARTS = 16
UAA_MAX_PERMUTE_TENSORS = 4
USP_MASK_FULL = 0
USP_MASK_CAUSAL = 1
USP_MASK_ZIGZAG = 2
USP_MASK_STRIPE = 3
USP_KERNEL_NONE = 0
USP_KERNEL_FP32 = 1
USP_KERNEL_GENERAL = 2
USP_KERNEL_GENERAL_MASKED = 3
USP_KERNEL_GENERAL_SPLIT = 4
USP_KERNEL_PIPELINED = 5
USP_KERNEL_PIPELINED_DIAG = 6
USP_KERNEL_PIPELINED_SPLIT = 7

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p


class usp_mask(ctypes.Structure):
    """Mirror of ``usp_mask`` in include/uaa.h."""
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("world", ctypes.c_int32),
        ("q_off", ctypes.c_int64),
        ("k_off", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
        ("q_chunks", ctypes.c_int32 * 2),
        ("k_chunks", ctypes.c_int32 * 2),
        ("q_rank", ctypes.c_int32),
        ("k_rank", ctypes.c_int32),
    ]


def mask_full() -> usp_mask:
    return usp_mask(kind=USP_MASK_FULL)


def mask_causal(q_off: int = 0, k_off: int = 0) -> usp_mask:
    """Contiguous ("basic") shards: qpos = q_off + i, kpos = k_off + j."""
    return usp_mask(kind=USP_MASK_CAUSAL, q_off=q_off, k_off=k_off)


def mask_zigzag(chunk: int, q_chunks: Sequence[int], k_chunks: Sequence[int]) -> usp_mask:
    """Rows are the listed global chunks (one or two) of length `chunk`."""
    qc = list(q_chunks) + [-1] * (2 - len(q_chunks))
    kc = list(k_chunks) + [-1] * (2 - len(k_chunks))
    m = usp_mask(kind=USP_MASK_ZIGZAG, chunk=chunk)
    m.q_chunks[0], m.q_chunks[1] = qc[0], qc[1]
    m.k_chunks[0], m.k_chunks[1] = kc[0], kc[1]
    return m


def mask_stripe(world: int, q_rank: int, k_rank: int) -> usp_mask:
    """qpos = q_rank + world * i, kpos = k_rank + world * j."""
    return usp_mask(kind=USP_MASK_STRIPE, world=world, q_rank=q_rank, k_rank=k_rank)


class UaaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("libuaa status %d: %s" % (status, message))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libuaa.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libuaa.so is not built (%s); run "
                               "`python -m sequence_attention_dits_amd.build`" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        l.uaa_build_id.restype = ctypes.c_char_p
        l.uaa_build_id.argtypes = []
        _check_build(l.uaa_build_id().decode())
        l.uaa_seq2head_permute.restype = ctypes.c_int
        l.uaa_seq2head_permute.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_p, _c_p,
                                           _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_p, _c_p, _c_p]
        l.uaa_seq2head_permute_multi.restype = ctypes.c_int
        l.uaa_seq2head_permute_multi.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_p,
                                                 _c_p, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_p, _c_p, _c_p]
        l.uaa_seq2head_permute_multi_ex.restype = ctypes.c_int
        l.uaa_seq2head_permute_multi_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_p,
                                                    _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p]
        l.usp_attn_fwd_lse.restype = ctypes.c_int
        l.usp_attn_fwd_lse.argtypes = [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                       _c_p, _c_p, _c_p, _c_p, ctypes.c_int, _c_p,
                                       ctypes.c_float, ctypes.POINTER(usp_mask), _c_p]
        l.usp_attn_fwd_lse_ws.restype = ctypes.c_int
        l.usp_attn_fwd_lse_ws.argtypes = l.usp_attn_fwd_lse.argtypes[:-1] + [_c_p, ctypes.c_size_t, _c_p]
        l.usp_attn_fwd_lse_static.restype = ctypes.c_int
        l.usp_attn_fwd_lse_static.argtypes = l.usp_attn_fwd_lse.argtypes
        l.usp_attn_fwd_lse_acc.restype = ctypes.c_int
        l.usp_attn_fwd_lse_acc.argtypes = l.usp_attn_fwd_lse_ws.argtypes
        l.usp_attn_fwd_lse_gather.restype = ctypes.c_int
        l.usp_attn_fwd_lse_gather.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_p, _c_p, _c_i64, _c_i64,
                                              _c_i64, _c_p, _c_p, _c_p, ctypes.c_int, _c_p, ctypes.c_int, _c_p,
                                              ctypes.c_float, ctypes.POINTER(usp_mask), _c_p, ctypes.c_size_t,
                                              ctypes.c_int, _c_p]
        l.usp_attn_workspace_bytes.restype = ctypes.c_size_t
        l.usp_attn_workspace_bytes.argtypes = [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                               ctypes.POINTER(usp_mask)]
        l.usp_lse_merge.restype = ctypes.c_int
        l.usp_lse_merge.argtypes = [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_int,
                                    _c_p, _c_p, ctypes.c_int, _c_p, _c_p]
        l.usp_attn_bwd_delta.restype = ctypes.c_int
        l.usp_attn_bwd_delta.argtypes = [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p]
        l.usp_attn_bwd.restype = ctypes.c_int
        l.usp_attn_bwd.argtypes = [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p,
                                   _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_int, ctypes.c_float,
                                   ctypes.POINTER(usp_mask), ctypes.c_int, _c_p]
        l.usp_attn_bwd_ws.restype = ctypes.c_int
        l.usp_attn_bwd_ws.argtypes = l.usp_attn_bwd.argtypes[:-1] + [_c_p, ctypes.c_size_t, _c_p]
        l.usp_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        l.usp_attn_bwd_workspace_bytes.argtypes = l.usp_attn_workspace_bytes.argtypes
        l.usp_attn_kernel.restype = ctypes.c_int
        l.usp_attn_kernel.argtypes = [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                      ctypes.POINTER(usp_mask), ctypes.c_size_t]
        l.uaa_split_offsets.restype = ctypes.c_int
        l.uaa_split_offsets.argtypes = [_c_i64, ctypes.c_int, _c_p]
        l.uaa_last_error.restype = ctypes.c_char_p
        l.uaa_last_error.argtypes = []
        l.uaa_abi_version.restype = ctypes.c_int
        l.uaa_abi_version.argtypes = []
        _lib = l
    return _lib


def _check_build(built: str) -> None:
    """The library must have been built from the sources beside it (when
    they are there): a stale build is refused, not run."""
    from . import build
    if not os.path.isdir(build.CSRC):
        return
    want = build.source_id()
    if built != want:
        raise RuntimeError("libuaa.so was built from other sources (build id %s, sources %s); rebuild with "
                           "`python -m sequence_attention_dits_amd.build`" % (built[:12], want[:12]))


def _check(status: int) -> None:
    if status != UAA_OK:
        raise UaaError(status, lib().uaa_last_error().decode(errors="replace"))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _code(dt: torch.dtype, name: str) -> int:
    if dt == torch.bfloat16:
        return UAA_BF16
    if dt == torch.float32:
        return UAA_FP32
    raise ValueError("%s must be bfloat16 or float32, got %s" % (name, dt))


def _i64_array(vals):
    return (ctypes.c_int64 * len(vals))(*[int(x) for x in vals])


def uaa_split_offsets(total: int, parts: int) -> list:
    """The library's default split of `total` items over `parts` ranks, as
    exclusive prefix sums (uaa_split_offsets): what the permute and the
    gathering attention use for the heads when head_off is None."""
    off = (ctypes.c_int64 * (parts + 1))() if parts >= 1 else None
    _check(lib().uaa_split_offsets(int(total), int(parts), off))
    return [int(x) for x in off]


def _head_offsets(head_off, H, world):
    """(offsets used for the shape checks, array handed to the library):
    with head_off None the library splits the heads itself (NULL is passed),
    and the checks use the split it reports."""
    if head_off is None:
        return uaa_split_offsets(H, world), None
    return [int(x) for x in head_off], _i64_array(head_off)


def _permute_shapes(direction, rank, src, dst, seq_off, head_off):
    """Check one tensor's shard shapes against the offsets; returns (B, H, D, head offsets,
    the head_off argument of the library call: NULL when the caller gave none)."""
    world = len(src)
    if len(seq_off) != world + 1:
        raise ValueError("seq_off needs world+1 entries")
    _dev(dst, "dst")
    for x in src:
        _dev(x, "src")
        if x.dtype != dst.dtype or x.device != dst.device:
            raise ValueError("src and dst must share dtype and device")
    if dst.dim() != 4 or any(x.dim() != 4 for x in src):
        raise ValueError("tensors are [B, S, H, D]")
    B, D = dst.shape[0], dst.shape[3]
    S = int(seq_off[-1])
    if direction == UAA_SEQ2HEAD:
        H = src[0].shape[2]
    elif direction == UAA_HEAD2SEQ:
        H = dst.shape[2]
    else:
        raise ValueError("direction must be UAA_SEQ2HEAD or UAA_HEAD2SEQ")
    hoff, harg = _head_offsets(head_off, H, world)
    if len(hoff) != world + 1:
        raise ValueError("head_off needs world+1 entries")
    if direction == UAA_SEQ2HEAD:
        for p, x in enumerate(src):
            if tuple(x.shape) != (B, seq_off[p + 1] - seq_off[p], H, D):
                raise ValueError("src[%d] shape %s does not match the offsets" % (p, tuple(x.shape)))
        if tuple(dst.shape) != (B, S, hoff[rank + 1] - hoff[rank], D):
            raise ValueError("dst shape %s does not match the offsets" % (tuple(dst.shape),))
    else:
        for r, x in enumerate(src):
            if tuple(x.shape) != (B, S, hoff[r + 1] - hoff[r], D):
                raise ValueError("src[%d] shape %s does not match the offsets" % (r, tuple(x.shape)))
        if tuple(dst.shape) != (B, seq_off[rank + 1] - seq_off[rank], H, D):
            raise ValueError("dst shape %s does not match the offsets" % (tuple(dst.shape),))
    return B, H, D, hoff, harg


def uaa_seq2head_permute(direction: int, rank: int, src: Sequence[torch.Tensor], dst: torch.Tensor,
                         seq_off: Sequence[int], head_off: Optional[Sequence[int]] = None) -> None:
    """Ulysses layout change for one rank (include/uaa.h).

    SEQ2HEAD: src[p] [B,S_p,H,D] -> dst [B,S,H_r,D] for head rank `rank`.
    HEAD2SEQ: src[r] [B,S,H_r,D] -> dst [B,S_p,H,D] for token rank `rank`.
    Any element dtype; bits are copied unchanged.
    """
    B, H, D, _, harg = _permute_shapes(direction, rank, src, dst, seq_off, head_off)
    ptrs = (ctypes.c_void_p * len(src))(*[x.data_ptr() if x.numel() else 0 for x in src])
    _check(lib().uaa_seq2head_permute(direction, rank, len(src), _i64_array(seq_off),
                                      harg, B, H, D, dst.element_size(), ptrs,
                                      dst.data_ptr() if dst.numel() else 0, _stream(dst)))


def uaa_seq2head_permute_multi(direction: int, rank: int, srcs: Sequence[Sequence[torch.Tensor]],
                               dsts: Sequence[torch.Tensor], seq_off: Sequence[int],
                               head_off: Optional[Sequence[int]] = None) -> None:
    """The same layout change for several tensors in one launch: srcs[t] are
    tensor t's shards, dsts[t] its destination.  The tensors share B, H and
    the offsets; when they also share D and dtype (e.g. Q, K, V) this is
    uaa_seq2head_permute_multi, otherwise (e.g. O and its LSE)
    uaa_seq2head_permute_multi_ex."""
    if len(srcs) != len(dsts) or not dsts:
        raise ValueError("need one source list per destination")
    shapes = []
    for src, dst in zip(srcs, dsts):
        shapes.append(_permute_shapes(direction, rank, src, dst, seq_off, head_off))
        if (shapes[-1][0], shapes[-1][1], shapes[-1][3]) != (shapes[0][0], shapes[0][1], shapes[0][3]):
            raise ValueError("all tensors of one call must share B, H and the offsets")
    B, H, D, _, harg = shapes[0]
    flat = [x for src in srcs for x in src]
    ptrs = (ctypes.c_void_p * len(flat))(*[x.data_ptr() if x.numel() else 0 for x in flat])
    dptrs = (ctypes.c_void_p * len(dsts))(*[d.data_ptr() if d.numel() else 0 for d in dsts])
    if all(sh[2] == D for sh in shapes) and all(d.dtype == dsts[0].dtype for d in dsts):
        _check(lib().uaa_seq2head_permute_multi(len(dsts), direction, rank, len(srcs[0]), _i64_array(seq_off),
                                                harg, B, H, D, dsts[0].element_size(), ptrs, dptrs,
                                                _stream(dsts[0])))
        return
    Ds = _i64_array([sh[2] for sh in shapes])
    elems = (ctypes.c_int * len(dsts))(*[d.element_size() for d in dsts])
    _check(lib().uaa_seq2head_permute_multi_ex(len(dsts), direction, rank, len(srcs[0]), _i64_array(seq_off),
                                               harg, B, H, Ds, elems, ptrs, dptrs, _stream(dsts[0])))


def attn_workspace(q: torch.Tensor, k: torch.Tensor, mask: Optional[usp_mask] = None) -> Optional[torch.Tensor]:
    """A zero-filled device workspace for usp_attn_fwd_lse(..., workspace=) for
    this problem on q's device, or None when the call would not use one."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k are [B, S, H, D]")
    B, Sq, H, D = q.shape
    m = mask if mask is not None else mask_full()
    with torch.cuda.device(q.device):
        n = lib().usp_attn_workspace_bytes(_code(q.dtype, "q"), B, H, Sq, k.shape[1], D, ctypes.byref(m))
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=q.device)


def usp_attn_kernel(q_shape, sk: int, dtype: torch.dtype = torch.bfloat16, o_dtype: Optional[torch.dtype] = None,
                    mask: Optional[usp_mask] = None, workspace_bytes: int = 0) -> int:
    """USP_KERNEL_* code of the forward kernel a usp_attn_fwd_lse call with
    queries of shape q_shape [B, Sq, H, D] and sk keys would run (host only)."""
    B, Sq, H, D = (int(x) for x in q_shape)
    m = mask if mask is not None else mask_full()
    r = lib().usp_attn_kernel(_code(dtype, "dtype"), B, H, Sq, int(sk), D, _code(o_dtype or dtype, "o_dtype"),
                              ctypes.byref(m), int(workspace_bytes))
    if r < 0:
        _check(r)
    return r


def usp_attn_fwd_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     lse: torch.Tensor, scale: float, mask: Optional[usp_mask] = None,
                     workspace: Optional[torch.Tensor] = None, accumulate: bool = False) -> None:
    """Attention forward with LSE into caller-owned o [B,Sq,H,D], lse [B,Sq,H] fp32.
    With a workspace from attn_workspace() the call is usp_attn_fwd_lse_ws,
    which may split each unit's keys over several workgroups.  With
    accumulate=True it is usp_attn_fwd_lse_acc: (o, lse) hold the running
    result of a Ring pass and this block is merged into them in place."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, k, v are [B, S, H, D] and k, v share a shape")
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
        raise ValueError("k/v shape %s does not match q %s" % (tuple(k.shape), tuple(q.shape)))
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if tuple(o.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Sq, H) or lse.dtype != torch.float32:
        raise ValueError("o must be shaped like q and lse [B, Sq, H] float32")
    dt, odt = _code(q.dtype, "q"), _code(o.dtype, "o")
    m = mask if mask is not None else mask_full()
    if workspace is None and not accumulate:
        _check(lib().usp_attn_fwd_lse(dt, B, H, Sq, Sk, D, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      o.data_ptr(), odt, lse.data_ptr(), float(scale), ctypes.byref(m),
                                      _stream(q)))
        return
    ws_ptr, ws_n = 0, 0
    if workspace is not None:
        _dev(workspace, "workspace")
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor (see attn_workspace)")
        ws_ptr, ws_n = workspace.data_ptr(), workspace.numel()
    fn = lib().usp_attn_fwd_lse_acc if accumulate else lib().usp_attn_fwd_lse_ws
    _check(fn(dt, B, H, Sq, Sk, D, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), odt, lse.data_ptr(),
              float(scale), ctypes.byref(m), ws_ptr, ws_n, _stream(q)))


def usp_attn_fwd_lse_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                            lse: torch.Tensor, scale: float, mask: Optional[usp_mask] = None) -> None:
    """usp_attn_fwd_lse_static: usp_attn_fwd_lse with the key split's
    workspace inside the library (nothing is allocated by the call)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, k, v are [B, S, H, D] and k, v share a shape")
    B, Sq, H, D = q.shape
    if k.shape[0] != B or k.shape[2] != H or k.shape[3] != D or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k/v must match q in batch, heads, features and dtype")
    if tuple(o.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Sq, H) or lse.dtype != torch.float32:
        raise ValueError("o must be shaped like q and lse [B, Sq, H] float32")
    m = mask if mask is not None else mask_full()
    _check(lib().usp_attn_fwd_lse_static(_code(q.dtype, "q"), B, H, Sq, k.shape[1], D, q.data_ptr(), k.data_ptr(),
                                         v.data_ptr(), o.data_ptr(), _code(o.dtype, "o"), lse.data_ptr(),
                                         float(scale), ctypes.byref(m), _stream(q)))


def usp_lse_merge(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor],
                  o_out: torch.Tensor, lse_out: torch.Tensor) -> None:
    """N-way LSE merge of partial (O, LSE) pairs into o_out, lse_out (see
    usp_lse_merge in include/uaa.h): a part whose LSE is -inf for a row has
    weight 0 there, and its O row is not read."""
    n = len(o_parts)
    if n != len(lse_parts) or n < 1:
        raise ValueError("need matching, non-empty part lists")
    _dev(o_out, "o_out")
    _dev(lse_out, "lse_out")
    if o_out.dim() != 4:
        raise ValueError("o tensors are [B, S, H, D]")
    B, S, H, D = o_out.shape
    pdt = _code(o_parts[0].dtype, "o_parts")
    for o, l in zip(o_parts, lse_parts):
        _dev(o, "o_parts")
        _dev(l, "lse_parts")
        if tuple(o.shape) != (B, S, H, D) or o.dtype != o_parts[0].dtype:
            raise ValueError("every o part must be [B, S, H, D] of one dtype")
        if tuple(l.shape) != (B, S, H) or l.dtype != torch.float32:
            raise ValueError("every lse part must be [B, S, H] float32")
    if tuple(lse_out.shape) != (B, S, H) or lse_out.dtype != torch.float32:
        raise ValueError("lse_out must be [B, S, H] float32")
    optr = (ctypes.c_void_p * n)(*[o.data_ptr() for o in o_parts])
    lptr = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lse_parts])
    _check(lib().usp_lse_merge(n, B, S, H, D, optr, pdt, lptr, o_out.data_ptr(),
                               _code(o_out.dtype, "o_out"), lse_out.data_ptr(), _stream(o_out)))


def usp_attn_fwd_lse_gather(rank: int, q_shards: Sequence[torch.Tensor], k_shards: Sequence[torch.Tensor],
                            v_shards: Sequence[torch.Tensor], k_shard: int, o: torch.Tensor, lse: torch.Tensor,
                            scale: float, seq_off: Sequence[int], head_off: Optional[Sequence[int]] = None,
                            mask: Optional[usp_mask] = None, workspace: Optional[torch.Tensor] = None,
                            accumulate: bool = False) -> None:
    """Attention of rank `rank`'s Ulysses view read straight from token shards
    [B, S_p, H, D] (bf16): queries = all tokens, keys = shard k_shard; into
    o [B, S, H_r, D] and lse [B, S, H_r] (usp_attn_fwd_lse_gather)."""
    world = len(q_shards)
    if len(k_shards) != world or len(v_shards) != world or len(seq_off) != world + 1:
        raise ValueError("need world shards of q, k and v and world+1 seq_off entries")
    for t in list(q_shards) + list(k_shards) + list(v_shards):
        _dev(t, "shard")
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError("shards are bf16 [B, S_p, H, D]")
    B, _, H, D = q_shards[0].shape
    S = int(seq_off[-1])
    for p in range(world):
        Sp = int(seq_off[p + 1]) - int(seq_off[p])
        for t in (q_shards[p], k_shards[p], v_shards[p]):
            if tuple(t.shape) != (B, Sp, H, D):
                raise ValueError("shard %d shape %s does not match the offsets" % (p, tuple(t.shape)))
    hoff, harg = _head_offsets(head_off, H, world)
    if len(hoff) != world + 1:
        raise ValueError("head_off needs world+1 entries")
    Hr = hoff[rank + 1] - hoff[rank]
    _dev(o, "o")
    _dev(lse, "lse")
    if tuple(o.shape) != (B, S, Hr, D) or tuple(lse.shape) != (B, S, Hr) or lse.dtype != torch.float32:
        raise ValueError("o must be [B, S, H_r, D] and lse [B, S, H_r] fp32")
    m = mask if mask is not None else mask_full()
    ws_ptr, ws_n = 0, 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_ptr, ws_n = workspace.data_ptr(), workspace.numel()
    ptrs = lambda ts: (ctypes.c_void_p * world)(*[t.data_ptr() if t.numel() else 0 for t in ts])
    _check(lib().usp_attn_fwd_lse_gather(UAA_BF16, world, rank, _i64_array(seq_off), harg, B, H, D,
                                         ptrs(q_shards), ptrs(k_shards), ptrs(v_shards), k_shard, o.data_ptr(),
                                         _code(o.dtype, "o"), lse.data_ptr(), float(scale), ctypes.byref(m),
                                         ws_ptr, ws_n, 1 if accumulate else 0, _stream(o)))


def usp_attn_bwd_delta(o: torch.Tensor, dout: torch.Tensor, delta: torch.Tensor,
                       dlse: Optional[torch.Tensor] = None) -> None:
    """delta [B,S,H] fp32 = rowsum(dout * o) - dlse for o, dout [B,S,H,D]."""
    for t, n in ((o, "o"), (dout, "dout"), (delta, "delta")):
        _dev(t, n)
    if o.dim() != 4 or tuple(dout.shape) != tuple(o.shape) or dout.dtype != o.dtype:
        raise ValueError("o and dout are [B, S, H, D] of one dtype")
    B, S, H, D = o.shape
    if tuple(delta.shape) != (B, S, H) or delta.dtype != torch.float32:
        raise ValueError("delta must be [B, S, H] float32")
    dl = 0
    if dlse is not None:
        _dev(dlse, "dlse")
        if tuple(dlse.shape) != (B, S, H) or dlse.dtype != torch.float32:
            raise ValueError("dlse must be [B, S, H] float32")
        dl = dlse.data_ptr()
    _check(lib().usp_attn_bwd_delta(_code(o.dtype, "o"), B, S, H, D, o.data_ptr(), dout.data_ptr(), dl,
                                    delta.data_ptr(), _stream(o)))


def attn_bwd_workspace_bytes(q: torch.Tensor, k: torch.Tensor, mask: Optional[usp_mask] = None) -> int:
    """Bytes of the dS workspace usp_attn_bwd(..., workspace=) uses for this
    problem (usp_attn_bwd_workspace_bytes; 0: the call does not use one)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k are [B, S, H, D]")
    B, Sq, H, D = q.shape
    m = mask if mask is not None else mask_full()
    return int(lib().usp_attn_bwd_workspace_bytes(_code(q.dtype, "q"), B, H, Sq, k.shape[1], D, ctypes.byref(m)))


def attn_bwd_workspace(q: torch.Tensor, k: torch.Tensor, mask: Optional[usp_mask] = None) -> Optional[torch.Tensor]:
    """A device workspace for usp_attn_bwd(..., workspace=) for this problem
    on q's device (dS of every pair), or None when the call would not use
    one."""
    n = attn_bwd_workspace_bytes(q, k, mask)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def usp_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                 delta: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, scale: float,
                 mask: Optional[usp_mask] = None, accumulate=False, workspace: Optional[torch.Tensor] = None) -> None:
    """Gradients of one attention call (one Ring key block) into caller-owned
    dq [B,Sq,H,D], dk, dv [B,Sk,H,D] (bf16 or float32), from the rows' final
    lse and delta (usp_attn_bwd_delta).  accumulate: False (write all), True
    (add into all three), "dq" (add into dq only) or "dkdv" (into dk, dv).
    With a workspace from attn_bwd_workspace() the call is usp_attn_bwd_ws:
    dq formed from the dS the dK/dV kernel stores there."""
    acc_code = {False: 0, True: 3, "dq": 1, "dkdv": 2}.get(accumulate)
    if acc_code is None:
        raise ValueError("accumulate must be False, True, 'dq' or 'dkdv'")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout"), (lse, "lse"), (delta, "delta"), (dq, "dq"),
                 (dk, "dk"), (dv, "dv")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("q, dout [B, Sq, H, D] and k, v [B, Sk, H, D]")
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
        raise ValueError("k/v shape %s does not match q %s" % (tuple(k.shape), tuple(q.shape)))
    if k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("q, k, v, dout must share a dtype")
    for t, n in ((lse, "lse"), (delta, "delta")):
        if tuple(t.shape) != (B, Sq, H) or t.dtype != torch.float32:
            raise ValueError("%s must be [B, Sq, H] float32" % n)
    if tuple(dq.shape) != tuple(q.shape) or tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(k.shape):
        raise ValueError("dq must be shaped like q and dk, dv like k")
    if dk.dtype != dq.dtype or dv.dtype != dq.dtype:
        raise ValueError("dq, dk, dv must share a dtype")
    m = mask if mask is not None else mask_full()
    args = (_code(q.dtype, "q"), B, H, Sq, Sk, D, q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _code(dq.dtype, "dq"),
            float(scale), ctypes.byref(m), acc_code)
    if workspace is None:
        _check(lib().usp_attn_bwd(*args, _stream(q)))
        return
    _dev(workspace, "workspace")
    _check(lib().usp_attn_bwd_ws(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _stream(q)))
