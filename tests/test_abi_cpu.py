"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/uaa.h declares, agrees with the binding on the mask
struct layout, and rejects malformed arguments with the documented status
before anything reaches the HIP runtime."""

import ctypes
import os
import re
import subprocess

import pytest

import sequence_attention_dits_amd as uaa
from sequence_attention_dits_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uaa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"uaa_seq2head_permute", "usp_attn_fwd_lse", "usp_attn_fwd_lse_ws", "usp_attn_workspace_bytes",
            "usp_lse_merge", "uaa_last_error"} <= set(names)
    lib = uaa.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(names) <= exported
    assert lib.uaa_abi_version() == 1


def test_mask_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "uaa.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(usp_mask),'
                   'offsetof(usp_mask,kind),offsetof(usp_mask,world),offsetof(usp_mask,q_off),'
                   'offsetof(usp_mask,k_off),offsetof(usp_mask,chunk),offsetof(usp_mask,q_chunks),'
                   'offsetof(usp_mask,k_chunks),offsetof(usp_mask,q_rank),offsetof(usp_mask,k_rank));return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    c_vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    M = binding.usp_mask
    py_vals = [ctypes.sizeof(M)] + [getattr(M, f).offset for f in
                                    ("kind", "world", "q_off", "k_off", "chunk", "q_chunks", "k_chunks",
                                     "q_rank", "k_rank")]
    assert c_vals == py_vals


def _perm(*args):
    lib = uaa.lib()
    return lib.uaa_seq2head_permute(*args), lib.uaa_last_error().decode()


def _i64(*v):
    return (ctypes.c_int64 * len(v))(*v)


def _ptrs(*v):
    return (ctypes.c_void_p * len(v))(*v)


FAKE = 0x10000  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("args,code,text", [
    ((7, 0, 2, _i64(0, 2, 4), None, 1, 2, 8, 2, _ptrs(FAKE, FAKE), FAKE, None), -1, "dir"),
    ((0, 0, 0, _i64(0), None, 1, 2, 8, 2, _ptrs(FAKE), FAKE, None), -1, "world"),
    ((0, 2, 2, _i64(0, 2, 4), None, 1, 2, 8, 2, _ptrs(FAKE, FAKE), FAKE, None), -1, "rank"),
    ((0, 0, 2, _i64(0, 2, 4), None, 1, 2, 8, 3, _ptrs(FAKE, FAKE), FAKE, None), -1, "elem_bytes"),
    ((0, 0, 2, _i64(1, 2, 4), None, 1, 2, 8, 2, _ptrs(FAKE, FAKE), FAKE, None), -1, "seq_off[0]"),
    ((0, 0, 2, _i64(0, 3, 2), None, 1, 2, 8, 2, _ptrs(FAKE, FAKE), FAKE, None), -1, "decreases"),
    ((0, 0, 3, _i64(0, 1, 2, 3), None, 1, 2, 8, 2, _ptrs(FAKE, FAKE, FAKE), FAKE, None), -1, "no heads"),
    ((0, 0, 2, _i64(0, 2, 4), _i64(0, 1, 3), 1, 2, 8, 2, _ptrs(FAKE, FAKE), FAKE, None), -1, "head_off"),
    ((0, 0, 2, _i64(0, 2, 4), None, 1, 2, 8, 2, _ptrs(FAKE, 0), FAKE, None), -1, "src[1]"),
    ((0, 0, 2, _i64(0, 2, 4), None, 1, 2, 8, 2, _ptrs(FAKE, FAKE), 0, None), -1, "dst"),
    ((0, 0, 2, _i64(0, 2, 4), None, 1, 2, 8, 4, _ptrs(FAKE + 2, FAKE), FAKE, None), -1, "aligned"),
    ((0, 0, 2, _i64(0, 2, 4), None, -1, 2, 8, 2, _ptrs(FAKE, FAKE), FAKE, None), -1, "B >= 0"),
])
def test_permute_validation(args, code, text):
    rc, msg = _perm(*args)
    assert rc == code and text in msg, (rc, msg)


def test_permute_empty_work_is_ok_without_pointers():
    # B = 0 and an empty destination shard need no pointers and no GPU
    assert _perm(0, 0, 2, _i64(0, 2, 4), None, 0, 2, 8, 2, _ptrs(0, 0), 0, None)[0] == 0
    assert _perm(1, 1, 2, _i64(0, 4, 4), None, 1, 2, 8, 2, _ptrs(0, 0), 0, None)[0] == 0


def _attn(dtype=0, B=1, H=1, Sq=4, Sk=4, D=128, q=FAKE, k=FAKE, v=FAKE, o=FAKE, odt=0, lse=FAKE,
          scale=0.1, mask=None):
    lib = uaa.lib()
    m = mask if mask is not None else uaa.mask_full()
    rc = lib.usp_attn_fwd_lse(dtype, B, H, Sq, Sk, D, q, k, v, o, odt, lse, scale, ctypes.byref(m), None)
    return rc, lib.uaa_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(dtype=5), -1, "dtype"),
    (dict(odt=9), -1, "o_dtype"),
    (dict(Sq=-1), -1, "negative"),
    (dict(scale=0.0), -1, "scale"),
    (dict(scale=float("inf")), -1, "scale"),
    (dict(scale=float("nan")), -1, "scale"),
    (dict(D=96), -2, "D must be"),
    (dict(dtype=1, odt=0), -2, "fp32 input"),
    (dict(q=0), -1, "NULL"),
    (dict(k=0), -1, "NULL"),
    (dict(o=FAKE + 8), -1, "16-byte"),
    (dict(lse=FAKE + 2), -1, "4-byte"),
    (dict(mask=binding.usp_mask(kind=9)), -1, "mask kind"),
    (dict(mask=uaa.mask_zigzag(0, [1], [2])), -1, "chunk length"),
    (dict(mask=uaa.mask_zigzag(2, [1], [2])), -1, "chunks hold"),
    (dict(mask=uaa.mask_zigzag(4, [-3], [2])), -1, "chunk id"),
    (dict(mask=uaa.mask_stripe(0, 0, 0)), -1, "stripe"),
    (dict(mask=uaa.mask_stripe(4, 1, 4)), -1, "stripe"),
])
def test_attention_validation(kw, code, text):
    rc, msg = _attn(**kw)
    assert rc == code and text in msg, (rc, msg)


def _attn_ws(ws, nbytes, dtype=0, D=128, mask=None):
    lib = uaa.lib()
    m = mask if mask is not None else uaa.mask_full()
    rc = lib.usp_attn_fwd_lse_ws(dtype, 1, 1, 4, 4, D, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0.1, ctypes.byref(m),
                                 ws, nbytes, None)
    return rc, lib.uaa_last_error().decode()


def test_accumulate_call_validates_like_the_plain_call():
    lib = uaa.lib()
    m = uaa.mask_full()
    for kw, code in ((dict(dtype=5), -1), (dict(D=96), -2)):
        args = dict(dtype=0, D=128)
        args.update(kw)
        rc = lib.usp_attn_fwd_lse_acc(args["dtype"], 1, 1, 4, 4, args["D"], FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0.1,
                                      ctypes.byref(m), None, 0, None)
        assert rc == code and lib.uaa_last_error().decode() == _attn(**kw)[1]


def test_workspace_call_validates_like_the_plain_call():
    assert _attn_ws(FAKE, 1 << 20, dtype=5) == (-1, _attn(dtype=5)[1])
    assert _attn_ws(FAKE, 1 << 20, D=96)[0] == -2
    rc, msg = _attn_ws(FAKE + 16, 1 << 20)
    assert rc == -1 and "256-byte" in msg, (rc, msg)


def test_gather_validation():
    lib = uaa.lib()
    m = uaa.mask_full()
    so = (ctypes.c_int64 * 3)(0, 4, 8)
    sh = (ctypes.c_void_p * 2)(FAKE, FAKE)

    def call(dtype=0, world=2, rank=0, seq=so, H=2, D=128, k_shard=0, o=FAKE):
        rc = lib.usp_attn_fwd_lse_gather(dtype, world, rank, seq, None, 1, H, D, sh, sh, sh, k_shard, o, 0, FAKE,
                                         0.1, ctypes.byref(m), None, 0, 0, None)
        return rc, lib.uaa_last_error().decode()

    assert call(dtype=1)[0] == -2                      # fp32: unsupported
    assert call(world=9)[0] == -1 and "world" in call(world=9)[1]
    assert call(rank=2)[0] == -1
    assert call(k_shard=-1)[0] == -1 and "k_shard" in call(k_shard=-1)[1]
    assert call(seq=(ctypes.c_int64 * 3)(0, 5, 4))[0] == -1
    assert call(H=1)[0] == -1 and "no heads" in call(H=1)[1]
    assert call(D=96)[0] == -2
    assert call(o=FAKE + 8)[0] == -1


def test_workspace_bytes_zero_where_no_split_applies():
    lib = uaa.lib()
    full, causal = uaa.mask_full(), uaa.mask_causal(0, 0)
    big = (1, 24, 3493, 3493)   # B, H, Sq, Sk
    assert lib.usp_attn_workspace_bytes(1, *big, 128, ctypes.byref(full)) == 0       # fp32
    assert lib.usp_attn_workspace_bytes(0, *big, 128, ctypes.byref(causal)) == 0     # masked
    assert lib.usp_attn_workspace_bytes(0, *big, 96, ctypes.byref(full)) == 0        # head dim
    assert lib.usp_attn_workspace_bytes(0, 1, 24, -1, 3493, 128, ctypes.byref(full)) == 0


def test_attention_empty_work_is_ok():
    assert _attn(Sq=0, q=0, o=0, lse=0)[0] == 0
    assert _attn(B=0)[0] == 0
    assert _attn(H=0)[0] == 0


def _merge(n=2, B=1, S=4, H=1, D=8, parts=None, pdt=0, lses=None, o=FAKE, odt=0, lse=FAKE):
    lib = uaa.lib()
    parts = parts if parts is not None else [FAKE] * max(n, 1)
    lses = lses if lses is not None else [FAKE] * max(n, 1)
    rc = lib.usp_lse_merge(n, B, S, H, D, _ptrs(*parts), pdt, _ptrs(*lses), o, odt, lse, None)
    return rc, lib.uaa_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(n=0), -1, "n_parts"),
    (dict(n=17, parts=[FAKE] * 17, lses=[FAKE] * 17), -1, "n_parts"),
    (dict(pdt=4), -1, "part_dtype"),
    (dict(odt=4), -1, "out_dtype"),
    (dict(D=0), -1, "sizes"),
    (dict(parts=[FAKE, 0]), -1, "part 1"),
    (dict(lses=[FAKE + 2, FAKE]), -1, "misaligned"),
    (dict(o=0), -1, "NULL"),
    (dict(parts=[FAKE, FAKE], o=FAKE, pdt=0, odt=1), -1, "alias"),
])
def test_merge_validation(kw, code, text):
    rc, msg = _merge(**kw)
    assert rc == code and text in msg, (rc, msg)


def test_merge_empty_work_is_ok():
    assert _merge(S=0, o=0, lse=0)[0] == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()


def test_multi_ex_permute_validation():
    lib = uaa.lib()
    ptrs = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    dsts = (ctypes.c_void_p * 2)(FAKE, FAKE)
    so = (ctypes.c_int64 * 3)(0, 2, 4)
    Ds = (ctypes.c_int64 * 2)(128, 1)
    for elems, text in (((2, 3), "elem_bytes"), ((2, 4), None)):
        e = (ctypes.c_int * 2)(*elems)
        rc = lib.uaa_seq2head_permute_multi_ex(2, 0, 0, 2, so, None, 0, 4, Ds, e, ptrs, dsts, None)
        if text is None:
            assert rc == 0          # B = 0: validated, no work
        else:
            assert rc == -1 and text in lib.uaa_last_error().decode()
    e = (ctypes.c_int * 2)(2, 4)
    assert lib.uaa_seq2head_permute_multi_ex(2, 0, 0, 2, so, None, 1, 4, None, e, ptrs, dsts, None) == -1
    bad = (ctypes.c_int64 * 2)(128, 0)
    assert lib.uaa_seq2head_permute_multi_ex(2, 0, 0, 2, so, None, 1, 4, bad, e, ptrs, dsts, None) == -1
    assert lib.uaa_seq2head_permute_multi_ex(5, 0, 0, 2, so, None, 1, 4, Ds, e, ptrs, dsts, None) == -1


def test_multi_permute_validation():
    lib = uaa.lib()
    src = _ptrs(*([FAKE] * 8))
    dst = _ptrs(FAKE, FAKE, FAKE, FAKE, FAKE)
    assert lib.uaa_seq2head_permute_multi(0, 0, 0, 2, _i64(0, 2, 4), None, 1, 2, 8, 2, src, dst, None) == -1
    assert "n_tensors" in lib.uaa_last_error().decode()
    assert lib.uaa_seq2head_permute_multi(5, 0, 0, 2, _i64(0, 2, 4), None, 1, 2, 8, 2, src, dst, None) == -1
    big = _i64(*range(0, 34))   # world 33 with 2 tensors exceeds 64 source pointers
    assert lib.uaa_seq2head_permute_multi(2, 0, 0, 33, big, None, 1, 40, 8, 2, src, dst, None) == -1
    assert "n_tensors" in lib.uaa_last_error().decode()
    dst0 = _ptrs(FAKE, 0)
    assert lib.uaa_seq2head_permute_multi(2, 0, 0, 2, _i64(0, 2, 4), None, 1, 2, 8, 2, src, dst0, None) == -1
    assert "dst[1]" in lib.uaa_last_error().decode()


def _bwd(dtype=0, B=1, H=1, Sq=4, Sk=4, D=128, q=FAKE, k=FAKE, v=FAKE, do=FAKE, lse=FAKE, delta=FAKE,
         dq=FAKE, dk=FAKE, dv=FAKE, gdt=1, scale=0.1, mask=None, acc=0):
    lib = uaa.lib()
    m = mask if mask is not None else uaa.mask_full()
    rc = lib.usp_attn_bwd(dtype, B, H, Sq, Sk, D, q, k, v, do, lse, delta, dq, dk, dv, gdt, scale,
                          ctypes.byref(m), acc, None)
    return rc, lib.uaa_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(dtype=5), -1, "dtype"),
    (dict(gdt=3), -1, "grad_dtype"),
    (dict(Sk=-1), -1, "negative"),
    (dict(scale=0.0), -1, "scale"),
    (dict(scale=float("nan")), -1, "scale"),
    (dict(acc=4), -1, "accumulate"),
    (dict(acc=-1), -1, "accumulate"),
    (dict(D=96), -2, "D must be"),
    (dict(delta=0), -1, "NULL"),
    (dict(dv=0), -1, "NULL"),
    (dict(dq=FAKE + 8), -1, "16-byte"),
    (dict(lse=FAKE + 2), -1, "4-byte"),
    (dict(mask=binding.usp_mask(kind=9)), -1, "mask kind"),
    (dict(mask=uaa.mask_zigzag(2, [1], [2])), -1, "chunks hold"),
    (dict(mask=uaa.mask_stripe(4, 1, 4)), -1, "stripe"),
    (dict(Sq=1 << 26, H=64), -2, "4 GiB"),
])
def test_backward_validation(kw, code, text):
    rc, msg = _bwd(**kw)
    assert rc == code and text in msg, (rc, msg)


def test_backward_empty_work_is_ok():
    assert _bwd(B=0)[0] == 0
    assert _bwd(H=0)[0] == 0
    assert _bwd(Sq=0, Sk=0, q=0, k=0, v=0, do=0, lse=0, delta=0, dq=0, dk=0, dv=0)[0] == 0


@pytest.mark.parametrize("kw,code,text", [
    (dict(dtype=4), -1, "dtype"),
    (dict(D=32), -2, "D must be"),
    (dict(o=0), -1, "NULL"),
    (dict(dout=FAKE + 4), -1, "16-byte"),
    (dict(dlse=FAKE + 1), -1, "4-byte"),
])
def test_backward_delta_validation(kw, code, text):
    a = dict(dtype=0, B=1, S=4, H=2, D=128, o=FAKE, dout=FAKE, dlse=None, delta=FAKE)
    a.update(kw)
    lib = uaa.lib()
    rc = lib.usp_attn_bwd_delta(a["dtype"], a["B"], a["S"], a["H"], a["D"], a["o"], a["dout"], a["dlse"],
                                a["delta"], None)
    assert rc == code and text in lib.uaa_last_error().decode(), (rc, lib.uaa_last_error())
    assert lib.usp_attn_bwd_delta(0, 0, 4, 2, 128, 0, 0, None, 0, None) == 0


def test_split_offsets_matches_the_oracle_split():
    """The library's default split (used for heads when head_off is NULL)
    against the oracle's, which is written independently from the pages'
    worked lengths (257 -> 129 / 128, 4481 -> 2241 / 2240)."""
    import oracle
    assert uaa.uaa_split_offsets(257, 2) == [0, 129, 257]
    assert uaa.uaa_split_offsets(4481, 2) == [0, 2241, 4481]
    for total in (0, 1, 5, 7, 24, 31, 4608, 6986):
        for parts in (1, 2, 3, 4, 7, 8, 64):
            assert uaa.uaa_split_offsets(total, parts) == oracle.split_offsets(total, parts), (total, parts)


@pytest.mark.parametrize("total,parts,text", [(5, 0, "parts"), (-1, 2, "total")])
def test_split_offsets_validation(total, parts, text):
    lib = uaa.lib()
    off = (ctypes.c_int64 * 4)(7, 7, 7, 7)
    assert lib.uaa_split_offsets(total, parts, off) == -1
    assert text in lib.uaa_last_error().decode()
    assert list(off) == [7, 7, 7, 7]
    assert lib.uaa_split_offsets(5, 2, None) == -1


def test_kernel_query_names_the_kernel_of_each_case():
    """usp_attn_kernel: the workloads' launches and the selection rules
    (pipelined for bf16 D = 128 without a key split: unmasked, masks whose
    256-row units see every key of the block or none, and in its DIAG form
    masks whose keys are one increasing piece; the general kernel
    otherwise).  Host only."""
    K = uaa
    bf, f32 = __import__("torch").bfloat16, __import__("torch").float32
    flux = (1, 4608, 12, 128)
    assert K.usp_attn_kernel(flux, 2304) == K.USP_KERNEL_PIPELINED
    assert K.usp_attn_kernel((1, 4481, 12, 128), 2241) == K.USP_KERNEL_PIPELINED
    assert K.usp_attn_kernel(flux, 2304, f32) == K.USP_KERNEL_FP32
    assert K.usp_attn_kernel(flux, 2304, bf, f32) == K.USP_KERNEL_PIPELINED
    assert K.usp_attn_kernel((1, 4608, 12, 64), 2304) == K.USP_KERNEL_GENERAL
    assert K.usp_attn_kernel((1, 300, 2, 128), 64 * 7) == K.USP_KERNEL_PIPELINED   # any tile count
    assert K.usp_attn_kernel((1, 300, 2, 128), 1) == K.USP_KERNEL_PIPELINED
    assert K.usp_attn_kernel((0, 300, 2, 128), 64) == K.USP_KERNEL_NONE
    lc = (1, 8192, 32, 128)
    zz = lambda c: K.mask_zigzag(4096, [1, 6], [c])
    assert K.usp_attn_kernel(lc, 4096, mask=zz(0)) == K.USP_KERNEL_PIPELINED      # wholly in the past
    assert K.usp_attn_kernel(lc, 4096, mask=zz(3)) == K.USP_KERNEL_PIPELINED      # units see all or none
    assert K.usp_attn_kernel((1, 300, 2, 128), 300, mask=K.mask_causal()) == K.USP_KERNEL_PIPELINED_DIAG
    assert K.usp_attn_kernel((1, 300, 2, 64), 300, mask=K.mask_causal()) == K.USP_KERNEL_GENERAL_MASKED
    # units on a diagonal: the pipelined kernel's DIAG form where the keys are one increasing piece
    assert K.usp_attn_kernel((1, 768, 2, 128), 768, mask=K.mask_causal()) == K.USP_KERNEL_PIPELINED_DIAG
    assert K.usp_attn_kernel(lc, 4096, mask=zz(1)) == K.USP_KERNEL_PIPELINED_DIAG
    assert K.usp_attn_kernel(lc, 4096, mask=zz(6)) == K.USP_KERNEL_PIPELINED_DIAG
    assert K.usp_attn_kernel((1, 768, 2, 128), 768, mask=K.mask_stripe(4, 1, 2)) == K.USP_KERNEL_PIPELINED_DIAG
    two_key_chunks = K.mask_zigzag(384, [1, 6], [1, 6])   # keys in two pieces: the general kernel
    assert K.usp_attn_kernel((1, 768, 2, 128), 768, mask=two_key_chunks) == K.USP_KERNEL_GENERAL_MASKED
    with pytest.raises(uaa.UaaError) as e:
        K.usp_attn_kernel(flux, 2304, mask=K.usp_mask(kind=7))
    assert e.value.status == K.UAA_ERR_INVALID_ARG
    with pytest.raises(uaa.UaaError) as e:
        K.usp_attn_kernel((1, 30, 2, 96), 30)
    assert e.value.status == K.UAA_ERR_UNSUPPORTED
