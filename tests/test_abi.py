"""The C-ABI boundary on the host: the library loads, exports what include/ffpa.h declares, and
checks arguments before any HIP call (these tests never touch a GPU)."""
import ctypes
import math
import os
import re

import pytest

import exact_attention_head_amd as ffpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffpa.h")

# fake, 16-byte aligned, non-overlapping "device addresses": ffpa_check_args never dereferences them
Q, K, V, O, L, M = (0x10_0000_0000 * (i + 1) for i in range(6))


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ffpa_\w+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(ffpa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ffpa.library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def check(B=1, Hq=2, Hkv=1, Nq=100, Nkv=130, D=512, scale=math.nan, causal=False, dtype=ffpa.FFPA_BF16,
          mask=None, q=Q, k=K, v=V, o=O, lse=L):
    return ffpa.ffpa_check_args(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype)


def detail():
    return ffpa.library().ffpa_last_error_detail().decode()


def test_valid_arguments_pass():
    assert check() == ffpa.OK
    assert detail() == ""
    for D in range(8, 1025, 8):  # every multiple of 8 (those without a kernel of their own run padded)
        assert check(D=D) == ffpa.OK, D
    assert check(causal=True) == ffpa.OK
    assert check(lse=None) == ffpa.OK
    assert check(scale=0.125) == ffpa.OK
    assert check(Hq=8, Hkv=8) == ffpa.OK
    assert check(Nq=1, Nkv=1) == ffpa.OK


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), ffpa.ERR_TYPE),
    (dict(dtype=-1), ffpa.ERR_TYPE),
    (dict(Hq=3, Hkv=2), ffpa.ERR_VALUE),
    (dict(B=0), ffpa.ERR_VALUE),
    (dict(Nq=0), ffpa.ERR_VALUE),
    (dict(Nkv=-5), ffpa.ERR_VALUE),
    (dict(causal=True, Nq=131, Nkv=130), ffpa.ERR_VALUE),
    (dict(scale=math.inf), ffpa.ERR_VALUE),
    (dict(scale=-math.inf), ffpa.ERR_VALUE),
    (dict(q=0), ffpa.ERR_VALUE),
    (dict(o=0), ffpa.ERR_VALUE),
    (dict(k=K + 8), ffpa.ERR_VALUE),
    (dict(lse=L + 2), ffpa.ERR_VALUE),
    (dict(o=Q), ffpa.ERR_VALUE),
    (dict(o=Q + 1024), ffpa.ERR_VALUE),
    (dict(lse=V + 64), ffpa.ERR_VALUE),
    (dict(D=100), ffpa.ERR_UNSUPPORTED),
    (dict(D=4), ffpa.ERR_UNSUPPORTED),
    (dict(D=1020), ffpa.ERR_UNSUPPORTED),
    (dict(D=1032), ffpa.ERR_UNSUPPORTED),
    (dict(D=1088), ffpa.ERR_UNSUPPORTED),
    (dict(D=2048), ffpa.ERR_UNSUPPORTED),
])
def test_argument_errors(kw, status):
    assert check(**kw) == status
    assert detail() != ""


def mdesc(kind=ffpa.MASK_ADD_F32, data=M, sb=0, sh=0, sq=130, sk=1):
    return ffpa.MaskDesc(data, kind, sb, sh, sq, sk)


def test_mask_descriptor_rules():
    assert check(mask=mdesc()) == ffpa.OK
    assert check(mask=mdesc(kind=ffpa.MASK_BOOL_U8)) == ffpa.OK
    assert check(mask=mdesc(kind=ffpa.MASK_ADD_BF16)) == ffpa.OK
    assert check(mask=mdesc(kind=ffpa.MASK_ADD_FP16)) == ffpa.OK
    assert check(mask=mdesc(kind=ffpa.MASK_NONE, data=0)) == ffpa.OK
    assert check(mask=mdesc(kind=7)) == ffpa.ERR_TYPE
    assert check(mask=mdesc(data=0)) == ffpa.ERR_VALUE
    assert check(mask=mdesc(), causal=True) == ffpa.OK  # both apply
    assert check(mask=mdesc(), causal=True, Nq=131, Nkv=130) == ffpa.ERR_VALUE
    assert check(mask=mdesc(sk=2)) == ffpa.ERR_UNSUPPORTED
    assert check(mask=mdesc(sk=0)) == ffpa.ERR_UNSUPPORTED
    assert check(mask=mdesc(sq=-130)) == ffpa.ERR_VALUE
    assert check(mask=mdesc(data=M + 2)) == ffpa.ERR_VALUE  # fp32 mask must be 4-byte aligned
    assert check(mask=mdesc(data=O)) == ffpa.ERR_VALUE  # overlaps the output


def test_status_strings():
    lib = ffpa.library()
    names = [lib.ffpa_status_string(s).decode() for s in range(5)]
    assert len(set(names)) == 5 and all(names)
    assert lib.ffpa_status_string(99).decode()


@pytest.mark.parametrize("status,exc", [(ffpa.ERR_TYPE, TypeError), (ffpa.ERR_VALUE, ValueError),
                                        (ffpa.ERR_UNSUPPORTED, NotImplementedError), (ffpa.ERR_HIP, RuntimeError)])
def test_status_maps_to_the_pages_error_classes(status, exc):
    with pytest.raises(exc):
        ffpa._raise(status)


def test_rows_per_block():
    rows = {D: ffpa.rows_per_block(D) for D in range(8, 1025, 8)}
    assert all(r in (64, 128, 256) for r in rows.values()), rows
    assert ffpa.rows_per_block(100) == 0 and ffpa.rows_per_block(1032) == 0
    assert ffpa.rows_per_block(80) == ffpa.rows_per_block(128)


def test_kernel_head_dim():
    row_dims = [64, 128, 192, 256, 320, 384, 448, 512, 640, 768, 896, 1024]
    for D in range(8, 1025, 8):
        want = min(d for d in row_dims if d >= D)
        assert ffpa.kernel_head_dim(D) == want, D
    assert ffpa.kernel_head_dim(8) == 64 and ffpa.kernel_head_dim(520) == 640 and ffpa.kernel_head_dim(1016) == 1024
    # the shared-staging head dims run the row kernel of the next head dim up (dropout aside)
    assert [ffpa.kernel_head_dim(D) for D in (576, 704, 832, 960)] == [640, 768, 896, 1024]
    for bad in (0, 4, 100, 1020, 1032, 2048):
        assert ffpa.kernel_head_dim(bad) == 0, bad


def test_kernel_name():
    names = {D: ffpa.kernel_name(D) for D in range(64, 1025, 64)}
    assert set(names.values()) == {"ffpa_fwd_row_kernel"}, names
    # the head dims of the benchmark run the row kernel
    assert names[512] == "ffpa_fwd_row_kernel" and names[1024] == "ffpa_fwd_row_kernel"
    # padded head dims run the row kernel of the next head dim up
    assert ffpa.kernel_name(96) == "ffpa_fwd_row_kernel" and ffpa.kernel_name(552) == "ffpa_fwd_row_kernel"
    assert ffpa.kernel_name(100) is None and ffpa.kernel_name(2048) is None


def test_python_layer_rejects_before_the_library():
    import torch

    q = torch.zeros(1, 2, 4, 64, dtype=torch.float32)
    for p in (1.0, -0.1, 1.5):  # dropout probability outside [0, 1)
        with pytest.raises(ValueError):
            ffpa.attn(q, q, q, dropout_p=p)
    with pytest.raises(TypeError):
        ffpa.attn(q, q, q)
    qb = q.to(torch.bfloat16)
    kb = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # not on a GPU
        ffpa.attn(qb, kb, kb, enable_gqa=True)


def test_strided_views_the_kernels_cannot_address_are_copied():
    """attn reads a strided view in place only when ffpa_check_strided_args accepts its layout; a view
    whose row stride or span exceeds the kernels' 32-bit buffer offsets goes through contiguous copies
    (the dense entry takes those) instead of failing."""
    B, H, N, D = 1, 64, 131072, 128
    ptrs = [Q, K, V, O]
    bnhd = [0, D, H * D]  # [B, N, H, D] storage seen as [B, H, N, D]: row stride H * D
    assert ffpa._strided_plan(ptrs, [bnhd] * 4, B, H, H, N, N, D, ffpa.FFPA_BF16) is None
    small = [0, D, 8 * D]
    lay = ffpa._strided_plan(ptrs, [small] * 4, B, 8, 8, 300, 300, D, ffpa.FFPA_BF16)
    assert lay is not None and list(lay.q) == small and list(lay.o) == small
    # K and V with different row strides: also copied
    assert ffpa._strided_plan(ptrs, [small, small, [0, D, 16 * D], small], B, 8, 8, 300, 300, D,
                              ffpa.FFPA_BF16) is None


# ---- packed variable-length entry (ffpa_fwd_varlen)
CQ, CK = 0x70_0000_0000, 0x80_0000_0000


def vcheck(B=3, Hq=4, Hkv=2, Tq=300, Tk=500, mq=200, mk=300, D=512, scale=math.nan, causal=False,
           dtype=ffpa.FFPA_BF16, q=Q, k=K, v=V, cq=CQ, ck=CK, o=O, lse=L):
    return ffpa.ffpa_check_varlen_args(q, k, v, cq, ck, o, lse, B, Hq, Hkv, Tq, Tk, mq, mk, D, scale, causal, dtype)


def test_varlen_valid_arguments_pass():
    assert vcheck() == ffpa.OK and detail() == ""
    for D in range(8, 1025, 8):
        assert vcheck(D=D) == ffpa.OK, D
    assert vcheck(causal=True, mq=500, mk=10) == ffpa.OK   # fewer keys than queries is allowed
    assert vcheck(Tq=0, Tk=0, mq=0, mk=0, q=None, k=None, v=None, o=None) == ffpa.OK
    assert vcheck(Tk=0, mk=0, k=None, v=None) == ffpa.OK
    assert vcheck(cq=CQ, ck=CQ) == ffpa.OK  # self-attention shares one offset array


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), ffpa.ERR_TYPE),
    (dict(B=0), ffpa.ERR_VALUE),
    (dict(Hq=3, Hkv=2), ffpa.ERR_VALUE),
    (dict(Tq=-1), ffpa.ERR_VALUE),
    (dict(mk=-1), ffpa.ERR_VALUE),
    (dict(causal=2), ffpa.ERR_VALUE),
    (dict(scale=math.inf), ffpa.ERR_VALUE),
    (dict(cq=None), ffpa.ERR_VALUE),
    (dict(ck=CK + 2), ffpa.ERR_VALUE),
    (dict(q=None), ffpa.ERR_VALUE),
    (dict(o=O + 8), ffpa.ERR_VALUE),
    (dict(o=Q + 64), ffpa.ERR_VALUE),          # o overlaps q
    (dict(o=CQ - 64), ffpa.ERR_VALUE),         # o overlaps the offsets
    (dict(D=100), ffpa.ERR_UNSUPPORTED),
    (dict(mk=1 << 20, Hkv=4, Hq=4, D=1024), ffpa.ERR_UNSUPPORTED),  # one sequence's K rows beyond 2 GiB
])
def test_varlen_argument_errors(kw, status):
    assert vcheck(**kw) == status, kw
    assert detail() != ""


def test_cu_seqlens_host_check():
    assert ffpa.ffpa_check_cu_seqlens([0, 3, 3, 10], 10, 7) == ffpa.OK
    assert ffpa.ffpa_check_cu_seqlens([1, 3, 10], 10, 7) == ffpa.ERR_VALUE
    assert ffpa.ffpa_check_cu_seqlens([0, 5, 3, 10], 10, 7) == ffpa.ERR_VALUE
    assert ffpa.ffpa_check_cu_seqlens([0, 3, 9], 10, 7) == ffpa.ERR_VALUE
    assert ffpa.ffpa_check_cu_seqlens([0, 3, 10], 10, 6) == ffpa.ERR_VALUE   # a sequence longer than max
    assert "max_seqlen" in detail()


def test_attn_records_autograd_when_inputs_need_grad():
    """With grad mode on and an input requiring grad, attn goes through the autograd function (here it
    then stops at the device check inside it); out and the dropout-word options are refused there."""
    import torch

    qb = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16, requires_grad=True)
    kb = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="autograd"):
        ffpa.attn(qb, kb, kb, out=torch.empty(1, 2, 4, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="autograd"):
        ffpa.attn(qb, kb, kb, dropout_p=0.1, return_dropout_keep=True)
    with pytest.raises(ValueError, match="same GPU"):  # recorded, then the forward's own checks
        ffpa.attn(qb, kb, kb)
    with torch.no_grad(), pytest.raises(ValueError, match="same GPU"):  # nothing recorded: out is fine
        ffpa.attn(qb, kb, kb, out=torch.empty(1, 2, 4, 64, dtype=torch.bfloat16))
    # a floating mask that requires grad is recorded too
    m = torch.zeros(1, 1, 4, 4, requires_grad=True)
    with pytest.raises(ValueError, match="autograd"):
        ffpa.attn(kb, kb, kb, attn_mask=m, out=torch.empty(1, 2, 4, 64, dtype=torch.bfloat16))


def test_pages_function_names():
    """ffpa_attn_func and ffpa_attn_varlen_func, the names and signatures of the "API Reference" page:
    the backend keywords are accepted, any other raises TypeError, and the call goes through attn."""
    import torch

    qb = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        ffpa.ffpa_attn_func(qb, qb, qb, acc="f32")
    with pytest.raises(ValueError, match="same GPU"):  # accepted, then attn's own checks
        ffpa.ffpa_attn_func(qb, qb, qb, backend="cutedsl", forward_backend=None, backward_backend=None)
    with pytest.raises(TypeError):  # attn's dtype rule
        ffpa.ffpa_attn_func(qb.float(), qb.float(), qb.float())
    assert ffpa.ffpa_attn_varlen_func is ffpa.attn_varlen

def test_varlen_refuses_inputs_that_need_grad():
    import torch

    q = torch.zeros(10, 2, 64, dtype=torch.bfloat16, requires_grad=True)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(NotImplementedError, match="no backward"):
        ffpa.attn_varlen(q, q, q, cu, cu, 6, 6)
    with torch.no_grad(), pytest.raises(ValueError):  # nothing recorded: on to the device check
        ffpa.attn_varlen(q, q, q, cu, None, 6, 6)

def test_varlen_python_layer_rejects_before_the_library():
    import torch

    q = torch.zeros(10, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(NotImplementedError):
        ffpa.attn_varlen(q, q, q, cu, cu, 6, 6, dropout_p=0.1)
    with pytest.raises(NotImplementedError):
        ffpa.attn_varlen(q, q, q, cu, cu, 6, 6, softcap=1.0)
    with pytest.raises(TypeError):
        ffpa.attn_varlen(q, q, q, cu.long(), cu, 6, 6)
    with pytest.raises(TypeError):
        ffpa.attn_varlen(q.float(), q.float(), q.float(), cu, cu, 6, 6)
    with pytest.raises(ValueError):  # malformed offsets
        ffpa.attn_varlen(q, q, q, torch.tensor([0, 7, 4], dtype=torch.int32), None, 7, 7)
    with pytest.raises(ValueError):  # max_seqlen below a sequence's length
        ffpa.attn_varlen(q, q, q, cu, None, 5, 5)
    with pytest.raises(ValueError):  # Hq != Hkv without enable_gqa
        ffpa.attn_varlen(q, q[:, :1], q[:, :1], cu, cu, 6, 6)
    with pytest.raises(ValueError):  # not on a GPU
        ffpa.attn_varlen(q, q, q, cu, None, 6, 6)


# ---- strided layouts (ffpa_fwd_strided)
def layout(q=None, k=None, v=None, o=None, B=1, Hq=2, Hkv=1, Nq=100, Nkv=130, D=512):
    """Default: [B, N, H, D] storage (NHD) seen as [B, H, N, D]."""
    nhd = lambda H, N: [N * H * D, D, H * D]
    return ffpa.LayoutDesc((ctypes.c_int64 * 3)(*(q or nhd(Hq, Nq))), (ctypes.c_int64 * 3)(*(k or nhd(Hkv, Nkv))),
                           (ctypes.c_int64 * 3)(*(v or nhd(Hkv, Nkv))), (ctypes.c_int64 * 3)(*(o or nhd(Hq, Nq))))


def scheck(lay, B=1, Hq=2, Hkv=1, Nq=100, Nkv=130, D=512, causal=False, q=Q, k=K, v=V, o=O, lse=L):
    return ffpa.ffpa_check_strided_args(q, k, v, None, o, lse, B, Hq, Hkv, Nq, Nkv, D, lay, math.nan, causal,
                                        ffpa.FFPA_BF16)


def test_strided_layouts_pass():
    assert scheck(layout()) == ffpa.OK and detail() == ""
    assert scheck(layout(B=2), B=2) == ffpa.OK
    # K and V broadcast over the batch, heads sliced out of a fused [N, 3, H, D] projection
    assert scheck(layout(k=[0, 512, 3 * 512], v=[0, 512, 3 * 512]), B=3) == ffpa.OK
    assert scheck(layout(o=[2 * 100 * 512, 100 * 512, 512])) == ffpa.OK  # contiguous O


@pytest.mark.parametrize("kw,status", [
    (dict(q=[1024 * 100, 512, 1020]), ffpa.ERR_VALUE),        # row stride not a multiple of 8
    (dict(k=[0, 512, -512]), ffpa.ERR_VALUE),                 # negative stride
    (dict(k=[0, 512, 1024], v=[0, 512, 2048]), ffpa.ERR_UNSUPPORTED),  # K and V row strides differ
    (dict(o=[0, 256, 1024]), ffpa.ERR_VALUE),                 # O rows of both heads overlap
    (dict(o=[0, 512, 512]), ffpa.ERR_VALUE),                  # row 1 of head 0 is row 0 of head 1
    (dict(k=[0, 0, 1 << 24], v=[0, 0, 1 << 24]), ffpa.ERR_UNSUPPORTED),  # K rows span beyond 2 GiB
    (dict(k=[0, 512, 0], v=[0, 512, 0]), ffpa.ERR_UNSUPPORTED),          # K/V expanded along N
    (dict(q=[0, 0, 256]), ffpa.ERR_UNSUPPORTED),                         # overlapping Q rows
])
def test_strided_layout_errors(kw, status):
    assert scheck(layout(**kw)) == status, kw
    assert detail() != ""


def test_strided_layout_overlap_uses_extents():
    # O placed right after Q's last element is fine; one element earlier it overlaps
    ext = ((1 - 1) * 100 * 2 * 512 + (2 - 1) * 512 + (100 - 1) * 2 * 512 + 512) * 2
    assert scheck(layout(), o=Q + ext) == ffpa.OK
    assert scheck(layout(), o=Q + ext - 16) == ffpa.ERR_VALUE
    assert ffpa.ffpa_check_strided_args(Q, K, V, None, O, L, 1, 2, 1, 100, 130, 512, None, math.nan, False,
                                        ffpa.FFPA_BF16) == ffpa.ERR_VALUE  # no layout


# ---- attention dropout (ffpa_fwd_dropout, ffpa_dropout_keep): host-side checks only
KEEP = 0x90_0000_0000


def dcheck(p=0.1, keep=KEEP, o=O, lse=L, Nkv=300, **kw):
    args = dict(B=2, Hq=4, Hkv=2, Nq=200, D=512, scale=math.nan, causal=False, dtype=ffpa.FFPA_BF16)
    args.update(kw)
    return ffpa.ffpa_check_dropout_args(Q, K, V, None, o, lse, args["B"], args["Hq"], args["Hkv"], args["Nq"], Nkv,
                                        args["D"], args["scale"], args["causal"], args["dtype"], keep, p)


def test_dropout_valid_arguments_pass():
    assert dcheck() == ffpa.OK
    assert dcheck(p=0.0) == ffpa.OK
    assert dcheck(p=0.999) == ffpa.OK
    assert dcheck(D=576) == ffpa.OK
    assert dcheck(D=80) == ffpa.OK  # padded head dims take dropout too


@pytest.mark.parametrize("kw,status", [
    (dict(p=1.0), ffpa.ERR_VALUE), (dict(p=-0.5), ffpa.ERR_VALUE), (dict(p=float("nan")), ffpa.ERR_VALUE),
    (dict(keep=None), ffpa.ERR_VALUE), (dict(keep=KEEP + 2), ffpa.ERR_VALUE),
    (dict(keep=O), ffpa.ERR_VALUE),            # o overlaps the keep words
    (dict(dtype=5), ffpa.ERR_TYPE), (dict(D=100), ffpa.ERR_UNSUPPORTED), (dict(Hkv=3), ffpa.ERR_VALUE),
])
def test_dropout_argument_errors(kw, status):
    assert dcheck(**kw) == status


def test_dropout_keep_rejects_before_launching():
    lib = ffpa.library()
    for args in ((KEEP, 0, 1, 1, 1, 0.1), (KEEP, 1, 1, 1, 1, 1.0), (KEEP, 1, 1, 1, 1, -0.1), (None, 1, 1, 1, 1, 0.1),
                 (KEEP + 1, 1, 1, 1, 1, 0.1)):
        assert ffpa.ffpa_dropout_keep(*args, 0, 0, None) == ffpa.ERR_VALUE
    ffpa.ffpa_dropout_keep(KEEP, 1, 1, 1, 1, 1.0, 0, 0, None)
    assert b"[0, 1)" in lib.ffpa_last_error_detail()


# ---- fp8 entry (ffpa_fwd_fp8): host checks only
DQ, DK, DV = 0x90_0000_0000, 0xA0_0000_0000, 0xB0_0000_0000


def fcheck(B=1, Hq=2, Hkv=1, Nq=100, Nkv=130, D=512, scale=math.nan, causal=False, out=ffpa.FFPA_BF16, q=Q, k=K,
           v=V, o=O, lse=L, dq=DQ, dk=DK, dv=DV, mask=None):
    return ffpa.ffpa_check_fp8_args(q, k, v, dq, dk, dv, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, out)


def test_fp8_valid_arguments_pass():
    assert fcheck() == ffpa.OK and detail() == ""
    for D in range(16, 1025, 16):
        assert fcheck(D=D) == ffpa.OK, D
    assert fcheck(dq=None, dk=None, dv=None) == ffpa.OK
    assert fcheck(out=ffpa.FFPA_FP16, causal=True, Nq=100, Nkv=130) == ffpa.OK
    assert fcheck(mask=mdesc(kind=ffpa.MASK_BOOL_U8)) == ffpa.OK


@pytest.mark.parametrize("kw,status", [
    (dict(out=2), ffpa.ERR_TYPE), (dict(D=8), ffpa.ERR_UNSUPPORTED), (dict(D=520), ffpa.ERR_UNSUPPORTED),
    (dict(D=100), ffpa.ERR_UNSUPPORTED), (dict(D=1040), ffpa.ERR_UNSUPPORTED), (dict(Hq=3, Hkv=2), ffpa.ERR_VALUE),
    (dict(causal=True, Nq=131, Nkv=130), ffpa.ERR_VALUE), (dict(dq=DQ + 2), ffpa.ERR_VALUE),
    (dict(dv=O), ffpa.ERR_VALUE), (dict(q=Q + 8), ffpa.ERR_VALUE), (dict(o=Q), ffpa.ERR_VALUE),
])
def test_fp8_argument_errors(kw, status):
    assert fcheck(**kw) == status, kw
    assert detail() != ""


def test_fp8_kernel_head_dim():
    lib = ffpa.library()
    for D in range(16, 1025, 16):
        want = (D + 127) // 128 * 128 if D <= 512 else (768 if D <= 768 else 1024)
        assert lib.ffpa_fp8_kernel_head_dim(D) == want, D
    for bad in (0, 8, 100, 520, 1040, 2048):
        assert lib.ffpa_fp8_kernel_head_dim(bad) == 0


# ---- backward entries: host checks and the workspace (one float per query row, for Delta)
def test_bwd_workspace_is_delta_only():
    for (B, Hq, Hkv, Nq, Nkv, D) in [(1, 8, 8, 4096, 4096, 512), (2, 3, 1, 5, 7, 64), (4, 16, 16, 1024, 4096, 1024)]:
        want = (4 * B * Hq * Nq + 255) // 256 * 256
        assert ffpa.ffpa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D) == want
    assert ffpa.ffpa_bwd_workspace_size(1, 3, 2, 8, 8, 64) == 0  # Hq not a multiple of Hkv


def bwd(D=512, Nq=100, Nkv=130, B=1, Hq=2, Hkv=1, causal=False, ws=M, nbytes=1 << 20):
    return ffpa.ffpa_bwd(Q, K, V, O, O + 0x1000_0000, L, None, DQ, DK, DV, B, Hq, Hkv, Nq, Nkv, D, math.nan, causal,
                         ffpa.FFPA_BF16, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=100), ffpa.ERR_UNSUPPORTED), (dict(D=1088), ffpa.ERR_UNSUPPORTED), (dict(D=4), ffpa.ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), ffpa.ERR_VALUE), (dict(causal=True, Nq=200, Nkv=100), ffpa.ERR_VALUE),
    (dict(Nq=(1 << 31) // 512), ffpa.ERR_UNSUPPORTED), (dict(ws=None), ffpa.ERR_VALUE),
    (dict(nbytes=16), ffpa.ERR_VALUE), (dict(ws=M + 16), ffpa.ERR_VALUE)])
def test_bwd_argument_errors(kw, status):
    assert bwd(**kw) == status, detail()
