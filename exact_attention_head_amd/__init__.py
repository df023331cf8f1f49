"""MI355X (gfx950) exact large-head-dim attention forward.

``attn`` computes O = softmax(scale * Q K^T + mask) V and, on request, the fp32 natural-log LSE,
with the semantics of ffpa_attn_func on the ffpa-attn "API Reference" page: SDPA-style layout
[B, H, N, D], GQA/MQA through enable_gqa, cross-attention (Nq != Nkv), tail-aligned causal masking
(row r sees keys k <= r + Nkv - Nq, requiring Nkv >= Nq), boolean masks (True takes part) and
additive floating masks, scale = 1/sqrt(D) by default, and SDPA-style attention dropout
(dropout_p: keep decisions drawn on the GPU by Philox4x32-10, or given).  ``attn_varlen`` is the packed
variable-length form of ffpa_attn_varlen_func on the same page: THD tensors [T, H, D], cumulative
sequence offsets, the longest lengths, and an [Hq, Tq] LSE.  ``attn_fp8`` is the FP8 attention of
the README: e4m3 tensors with per-head dequantisation factors, both products on the fp8 matrix core.

Everything here is argument marshalling around the C ABI of ``libffpa.so`` (include/ffpa.h):
tensors are passed by device pointer, outputs are allocated with torch, and the work is enqueued
on torch's current HIP stream.  There is no fallback path: if the library is missing, importing
works but every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = ["attn", "attn_varlen", "attn_fp8", "ffpa_fwd_fp8", "ffpa_check_fp8_args", "ffpa_fwd", "ffpa_check_args", "ffpa_fwd_varlen", "ffpa_check_varlen_args",
           "ffpa_check_cu_seqlens", "ffpa_fwd_strided", "ffpa_check_strided_args", "LayoutDesc", "ffpa_bwd",
           "ffpa_bwd_workspace_size", "ffpa_bwd_dropout", "ffpa_bwd_mask_grad", "ffpa_bwd_noalloc", "ffpa_dropout_keep", "ffpa_fwd_dropout", "ffpa_check_dropout_args",
           "dropout_keep", "attn_backward", "attn_with_grad", "AttnFunction", "library", "rows_per_block", "kernel_head_dim", "kernel_name", "FFPA_BF16", "FFPA_FP16",
           "MASK_NONE", "MASK_BOOL_U8", "MASK_ADD_F32", "MASK_ADD_BF16", "MASK_ADD_FP16", "MaskDesc",
           "ffpa_attn_func", "ffpa_attn_varlen_func"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libffpa.so")

FFPA_BF16, FFPA_FP16 = 0, 1
MASK_NONE, MASK_BOOL_U8, MASK_ADD_F32, MASK_ADD_BF16, MASK_ADD_FP16 = 0, 1, 2, 3, 4
OK, ERR_TYPE, ERR_VALUE, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3, 4

EXPORTED = ("ffpa_fwd", "ffpa_check_args", "ffpa_status_string", "ffpa_last_error_detail", "ffpa_rows_per_block",
            "ffpa_kernel_name", "ffpa_fwd_varlen", "ffpa_check_varlen_args", "ffpa_check_cu_seqlens",
            "ffpa_fwd_strided", "ffpa_check_strided_args", "ffpa_bwd", "ffpa_bwd_workspace_size",
            "ffpa_dropout_keep", "ffpa_fwd_dropout", "ffpa_check_dropout_args", "ffpa_bwd_dropout",
            "ffpa_kernel_head_dim", "ffpa_fwd_fp8", "ffpa_check_fp8_args", "ffpa_fp8_kernel_head_dim",
            "ffpa_clock_stamps", "ffpa_bwd_mask_grad", "ffpa_bwd_noalloc")


class MaskDesc(ctypes.Structure):
    """ffpa_mask_t: element (b, h, r, k) at data + b*stride_b + h*stride_h + r*stride_q + k*stride_k."""
    _fields_ = [("data", ctypes.c_void_p), ("kind", ctypes.c_int32), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_q", ctypes.c_int64), ("stride_k", ctypes.c_int64)]


class LayoutDesc(ctypes.Structure):
    """ffpa_layout_t: element strides {batch, head, row} of Q, K, V and O (head-dim stride 1)."""
    _fields_ = [("q", ctypes.c_int64 * 3), ("k", ctypes.c_int64 * 3), ("v", ctypes.c_int64 * 3),
                ("o", ctypes.c_int64 * 3)]


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libffpa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with exact_attention_head_amd/build.py "
                           "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    i64, p, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    args = [p, p, p, ctypes.POINTER(MaskDesc), p, p, i64, i64, i64, i64, i64, i64, f32, i32, i32]
    lib.ffpa_fwd.argtypes = args + [p]
    lib.ffpa_fwd.restype = i32
    lib.ffpa_check_args.argtypes = args
    lib.ffpa_check_args.restype = i32
    lib.ffpa_status_string.argtypes = [i32]
    lib.ffpa_status_string.restype = ctypes.c_char_p
    lib.ffpa_last_error_detail.argtypes = []
    lib.ffpa_last_error_detail.restype = ctypes.c_char_p
    lib.ffpa_rows_per_block.argtypes = [i64]
    lib.ffpa_rows_per_block.restype = i32
    lib.ffpa_kernel_name.argtypes = [i64]
    lib.ffpa_kernel_name.restype = ctypes.c_char_p
    lib.ffpa_kernel_head_dim.argtypes = [i64]
    lib.ffpa_kernel_head_dim.restype = i64
    fargs = [p, p, p, p, p, p, ctypes.POINTER(MaskDesc), p, p, i64, i64, i64, i64, i64, i64, f32, i32, i32]
    lib.ffpa_fwd_fp8.argtypes = fargs + [p]
    lib.ffpa_fwd_fp8.restype = i32
    lib.ffpa_check_fp8_args.argtypes = fargs
    lib.ffpa_check_fp8_args.restype = i32
    lib.ffpa_fp8_kernel_head_dim.argtypes = [i64]
    lib.ffpa_fp8_kernel_head_dim.restype = i64
    lib.ffpa_clock_stamps.argtypes = [p]
    lib.ffpa_clock_stamps.restype = i32
    vargs = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, i64, f32, i32, i32]
    lib.ffpa_fwd_varlen.argtypes = vargs + [p]
    lib.ffpa_fwd_varlen.restype = i32
    lib.ffpa_check_varlen_args.argtypes = vargs
    lib.ffpa_check_varlen_args.restype = i32
    lib.ffpa_check_cu_seqlens.argtypes = [ctypes.POINTER(ctypes.c_int32), i64, i64, i64]
    lib.ffpa_check_cu_seqlens.restype = i32
    sargs = [p, p, p, ctypes.POINTER(MaskDesc), p, p, i64, i64, i64, i64, i64, i64, ctypes.POINTER(LayoutDesc), f32,
             i32, i32]
    lib.ffpa_fwd_strided.argtypes = sargs + [p]
    lib.ffpa_fwd_strided.restype = i32
    lib.ffpa_check_strided_args.argtypes = sargs
    lib.ffpa_check_strided_args.restype = i32
    lib.ffpa_bwd.argtypes = [p, p, p, p, p, p, ctypes.POINTER(MaskDesc), p, p, p, i64, i64, i64, i64, i64, i64, f32,
                             i32, i32, p, ctypes.c_size_t, p]
    lib.ffpa_bwd.restype = i32
    lib.ffpa_bwd_dropout.argtypes = [p, p, p, p, p, p, ctypes.POINTER(MaskDesc), p, p, p, i64, i64, i64, i64, i64, i64,
                                     f32, i32, i32, p, f32, p, ctypes.c_size_t, p]
    lib.ffpa_bwd_dropout.restype = i32
    lib.ffpa_bwd_mask_grad.argtypes = [p, p, p, p, p, p, ctypes.POINTER(MaskDesc), p, p, p, p, i64, i64, i64, i64, i64,
                                       i64, f32, i32, i32, p, f32, p, ctypes.c_size_t, p]
    lib.ffpa_bwd_mask_grad.restype = i32
    lib.ffpa_bwd_noalloc.argtypes = [p, p, p, p, p, p, ctypes.POINTER(MaskDesc), p, p, p, i64, i64, i64, i64, i64, i64,
                                     f32, i32, i32, p]
    lib.ffpa_bwd_noalloc.restype = i32
    lib.ffpa_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64]
    lib.ffpa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ffpa_dropout_keep.argtypes = [p, i64, i64, i64, i64, f32, ctypes.c_uint64, ctypes.c_uint32, p]
    lib.ffpa_dropout_keep.restype = i32
    lib.ffpa_fwd_dropout.argtypes = args + [p, f32, p]
    lib.ffpa_fwd_dropout.restype = i32
    lib.ffpa_check_dropout_args.argtypes = args + [p, f32]
    lib.ffpa_check_dropout_args.restype = i32
    _lib = lib
    return lib


def _raise(status: int) -> None:
    lib = library()
    detail = lib.ffpa_last_error_detail().decode()
    name = lib.ffpa_status_string(status).decode()
    msg = f"ffpa: {name}: {detail}" if detail else f"ffpa: {name}"
    raise {ERR_TYPE: TypeError, ERR_VALUE: ValueError, ERR_UNSUPPORTED: NotImplementedError}.get(status,
                                                                                                 RuntimeError)(msg)


def ffpa_fwd(q, k, v, mask: Optional[MaskDesc], o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype,
             stream) -> int:
    """The raw C entry point: pointers are integers (device addresses), returns the status code."""
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_fwd(q, k, v, m, o, lse, B, Hq, Hkv, Nq, Nkv, D, ctypes.c_float(scale), int(is_causal),
                              dtype, stream)


def ffpa_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, mask: Optional[MaskDesc], o, lse, B, Hq, Hkv, Nq, Nkv,
                 D, scale, is_causal, out_dtype, stream) -> int:
    """The raw fp8 entry point: pointers are integers (device addresses, None for absent factors)."""
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, m, o, lse, B, Hq, Hkv, Nq, Nkv, D,
                                  ctypes.c_float(scale), int(is_causal), out_dtype, stream)


def ffpa_check_fp8_args(q, k, v, q_descale, k_descale, v_descale, mask: Optional[MaskDesc], o, lse, B, Hq, Hkv, Nq,
                        Nkv, D, scale, is_causal, out_dtype) -> int:
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_check_fp8_args(q, k, v, q_descale, k_descale, v_descale, m, o, lse, B, Hq, Hkv, Nq, Nkv, D,
                                         ctypes.c_float(scale), int(is_causal), out_dtype)


def ffpa_dropout_keep(keep, B, Hq, Nq, Nkv, p, seed, offset, stream) -> int:
    """The raw C entry point drawing dropout keep bits into keep (a device address)."""
    return library().ffpa_dropout_keep(keep, B, Hq, Nq, Nkv, ctypes.c_float(p), seed & (2**64 - 1),
                                       offset & 0xFFFFFFFF, stream)


def ffpa_fwd_dropout(q, k, v, mask: Optional[MaskDesc], o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype,
                     keep, dropout_p, stream) -> int:
    """The raw C entry point of the forward with dropout: pointers are integers, returns the status."""
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_fwd_dropout(q, k, v, m, o, lse, B, Hq, Hkv, Nq, Nkv, D, ctypes.c_float(scale),
                                      int(is_causal), dtype, keep, ctypes.c_float(dropout_p), stream)


def ffpa_check_dropout_args(q, k, v, mask: Optional[MaskDesc], o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal,
                            dtype, keep, dropout_p) -> int:
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_check_dropout_args(q, k, v, m, o, lse, B, Hq, Hkv, Nq, Nkv, D, ctypes.c_float(scale),
                                             int(is_causal), dtype, keep, ctypes.c_float(dropout_p))


def dropout_keep(B: int, Hq: int, Nq: int, Nkv: int, p: float, seed: int, offset: int = 0, device=None):
    """Keep bits of attention dropout, drawn on the GPU: int32 [B, Hq, Nq, ceil(Nkv / 32)] holding
    the uint32 words of ffpa_dropout_keep (bit i of word w keeps key 32 w + i)."""
    import torch

    device = torch.device("cuda") if device is None else torch.device(device)
    keep = torch.empty((B, Hq, Nq, (Nkv + 31) // 32), dtype=torch.int32, device=device)
    with torch.cuda.device(device):
        stream = torch.cuda.current_stream(device).cuda_stream
        st = ffpa_dropout_keep(keep.data_ptr(), B, Hq, Nq, Nkv, float(p), int(seed), int(offset), stream)
    if st != OK:
        _raise(st)
    return keep


def ffpa_check_args(q, k, v, mask: Optional[MaskDesc], o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal,
                    dtype) -> int:
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_check_args(q, k, v, m, o, lse, B, Hq, Hkv, Nq, Nkv, D, ctypes.c_float(scale),
                                     int(is_causal), dtype)


def ffpa_fwd_strided(q, k, v, mask: Optional[MaskDesc], o, lse, B, Hq, Hkv, Nq, Nkv, D, layout: LayoutDesc, scale,
                     is_causal, dtype, stream) -> int:
    """The raw strided entry point: pointers are integers (device addresses), returns the status code."""
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_fwd_strided(q, k, v, m, o, lse, B, Hq, Hkv, Nq, Nkv, D, ctypes.byref(layout),
                                      ctypes.c_float(scale), int(is_causal), dtype, stream)


def ffpa_check_strided_args(q, k, v, mask: Optional[MaskDesc], o, lse, B, Hq, Hkv, Nq, Nkv, D, layout, scale,
                            is_causal, dtype) -> int:
    m = ctypes.byref(mask) if mask is not None else None
    lay = ctypes.byref(layout) if layout is not None else None
    return library().ffpa_check_strided_args(q, k, v, m, o, lse, B, Hq, Hkv, Nq, Nkv, D, lay, ctypes.c_float(scale),
                                             int(is_causal), dtype)


def _strides3(t):
    """{batch, head, row} element strides of a [B, H, N, D] tensor usable in place (head-dim stride 1,
    16-byte aligned, strides multiples of 8, rows not overlapping), else None.  A batch or head
    dimension of size 1 counts as stride 0 and a single row as stride D."""
    D = t.shape[3]
    if t.stride(3) != 1 and D > 1:
        return None
    st = [0 if t.shape[0] == 1 else t.stride(0), 0 if t.shape[1] == 1 else t.stride(1),
          D if t.shape[2] == 1 else t.stride(2)]
    if t.data_ptr() % 16 or any(x % 8 or x < 0 for x in st) or st[2] < D:
        return None
    return st


def _strided_plan(ptrs, strides, B, Hq, Hkv, Nq, Nkv, D, dtype) -> Optional[LayoutDesc]:
    """The layout descriptor for reading Q, K, V and writing O in place through ffpa_fwd_strided
    (ptrs: their device addresses; strides: their {batch, head, row} element strides), or None when the
    strided entry cannot address them (ffpa_check_strided_args: FFPA_ERR_UNSUPPORTED, e.g. row strides
    or one head's rows beyond the kernels' 32-bit buffer offsets, or K and V row strides that differ):
    the caller then works on contiguous copies, which the dense entry takes.  Host-only."""
    lay = LayoutDesc(*((ctypes.c_int64 * 3)(*st) for st in strides))
    st = ffpa_check_strided_args(ptrs[0], ptrs[1], ptrs[2], None, ptrs[3], None, B, Hq, Hkv, Nq, Nkv, D, lay,
                                 math.nan, False, dtype)
    return None if st == ERR_UNSUPPORTED else lay


def ffpa_fwd_varlen(q, k, v, cu_q, cu_k, o, lse, B, Hq, Hkv, Tq, Tk, max_q, max_k, D, scale, is_causal, dtype,
                    stream) -> int:
    """The raw packed entry point: pointers are integers (device addresses), returns the status code."""
    return library().ffpa_fwd_varlen(q, k, v, cu_q, cu_k, o, lse, B, Hq, Hkv, Tq, Tk, max_q, max_k, D,
                                     ctypes.c_float(scale), int(is_causal), dtype, stream)


def ffpa_check_varlen_args(q, k, v, cu_q, cu_k, o, lse, B, Hq, Hkv, Tq, Tk, max_q, max_k, D, scale, is_causal,
                           dtype) -> int:
    return library().ffpa_check_varlen_args(q, k, v, cu_q, cu_k, o, lse, B, Hq, Hkv, Tq, Tk, max_q, max_k, D,
                                            ctypes.c_float(scale), int(is_causal), dtype)


def ffpa_check_cu_seqlens(offsets, T: int, max_seqlen: int) -> int:
    """Checks a host sequence of B+1 cumulative offsets (ints); returns the status code."""
    arr = (ctypes.c_int32 * len(offsets))(*[int(x) for x in offsets])
    return library().ffpa_check_cu_seqlens(arr, len(offsets) - 1, T, max_seqlen)


def rows_per_block(D: int) -> int:
    return int(library().ffpa_rows_per_block(D))


def kernel_head_dim(D: int) -> int:
    """Head dim of the kernel serving tensors of head dim D (D itself, or the next compiled one up whose
    columns past D are padding); 0 if unsupported."""
    return int(library().ffpa_kernel_head_dim(D))


def kernel_name(D: int):
    """Name of the GPU kernel serving head dim D (None if D is unsupported)."""
    name = library().ffpa_kernel_name(D)
    return None if name is None else name.decode()


def _mask_desc(attn_mask, B, Hq, Nq, Nkv):
    """MaskDesc for a torch mask broadcastable to [B, Hq, Nq, Nkv] (plus the tensor to keep alive)."""
    import torch

    kinds = {torch.bool: MASK_BOOL_U8, torch.float32: MASK_ADD_F32, torch.bfloat16: MASK_ADD_BF16,
             torch.float16: MASK_ADD_FP16}
    if attn_mask.dtype not in kinds:
        raise TypeError(f"attn_mask dtype {attn_mask.dtype} is not bool, float32, bfloat16 or float16")
    m = attn_mask
    if m.dim() > 4:
        raise ValueError("attn_mask has more than 4 dims")
    while m.dim() < 4:
        m = m.unsqueeze(0)
    for have, want in zip(m.shape, (B, Hq, Nq, Nkv)):
        if have not in (1, want):
            raise ValueError(f"attn_mask of shape {tuple(attn_mask.shape)} is not broadcastable to "
                             f"{(B, Hq, Nq, Nkv)}")
    if m.shape[3] != Nkv or m.stride(3) != 1:
        # keys must be contiguous in memory: lay the mask out densely in its own (broadcast) shape
        m = m.expand(m.shape[0], m.shape[1], m.shape[2], Nkv).contiguous()
    strides = [0 if m.shape[i] == 1 else m.stride(i) for i in range(3)]
    desc = MaskDesc(m.data_ptr(), kinds[m.dtype], strides[0], strides[1], strides[2], 1)
    return desc, m


def _records_grad(torch, tensors) -> bool:
    """Whether autograd would record an operation on these tensors (None entries are skipped)."""
    return torch.is_grad_enabled() and any(t is not None and t.requires_grad for t in tensors)


def attn(query, key, value, attn_mask=None, dropout_p: float = 0.0, is_causal: bool = False,
         scale: Optional[float] = None, enable_gqa: bool = False, return_lse: bool = False, out=None,
         dropout_seed: Optional[int] = None, dropout_keep=None, return_dropout_keep: bool = False):
    """SDPA-aligned forward.  query [B, Hq, Nq, D]; key/value [B, Hkv, Nkv, D]; bf16 or fp16.

    Returns O [B, Hq, Nq, D] (dtype of query), or (O, LSE [B, Hq, Nq] float32) with return_lse.
    Strided views (for instance a [B, N, H, D] tensor transposed to [B, H, N, D]) are read in place
    through ffpa_fwd_strided when their strides allow it, and so is a strided ``out``.

    Dropout (0 < dropout_p < 1, SDPA-style: each softmax weight kept with probability 1 - p, kept
    ones scaled by 1 / (1 - p); the LSE is unchanged): the keep bits are drawn on the GPU by
    ffpa_dropout_keep with seed ``dropout_seed`` (default: drawn from torch's CPU generator) and
    offset 0, or taken from ``dropout_keep`` (int32 [B, Hq, Nq, ceil(Nkv / 32)] words, any bits;
    dropout_p then sets the scaling).  ``return_dropout_keep`` appends the keep words to the result.
    Dropout runs on contiguous tensors (others are copied first).

    Autograd, as for SDPA: with grad mode on and query, key, value or a floating attn_mask requiring
    grad, the call is recorded (``attn_with_grad``): the backward runs ffpa_bwd, ffpa_bwd_dropout or
    ffpa_bwd_mask_grad, and the LSE is returned without a gradient.  ``out``, ``dropout_keep`` and
    ``return_dropout_keep`` are not recorded and raise in that case.
    """
    import torch

    if not (0.0 <= float(dropout_p) < 1.0):
        raise ValueError("dropout_p must lie in [0, 1)")
    dropping = dropout_p != 0.0 or dropout_keep is not None
    for name, t in (("query", query), ("key", key), ("value", value)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D tensor [B, H, N, D]")
    if _records_grad(torch, (query, key, value, attn_mask)):
        if out is not None or dropout_keep is not None or return_dropout_keep:
            raise ValueError("out, dropout_keep and return_dropout_keep are not recorded for autograd: call "
                             "under torch.no_grad(), or leave them out")
        o, lse = AttnFunction().apply(query, key, value, attn_mask, is_causal, scale, enable_gqa, float(dropout_p),
                                      dropout_seed)
        return (o, lse) if return_lse else o
    if query.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"query dtype {query.dtype} is neither bfloat16 nor float16")
    if key.dtype != query.dtype or value.dtype != query.dtype:
        raise TypeError("query, key and value must share one dtype")
    if not (query.is_cuda and key.device == query.device and value.device == query.device):
        raise ValueError("query, key and value must live on the same GPU")
    B, Hq, Nq, D = query.shape
    Bk, Hkv, Nkv, Dk = key.shape
    if tuple(value.shape) != tuple(key.shape):
        raise ValueError("key and value must share [B, Hkv, Nkv, D]")
    if Bk != B or Dk != D:
        raise ValueError("query and key disagree on batch or head dim")
    if Hq != Hkv and not enable_gqa:
        raise ValueError("Hq != Hkv needs enable_gqa=True")
    # strided views (e.g. [B, N, H, D] storage seen as [B, H, N, D]) are read in place when the
    # kernels can address them; anything else is made contiguous first
    sq, sk, sv = _strides3(query), _strides3(key), _strides3(value)
    in_place = sq is not None and sk is not None and sv is not None and sk[2] == sv[2]
    if in_place:
        q, k, v = query, key, value
    else:
        q, k, v = query.contiguous(), key.contiguous(), value.contiguous()
        sq, sk, sv = _strides3(q), _strides3(k), _strides3(v)
    dtype = FFPA_BF16 if query.dtype == torch.bfloat16 else FFPA_FP16
    if out is None:
        o = torch.empty((B, Hq, Nq, D), dtype=query.dtype, device=query.device)
    else:
        if tuple(out.shape) != (B, Hq, Nq, D) or out.dtype != query.dtype or _strides3(out) is None:
            raise ValueError("out must be a [B, Hq, Nq, D] tensor of the query dtype, unit stride along D, "
                             "16-byte aligned, other strides multiples of 8")
        o = out
    so = _strides3(o)
    contiguous = all(t.is_contiguous() for t in (q, k, v, o))
    if not contiguous and None in (sq, sk, sv):
        raise ValueError("query, key and value must be 16-byte aligned")
    lay, o_user = None, o
    if not contiguous and not dropping:
        lay = _strided_plan([t.data_ptr() for t in (q, k, v, o)], [sq, sk, sv, so], B, Hq, Hkv, Nq, Nkv, D, dtype)
        if lay is None:  # a layout the kernels cannot address in place: contiguous copies instead
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            if not o.is_contiguous():
                o = torch.empty((B, Hq, Nq, D), dtype=query.dtype, device=query.device)
            contiguous = True
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=query.device) if return_lse else None
    desc, keep = (None, None) if attn_mask is None else _mask_desc(attn_mask.to(query.device), B, Hq, Nq, Nkv)
    sc = math.nan if scale is None else float(scale)
    if dropping:
        return _attn_dropout(q, k, v, o, out, lse, desc, keep, B, Hq, Hkv, Nq, Nkv, D, sc, is_causal, dtype,
                             float(dropout_p), dropout_seed, dropout_keep, return_lse, return_dropout_keep)
    with torch.cuda.device(query.device):
        stream = torch.cuda.current_stream(query.device).cuda_stream
        lp = lse.data_ptr() if lse is not None else None
        if contiguous:
            st = ffpa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), desc, o.data_ptr(), lp, B, Hq, Hkv, Nq, Nkv, D,
                          sc, bool(is_causal), dtype, stream)
        else:
            st = ffpa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), desc, o.data_ptr(), lp, B, Hq, Hkv, Nq,
                                  Nkv, D, lay, sc, bool(is_causal), dtype, stream)
    del keep
    if st != OK:
        _raise(st)
    if o is not o_user:
        o_user.copy_(o)
    return (o_user, lse) if return_lse else o_user


def attn_fp8(query, key, value, q_descale=None, k_descale=None, v_descale=None, attn_mask=None,
             is_causal: bool = False, scale: Optional[float] = None, enable_gqa: bool = False,
             return_lse: bool = False, out_dtype=None, out=None):
    """FP8 attention forward (ffpa_fwd_fp8).  query [B, Hq, Nq, D], key/value [B, Hkv, Nkv, D] are
    torch.float8_e4m3fn tensors on the GPU; q_descale [B, Hq], k_descale and v_descale [B, Hkv] are
    positive float32 per-head dequantisation factors (None = 1), so that the attention runs over
    descale * tensor.  O is returned in out_dtype (torch.bfloat16 by default, or torch.float16), and
    with return_lse also the fp32 [B, Hq, Nq] LSE.  Other arguments as for ``attn``; 16 <= D <= 1024
    with D % 16 == 0.  Non-contiguous inputs are copied to contiguous ones first."""
    import torch

    for name, t in (("query", query), ("key", key), ("value", value)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D tensor [B, H, N, D]")
        if t.dtype != torch.float8_e4m3fn:
            raise TypeError(f"{name} dtype {t.dtype} is not float8_e4m3fn")
    if not (query.is_cuda and key.device == query.device and value.device == query.device):
        raise ValueError("query, key and value must live on the same GPU")
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"out_dtype {out_dtype} is neither bfloat16 nor float16")
    B, Hq, Nq, D = query.shape
    Bk, Hkv, Nkv, Dk = key.shape
    if tuple(value.shape) != tuple(key.shape) or Bk != B or Dk != D:
        raise ValueError("query, key and value disagree on [B, H, N, D]")
    if Hq != Hkv and not enable_gqa:
        raise ValueError("Hq != Hkv needs enable_gqa=True")
    q, k, v = query.contiguous(), key.contiguous(), value.contiguous()
    facs = []
    for name, f, heads in (("q_descale", q_descale, Hq), ("k_descale", k_descale, Hkv), ("v_descale", v_descale, Hkv)):
        if f is None:
            facs.append(None)
            continue
        if not isinstance(f, torch.Tensor) or f.numel() != B * heads:
            raise ValueError(f"{name} must hold B * heads = {B * heads} factors")
        facs.append(f.to(device=query.device, dtype=torch.float32).contiguous())
    if out is None:
        o = torch.empty((B, Hq, Nq, D), dtype=out_dtype, device=query.device)
    else:
        if tuple(out.shape) != (B, Hq, Nq, D) or out.dtype != out_dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B, Hq, Nq, D] tensor of out_dtype")
        o = out
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=query.device) if return_lse else None
    desc, keep = (None, None) if attn_mask is None else _mask_desc(attn_mask.to(query.device), B, Hq, Nq, Nkv)
    sc = math.nan if scale is None else float(scale)
    with torch.cuda.device(query.device):
        stream = torch.cuda.current_stream(query.device).cuda_stream
        st = ffpa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), *[f.data_ptr() if f is not None else None
                                                                     for f in facs],
                          desc, o.data_ptr(), lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Nq, Nkv, D, sc,
                          bool(is_causal), FFPA_BF16 if out_dtype == torch.bfloat16 else FFPA_FP16, stream)
    del keep, facs
    if st != OK:
        _raise(st)
    return (o, lse) if return_lse else o


def _attn_dropout(q, k, v, o, out, lse, desc, mask_keep, B, Hq, Hkv, Nq, Nkv, D, sc, is_causal, dtype, p, seed,
                  keep, return_lse, return_keep):
    """attn with dropout: contiguous tensors, keep bits drawn (or given), ffpa_fwd_dropout."""
    import torch

    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    o_c = o if o.is_contiguous() else torch.empty((B, Hq, Nq, D), dtype=q.dtype, device=q.device)
    W = (Nkv + 31) // 32
    if keep is None:
        if seed is None:
            seed = int(torch.randint(0, 2**62, (1,)).item())
        keep = dropout_keep(B, Hq, Nq, Nkv, p, seed, 0, q.device)
    else:
        if not isinstance(keep, torch.Tensor) or keep.dtype != torch.int32 or tuple(keep.shape) != (B, Hq, Nq, W):
            raise ValueError(f"dropout_keep must be an int32 tensor of shape {(B, Hq, Nq, W)}")
        keep = keep.to(q.device).contiguous()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        lp = lse.data_ptr() if lse is not None else None
        st = ffpa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), desc, o_c.data_ptr(), lp, B, Hq, Hkv, Nq, Nkv,
                              D, sc, bool(is_causal), dtype, keep.data_ptr(), p, stream)
    del mask_keep
    if st != OK:
        _raise(st)
    if o_c is not o:
        o.copy_(o_c)
    res = (o, lse) if return_lse else (o,)
    if return_keep:
        res = res + (keep,)
    return res if len(res) > 1 else res[0]


# keyword arguments of ffpa_attn_varlen_func that this forward rejects when given a non-default value
# the page's extension keywords of ffpa_attn_func ("API Reference"): they choose among its NVIDIA
# implementations; this library has one gfx950 path
_BACKEND_KWARGS = ("backend", "forward_backend", "backward_backend")


def ffpa_attn_func(query, key, value, attn_mask=None, dropout_p: float = 0.0, is_causal: bool = False,
                   scale: Optional[float] = None, enable_gqa: bool = False, **kwargs):
    """``attn`` under the name and SDPA-aligned signature of ffpa_attn_func ("API Reference"), for code
    written against that page: returns O [B, Hq, Nq, D], recorded for autograd when an input requires
    grad.  The page's backend keywords (backend, forward_backend, backward_backend) are accepted and
    have no effect; any other keyword raises TypeError, as on the page."""
    for name in kwargs:
        if name not in _BACKEND_KWARGS:
            raise TypeError(f"unexpected keyword argument {name!r}")
    return attn(query, key, value, attn_mask=attn_mask, dropout_p=dropout_p, is_causal=is_causal, scale=scale,
                enable_gqa=enable_gqa)


_VARLEN_UNSUPPORTED = ("window_size", "softcap", "sink", "attention_mask", "attn_mask", "block_mask", "score_mod",
                       "aux_tensors", "seqused_k", "block_table", "num_splits", "alibi_slopes")


def attn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, *,
                dropout_p: float = 0.0, softmax_scale: Optional[float] = None, causal: bool = False,
                enable_gqa: bool = False, return_lse: bool = False, **kwargs):
    """Packed variable-length forward.  q [Tq, Hq, D]; k/v [Tk, Hkv, D]; cu_seqlens_* int32 [B+1]
    (cu_seqlens_k None: the query offsets, for self-attention).  Each sequence is attended on its
    own, with the tail-aligned causal rule of its own lengths.

    Returns O [Tq, Hq, D], or (O, LSE [Hq, Tq] float32) with return_lse.  The offsets are checked on
    a host copy (one device-to-host transfer) before the launch.  There is no backward: with grad mode
    on, inputs that require grad raise NotImplementedError.
    """
    import torch

    for name, val in kwargs.items():
        if name in _VARLEN_UNSUPPORTED:
            if val is not None and val is not False and not (name == "window_size" and tuple(val) == (-1, -1)):
                raise NotImplementedError(f"{name} is not supported")
        else:
            raise TypeError(f"unexpected keyword argument {name!r}")
    if dropout_p != 0.0:
        raise NotImplementedError("attention dropout is not implemented (dropout_p must be 0)")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3:
            raise ValueError(f"{name} must be a 3-D tensor [T, H, D]")
    if _records_grad(torch, (q, k, v)):
        # a result without a gradient would drop the attention's share of it without a word
        raise NotImplementedError("packed batches have no backward: call under torch.no_grad(), or run each "
                                  "sequence through attn")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"q dtype {q.dtype} is neither bfloat16 nor float16")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if cu_seqlens_k is None:
        cu_seqlens_k = cu_seqlens_q
    for name, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not isinstance(c, torch.Tensor) or c.dtype != torch.int32:
            raise TypeError(f"{name} must be an int32 tensor")
        if c.dim() != 1 or c.numel() < 2:
            raise ValueError(f"{name} must be 1-D with B+1 >= 2 entries")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    Tq, Hq, D = q.shape
    Tk, Hkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must share [Tk, Hkv, D]")
    if Dk != D:
        raise ValueError("q and k disagree on the head dim")
    if Hq != Hkv and not enable_gqa:
        raise ValueError("Hq != Hkv needs enable_gqa=True")
    B = cu_seqlens_q.numel() - 1
    for c, T, mx in ((cu_seqlens_q, Tq, max_seqlen_q), (cu_seqlens_k, Tk, max_seqlen_k)):
        st = ffpa_check_cu_seqlens(c.cpu().tolist(), T, int(mx))
        if st != OK:
            _raise(st)
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k and v must live on the same GPU")
    cq = cu_seqlens_q.to(q.device).contiguous()
    ck = cq if cu_seqlens_k is cu_seqlens_q else cu_seqlens_k.to(q.device).contiguous()
    qc, kc, vc = q.contiguous(), k.contiguous(), v.contiguous()
    dtype = FFPA_BF16 if q.dtype == torch.bfloat16 else FFPA_FP16
    o = torch.empty((Tq, Hq, D), dtype=q.dtype, device=q.device)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device) if return_lse else None
    sc = math.nan if softmax_scale is None else float(softmax_scale)

    def ptr(t):
        return t.data_ptr() if t is not None and t.numel() > 0 else None

    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = ffpa_fwd_varlen(ptr(qc), ptr(kc), ptr(vc), cq.data_ptr(), ck.data_ptr(), ptr(o), ptr(lse), B, Hq, Hkv,
                             Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), D, sc, bool(causal), dtype, stream)
    if st != OK:
        _raise(st)
    return (o, lse) if return_lse else o


# ffpa_attn_varlen_func ("API Reference") has attn_varlen's signature
ffpa_attn_varlen_func = attn_varlen


def ffpa_bwd(q, k, v, o, dout, lse, mask: Optional[MaskDesc], dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal,
             dtype, workspace, workspace_bytes, stream) -> int:
    """The raw backward entry point: pointers are integers (device addresses), returns the status code."""
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_bwd(q, k, v, o, dout, lse, m, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, ctypes.c_float(scale),
                              int(is_causal), dtype, workspace, workspace_bytes, stream)


def ffpa_bwd_dropout(q, k, v, o, dout, lse, mask: Optional[MaskDesc], dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale,
                     is_causal, dtype, keep, dropout_p, workspace, workspace_bytes, stream) -> int:
    """The raw backward entry point of the forward with dropout; returns the status code."""
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_bwd_dropout(q, k, v, o, dout, lse, m, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D,
                                      ctypes.c_float(scale), int(is_causal), dtype, keep, ctypes.c_float(dropout_p),
                                      workspace, workspace_bytes, stream)


def ffpa_bwd_mask_grad(q, k, v, o, dout, lse, mask: MaskDesc, dq, dk, dv, dmask, B, Hq, Hkv, Nq, Nkv, D, scale,
                       is_causal, dtype, keep, dropout_p, workspace, workspace_bytes, stream) -> int:
    """The raw backward entry point that also writes the additive mask's gradient; returns the status code."""
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_bwd_mask_grad(q, k, v, o, dout, lse, m, dq, dk, dv, dmask, B, Hq, Hkv, Nq, Nkv, D,
                                        ctypes.c_float(scale), int(is_causal), dtype, keep, ctypes.c_float(dropout_p),
                                        workspace, workspace_bytes, stream)


def ffpa_bwd_noalloc(q, k, v, o, dout, lse, mask: Optional[MaskDesc], dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale,
                     is_causal, dtype, stream) -> int:
    """The raw backward entry point that takes no workspace (its Delta buffer is built into the
    library, at most 2^22 query rows); returns the status code."""
    m = ctypes.byref(mask) if mask is not None else None
    return library().ffpa_bwd_noalloc(q, k, v, o, dout, lse, m, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D,
                                      ctypes.c_float(scale), int(is_causal), dtype, stream)


def ffpa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D) -> int:
    return int(library().ffpa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D))


def attn_backward(query, key, value, out, grad_out, lse, attn_mask=None, is_causal: bool = False,
                  scale: Optional[float] = None, dropout_p: float = 0.0, dropout_keep=None, mask_grad: bool = False):
    """Gradients (dQ, dK, dV) of ``attn`` at (query, key, value), given its output ``out``, its LSE and
    the output's gradient.  Tensors [B, H, N, D] as for ``attn``.  After a forward with dropout, pass its
    dropout_p and keep words (``return_dropout_keep``).  With mask_grad (a floating attn_mask), returns
    (dQ, dK, dV, dMask) with dMask the gradient of the additive mask: float32, in the mask's shape."""
    import torch

    q, k, v, o, do = (t.contiguous() for t in (query, key, value, out, grad_out))
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if tuple(o.shape) != tuple(q.shape) or tuple(do.shape) != tuple(q.shape):
        raise ValueError("out and grad_out must have the query's shape")
    if do.dtype != q.dtype or o.dtype != q.dtype:
        raise TypeError("out and grad_out must have the query's dtype")
    lse = lse.contiguous()
    if tuple(lse.shape) != (B, Hq, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be the forward's float32 [B, Hq, Nq] LSE")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = ffpa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if mask_grad and (attn_mask is None or not attn_mask.is_floating_point()):
        raise ValueError("mask_grad needs a floating (additive) attn_mask")
    if mask_grad:
        # a dimension the mask has at full size gets a gradient at full size, also if it is a
        # stride-0 view: lay such masks out densely so that only size-1 dimensions broadcast
        attn_mask = attn_mask.contiguous()
    desc, keep = (None, None) if attn_mask is None else _mask_desc(attn_mask.to(q.device), B, Hq, Nq, Nkv)
    dtype = FFPA_BF16 if q.dtype == torch.bfloat16 else FFPA_FP16
    sc = math.nan if scale is None else float(scale)
    dm = None
    if mask_grad:
        m4 = keep  # the 4-D mask the descriptor points into: size 1 exactly where the stride is 0
        dm = torch.empty((m4.shape[0], m4.shape[1], m4.shape[2], Nkv), dtype=torch.float32, device=q.device)
    if dropout_keep is not None:
        W = (Nkv + 31) // 32
        if dropout_keep.dtype != torch.int32 or tuple(dropout_keep.shape) != (B, Hq, Nq, W):
            raise ValueError(f"dropout_keep must be an int32 tensor of shape {(B, Hq, Nq, W)}")
        dropout_keep = dropout_keep.to(q.device).contiguous()
    elif dropout_p != 0.0:
        raise ValueError("a backward with dropout needs the forward's keep words (dropout_keep)")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if mask_grad:
            kp = dropout_keep.data_ptr() if dropout_keep is not None else None
            st = ffpa_bwd_mask_grad(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), desc, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dm.data_ptr(),
                                    B, Hq, Hkv, Nq, Nkv, D, sc, bool(is_causal), dtype, kp,
                                    float(dropout_p) if dropout_keep is not None else 0.0, ws.data_ptr(), nbytes,
                                    stream)
        elif dropout_keep is None:
            st = ffpa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), desc,
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nkv, D, sc, bool(is_causal),
                          dtype, ws.data_ptr(), nbytes, stream)
        else:
            st = ffpa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), desc, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq,
                                  Nkv, D, sc, bool(is_causal), dtype, dropout_keep.data_ptr(), float(dropout_p),
                                  ws.data_ptr(), nbytes, stream)
    del keep
    if st != OK:
        _raise(st)
    if not mask_grad:
        return dq, dk, dv
    if attn_mask.shape[-1] == 1 and Nkv != 1:
        # a mask constant along the keys adds the same value to a whole row of logits, which the
        # softmax cancels: its gradient is exactly zero
        dm = torch.zeros(attn_mask.shape, dtype=torch.float32, device=q.device)
    return dq, dk, dv, dm.reshape(attn_mask.shape)


def _autograd_function():
    import torch

    class AttnFunction(torch.autograd.Function):
        """Forward through ffpa_fwd or ffpa_fwd_dropout (keeping O, the LSE and the keep words),
        backward through ffpa_bwd or ffpa_bwd_dropout, or ffpa_bwd_mask_grad when a floating attn_mask
        needs its gradient."""

        @staticmethod
        def forward(ctx, query, key, value, attn_mask, is_causal, scale, enable_gqa, dropout_p=0.0, dropout_seed=None):
            keep = None
            if dropout_p != 0.0:
                o, lse, keep = attn(query, key, value, attn_mask=attn_mask, is_causal=is_causal, scale=scale,
                                    enable_gqa=enable_gqa, return_lse=True, dropout_p=dropout_p,
                                    dropout_seed=dropout_seed, return_dropout_keep=True)
            else:
                o, lse = attn(query, key, value, attn_mask=attn_mask, is_causal=is_causal, scale=scale,
                              enable_gqa=enable_gqa, return_lse=True)
            ctx.save_for_backward(query, key, value, o, lse)
            ctx.attn_mask, ctx.is_causal, ctx.scale = attn_mask, is_causal, scale
            ctx.dropout_p, ctx.keep = dropout_p, keep
            ctx.mark_non_differentiable(lse)
            return o, lse

        @staticmethod
        def backward(ctx, grad_o, grad_lse):
            query, key, value, o, lse = ctx.saved_tensors
            want_dm = bool(ctx.needs_input_grad[3]) and ctx.attn_mask is not None
            grads = attn_backward(query, key, value, o, grad_o, lse, attn_mask=ctx.attn_mask,
                                  is_causal=ctx.is_causal, scale=ctx.scale, dropout_p=ctx.dropout_p,
                                  dropout_keep=ctx.keep, mask_grad=want_dm)
            dq, dk, dv = grads[:3]
            dm = grads[3] if want_dm else None
            return dq, dk, dv, dm, None, None, None, None, None

    return AttnFunction


class _Lazy:
    fn = None


def AttnFunction():
    """The torch.autograd.Function class (created on first use, so importing needs no torch)."""
    if _Lazy.fn is None:
        _Lazy.fn = _autograd_function()
    return _Lazy.fn


def attn_with_grad(query, key, value, attn_mask=None, is_causal: bool = False, scale: Optional[float] = None,
                   enable_gqa: bool = False, dropout_p: float = 0.0, dropout_seed: Optional[int] = None):
    """``attn`` recorded for autograd: O is differentiable in query, key and value, and in a floating
    attn_mask that requires grad (with dropout, the keep words drawn by the forward are reused by the
    backward)."""
    o, _ = AttnFunction().apply(query, key, value, attn_mask, is_causal, scale, enable_gqa, dropout_p, dropout_seed)
    return o
