"""Exact-attention oracle (fp64, CPU).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users; the product path never imports this
package, and this package imports nothing from the product.

The arithmetic lives in ``attn_oracle.c`` (plain C, IEEE double, no
fast-math).  This module only marshals arguments: it hands the raw 16-bit
patterns of bf16/fp16 tensors and the mask's broadcast strides to the C code
and returns numpy float64 arrays.

What is computed (ffpa-attn "API Reference", ``ffpa_attn_func``): for every
query row r of batch b and query head h, with kv head ``h // (Hq // Hkv)``,

    logit_k = scale * <q_r, k_k> + bias(b, h, r, k)     (bias after scaling)
    logit_k = -inf  if causal and k > r + (Nkv - Nq)     (tail-aligned causal)
    LSE     = log(sum_k exp(logit_k))                     (natural log)
    O_r     = sum_k exp(logit_k - LSE) * v_k

``scale=None`` means 1/sqrt(D).  A boolean mask excludes keys whose entry is
false.  A row with every key excluded gets O = 0 and LSE = -inf.

``attention_rows_fp8`` takes fp8 e4m3 inputs with per-head dequantisation factors and computes the
same attention over the values they stand for.

``attention_varlen`` is the packed variable-length form (same page,
``ffpa_attn_varlen_func``): sequence b of a batch packed as [T, H, D] holds
query tokens cu_q[b] .. cu_q[b+1]-1 and key tokens cu_k[b] .. cu_k[b+1]-1 and
is attended on its own, with the causal rule of its own lengths; the LSE is
laid out [Hq, Tq].
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

MASK_NONE, MASK_BOOL_U8, MASK_ADD_F32, MASK_ADD_BF16, MASK_ADD_FP16 = 0, 1, 2, 3, 4
DT_BF16, DT_FP16 = 0, 1

# Planted-mistake switches (only for the tests proving the pins discriminate).
FAULT_NONE = 0
FAULT_TOPLEFT_CAUSAL = 1
FAULT_HEAD_MODULO = 2
FAULT_MASK_BEFORE_SCALE = 3
FAULT_LSE_LOG2 = 4
FAULT_DROP_LAST_KEY = 5
FAULT_V_TRANSPOSED = 6

_lib = None


def build(force: bool = True) -> str:
    """Compile ``attn_oracle.c`` into ``liboracle.so`` with gcc (no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_attn_rows.argtypes = [p, p, p, p, ctypes.c_int, i64, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                     ctypes.c_double, ctypes.c_int, ctypes.c_int, p, i64, p, p, p, ctypes.c_int,
                                     ctypes.c_int]
    lib.oracle_attn_rows_e4m3.restype = ctypes.c_int
    lib.oracle_attn_rows_e4m3.argtypes = [p, p, p, p, p, p, p, ctypes.c_int, i64, i64, i64, i64, i64, i64, i64, i64,
                                          i64, i64, ctypes.c_double, ctypes.c_int, p, i64, p, p, p, ctypes.c_int,
                                          ctypes.c_int]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_causal_visible.restype = i64
    lib.oracle_causal_visible.argtypes = [i64, i64, i64]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def causal_visible(r: int, nq: int, nkv: int) -> int:
    """Number of keys query row r sees under the tail-aligned causal rule."""
    return int(_load().oracle_causal_visible(r, nq, nkv))


def _bits16(t) -> np.ndarray:
    """Raw 16-bit patterns of a bf16/fp16 torch tensor (or a uint16 numpy array)."""
    if isinstance(t, np.ndarray):
        if t.dtype != np.uint16:
            raise TypeError("numpy inputs must hold raw uint16 bit patterns")
        return np.ascontiguousarray(t)
    import torch

    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"oracle inputs must be bf16 or fp16, got {t.dtype}")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _dtype_code(t) -> int:
    import torch

    if isinstance(t, np.ndarray):
        raise TypeError("pass dtype= with numpy inputs")
    return DT_FP16 if t.dtype == torch.float16 else DT_BF16


def _mask_args(mask, B, Hq, Nq, Nkv):
    """(array, kind, strides) for a torch mask broadcastable to [B, Hq, Nq, Nkv]."""
    import torch

    if mask is None:
        return None, MASK_NONE, (0, 0, 0, 0)
    m = mask.detach().cpu()
    while m.dim() < 4:
        m = m.unsqueeze(0)
    if m.dim() != 4:
        raise ValueError("mask must have at most 4 dims")
    for have, want in zip(m.shape, (B, Hq, Nq, Nkv)):
        if have not in (1, want):
            raise ValueError(f"mask shape {tuple(mask.shape)} does not broadcast to {(B, Hq, Nq, Nkv)}")
    m = m.contiguous()
    strides = [0 if m.shape[i] == 1 else m.stride(i) for i in range(4)]
    if m.dtype == torch.bool:
        arr, kind = m.to(torch.uint8).numpy(), MASK_BOOL_U8
    elif m.dtype == torch.float32:
        arr, kind = m.numpy(), MASK_ADD_F32
    elif m.dtype == torch.bfloat16:
        arr, kind = m.view(torch.int16).numpy().view(np.uint16), MASK_ADD_BF16
    elif m.dtype == torch.float16:
        arr, kind = m.view(torch.int16).numpy().view(np.uint16), MASK_ADD_FP16
    else:
        raise TypeError(f"unsupported mask dtype {m.dtype}")
    return np.ascontiguousarray(arr), kind, tuple(strides)


def attention_rows(q, k, v, rows: Sequence[int], mask=None, scale: Optional[float] = None, is_causal: bool = False,
                   want_probs: bool = False, threads: int = 0, fault: int = FAULT_NONE):
    """Selected rows of exact attention in fp64.

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nkv, D] (torch bf16/fp16, any device).
    rows: flat row indices ``(b * Hq + h) * Nq + r``.
    Returns (O [n, D] float64, LSE [n] float64) or, with want_probs, also P [n, Nkv].
    """
    lib = _load()
    B, Hq, Nq, D = (int(x) for x in q.shape)
    Bk, Hkv, Nkv, Dk = (int(x) for x in k.shape)
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("q/k/v shapes are inconsistent")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share one dtype")
    qb, kb, vb = _bits16(q), _bits16(k), _bits16(v)
    dtype = _dtype_code(q)
    if scale is None or (isinstance(scale, float) and math.isnan(scale)):
        scale = 1.0 / math.sqrt(D)
    marr, mkind, ms = _mask_args(mask, B, Hq, Nq, Nkv)
    rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows_arr.size
    if n and (rows_arr.min() < 0 or rows_arr.max() >= B * Hq * Nq):
        raise ValueError("row index out of range")
    O = np.zeros((n, D), dtype=np.float64)
    L = np.zeros((n,), dtype=np.float64)
    P = np.zeros((n, Nkv), dtype=np.float64) if want_probs else None
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = lib.oracle_attn_rows(ptr(qb), ptr(kb), ptr(vb), ptr(marr), mkind, ms[0], ms[1], ms[2], ms[3], B, Hq, Hkv,
                              Nq, Nkv, D, float(scale), int(bool(is_causal)), dtype, ptr(rows_arr), n, ptr(O), ptr(L),
                              ptr(P), int(threads), int(fault))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_rows failed with code {rc}")
    return (O, L, P) if want_probs else (O, L)


# Planted-mistake switches of the fp8 dequantisation (tests of its pins only).
Q8_FAULT_KSCALE_QHEAD = 101  # K's factor taken at the query head's index
Q8_FAULT_NO_VSCALE = 102     # V's factor left out
Q8_FAULT_DIVIDE = 103        # the factors divide instead of multiply


def e4m3_value(code: int) -> float:
    """The value of one fp8 e4m3 (OCP "e4m3fn") code, as the oracle widens it."""
    return float(_load().oracle_e4m3_value(code))


def _bytes8(t) -> np.ndarray:
    """Raw bytes of an fp8 e4m3 torch tensor (or a uint8 numpy array)."""
    if isinstance(t, np.ndarray):
        if t.dtype != np.uint8:
            raise TypeError("numpy fp8 inputs must hold raw uint8 codes")
        return np.ascontiguousarray(t)
    import torch

    if t.dtype != torch.float8_e4m3fn:
        raise TypeError(f"fp8 oracle inputs must be float8_e4m3fn, got {t.dtype}")
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def _factors(f, n: int):
    if f is None:
        return None
    a = np.ascontiguousarray(np.asarray(f.detach().cpu().numpy() if hasattr(f, "detach") else f, dtype=np.float32))
    if a.size != n:
        raise ValueError(f"descale factors must hold {n} values")
    return a.reshape(-1)


def attention_rows_fp8(q, k, v, rows: Sequence[int], q_descale=None, k_descale=None, v_descale=None, mask=None,
                       scale: Optional[float] = None, is_causal: bool = False, want_probs: bool = False,
                       threads: int = 0, fault: int = FAULT_NONE):
    """Selected rows of exact attention over fp8 e4m3 inputs in fp64.

    q [B, Hq, Nq, D], k and v [B, Hkv, Nkv, D] are float8_e4m3fn tensors (or uint8 code arrays);
    q_descale [B, Hq], k_descale and v_descale [B, Hkv] (fp32; None = 1) are per-head factors: the
    tensor taking part in the attention holds descale[b, head] times each element's e4m3 value.
    Everything else is as in ``attention_rows`` (``scale=None`` means 1/sqrt(D)).
    """
    lib = _load()
    B, Hq, Nq, D = (int(x) for x in q.shape)
    Bk, Hkv, Nkv, Dk = (int(x) for x in k.shape)
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("q/k/v shapes are inconsistent")
    qb, kb, vb = _bytes8(q), _bytes8(k), _bytes8(v)
    fq, fk, fv = _factors(q_descale, B * Hq), _factors(k_descale, B * Hkv), _factors(v_descale, B * Hkv)
    if scale is None or (isinstance(scale, float) and math.isnan(scale)):
        scale = 1.0 / math.sqrt(D)
    marr, mkind, ms = _mask_args(mask, B, Hq, Nq, Nkv)
    rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows_arr.size
    if n and (rows_arr.min() < 0 or rows_arr.max() >= B * Hq * Nq):
        raise ValueError("row index out of range")
    O = np.zeros((n, D), dtype=np.float64)
    L = np.zeros((n,), dtype=np.float64)
    P = np.zeros((n, Nkv), dtype=np.float64) if want_probs else None
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = lib.oracle_attn_rows_e4m3(ptr(qb), ptr(kb), ptr(vb), ptr(fq), ptr(fk), ptr(fv), ptr(marr), mkind, ms[0], ms[1],
                                   ms[2], ms[3], B, Hq, Hkv, Nq, Nkv, D, float(scale), int(bool(is_causal)),
                                   ptr(rows_arr), n, ptr(O), ptr(L), ptr(P), int(threads), int(fault))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_rows_e4m3 failed with code {rc}")
    return (O, L, P) if want_probs else (O, L)


def attention(q, k, v, mask=None, scale: Optional[float] = None, is_causal: bool = False, threads: int = 0,
              fault: int = FAULT_NONE):
    """All rows: returns O [B, Hq, Nq, D] and LSE [B, Hq, Nq] as float64 numpy arrays."""
    B, Hq, Nq, D = (int(x) for x in q.shape)
    O, L = attention_rows(q, k, v, np.arange(B * Hq * Nq), mask=mask, scale=scale, is_causal=is_causal,
                          threads=threads, fault=fault)
    return O.reshape(B, Hq, Nq, D), L.reshape(B, Hq, Nq)


# Planted-mistake switches of the packed form (tests of the pins only).
VL_FAULT_NONE = 0
VL_FAULT_SHARED_OFFSETS = 1   # keys cut with the query offsets
VL_FAULT_TOPLEFT_CAUSAL = 2   # each sequence's causal rule aligned at the top-left
VL_FAULT_LSE_TOKEN_MAJOR = 3  # LSE laid out [Tq, Hq] instead of [Hq, Tq]


def attention_varlen(q, k, v, cu_q: Sequence[int], cu_k: Optional[Sequence[int]] = None,
                     scale: Optional[float] = None, is_causal: bool = False, tokens: Optional[Sequence[int]] = None,
                     threads: int = 0, fault: int = VL_FAULT_NONE):
    """Packed variable-length attention in fp64: each sequence is one dense problem.

    q [Tq, Hq, D]; k, v [Tk, Hkv, D] (torch bf16/fp16); cu_q, cu_k: B+1 offsets (cu_k None: cu_q).
    tokens: query token indices to compute (None: all).  Returns O [n, Hq, D] and LSE [Hq, n] as
    float64 arrays, n = Tq or len(tokens).  A sequence with no key gives its rows O = 0, LSE = -inf
    (the rule for rows that see no key).
    """
    cq = [int(x) for x in (cu_q.tolist() if hasattr(cu_q, "tolist") else cu_q)]
    ck = cq if cu_k is None else [int(x) for x in (cu_k.tolist() if hasattr(cu_k, "tolist") else cu_k)]
    Tq, Hq, D = (int(x) for x in q.shape)
    Tk, Hkv, Dk = (int(x) for x in k.shape)
    if tuple(v.shape) != tuple(k.shape) or Dk != D or len(cq) != len(ck) or len(cq) < 2:
        raise ValueError("inconsistent packed shapes or offsets")
    if cq[0] != 0 or ck[0] != 0 or cq[-1] != Tq or ck[-1] != Tk:
        raise ValueError("offsets must start at 0 and end at the token counts")
    if any(b < a for a, b in zip(cq, cq[1:])) or any(b < a for a, b in zip(ck, ck[1:])):
        raise ValueError("offsets must not decrease")
    if fault == VL_FAULT_SHARED_OFFSETS:
        ck = [min(x, Tk) for x in cq]
    want = np.arange(Tq) if tokens is None else np.asarray(tokens, dtype=np.int64)
    O = np.zeros((want.size, Hq, D), dtype=np.float64)
    L = np.full((Hq, want.size), -np.inf, dtype=np.float64)
    seq_of = np.searchsorted(np.asarray(cq[1:]), want, side="right")
    dense_fault = FAULT_TOPLEFT_CAUSAL if fault == VL_FAULT_TOPLEFT_CAUSAL else FAULT_NONE
    for b in range(len(cq) - 1):
        sel = np.nonzero(seq_of == b)[0]
        nq, nk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        if sel.size == 0 or nq == 0 or nk == 0:
            continue  # no key: the rows keep O = 0, LSE = -inf
        r = want[sel] - cq[b]
        qs = q[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0)   # [1, Hq, nq, D]
        ks = k[ck[b]:ck[b + 1]].permute(1, 0, 2).unsqueeze(0)   # [1, Hkv, nk, D]
        vs = v[ck[b]:ck[b + 1]].permute(1, 0, 2).unsqueeze(0)
        rows = (np.arange(Hq)[:, None] * nq + r[None, :]).reshape(-1)
        o, lse = attention_rows(qs, ks, vs, rows, scale=scale, is_causal=is_causal, threads=threads,
                                fault=dense_fault)
        O[sel] = o.reshape(Hq, sel.size, D).transpose(1, 0, 2)
        L[:, sel] = lse.reshape(Hq, sel.size)
    if fault == VL_FAULT_LSE_TOKEN_MAJOR:
        L = np.ascontiguousarray(L.T).reshape(Hq, want.size)
    return O, L


# Planted-mistake switches of the backward (tests of the pins only).
BWD_FAULT_NONE = 0
BWD_FAULT_NO_DELTA = 1        # dS = P * dP, the row term dropped
BWD_FAULT_DK_UNSCALED = 2     # dK without the scale factor
BWD_FAULT_GQA_LAST_HEAD = 3   # a KV head's gradient from the last head of its group only
BWD_FAULT_KEEP_BIT_REVERSED = 4  # dropout keep words decoded with key 32 w + i at bit 31 - i
BWD_FAULT_KEEP_WORD_SHIFTED = 5  # dropout keep words decoded one word late
BWD_FAULT_DMASK_SCALED = 6       # the mask's gradient taken as scale * dS (the scores' gradient)
BWD_FAULT_DMASK_ONE_HEAD = 7     # the mask's gradient from the first head of a broadcast only


def attention_backward(q, k, v, do, mask=None, scale: Optional[float] = None, is_causal: bool = False,
                       fault: int = BWD_FAULT_NONE, keep_bits=None, dropout_p: float = 0.0, want_dmask: bool = False):
    """Gradients of the attention output with respect to Q, K and V in fp64 (the mask is a constant).

    q [B, Hq, Nq, D]; k, v [B, Hkv, Nkv, D]; do (the output's gradient) like q; torch bf16/fp16 or
    float tensors, widened exactly.  With logits s = scale q.k + bias (-inf where excluded),
    P = softmax over the keys and dP = dO V^T per head:

        dV = sum over the group's heads of P^T dO
        dS = P * (dP - rowsum(P * dP))          (the softmax's Jacobian applied to dP)
        dQ = scale dS K,   dK = scale * sum over the group's heads of dS^T Q

    A row with every key excluded contributes nothing.  Returns (dQ, dK, dV) as float64 arrays.

    With dropout (keep_bits [B, Hq, Nq, ceil(Nkv / 32)] uint32 words, ``oracle.philox`` layout, and
    dropout_p), the output is O = (P * M) V with M = keep / (1 - p) a constant; then
    dV = sum of (P * M)^T dO and the softmax's Jacobian is applied to dP = (dO V^T) * M.

    With want_dmask (an additive floating mask), also the gradient with respect to the mask: the
    logits are scale q.k + bias, so it is dS = P * (dP - rowsum(P * dP)) itself, summed over the
    dimensions the mask broadcasts (size 1 in its shape).  Returns (dQ, dK, dV, dMask) then, dMask in
    the mask's own shape.
    """
    import torch

    B, Hq, Nq, D = (int(x) for x in q.shape)
    Hkv, Nkv = int(k.shape[1]), int(k.shape[2])
    G = Hq // Hkv
    if scale is None or (isinstance(scale, float) and math.isnan(scale)):
        scale = 1.0 / math.sqrt(D)
    Q, K, V, dO = (t.detach().cpu().double().numpy() for t in (q, k, v, do))
    bias = np.zeros((B, Hq, Nq, Nkv))
    if mask is not None:
        m = mask.detach().cpu()
        if m.dtype == torch.bool:
            m = torch.where(m, torch.zeros((), dtype=torch.float64), torch.full((), -math.inf, dtype=torch.float64))
        bias = bias + m.double().numpy()  # broadcasts to [B, Hq, Nq, Nkv]
    if is_causal:
        keep = np.arange(Nkv)[None, :] <= np.arange(Nq)[:, None] + (Nkv - Nq)
        bias = np.where(keep, bias, -np.inf)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dS_all = np.zeros((B, Hq, Nq, Nkv)) if want_dmask else None
    Mdrop = None
    if keep_bits is not None:
        from .philox import KEEP_FAULT_BIT_REVERSED, KEEP_FAULT_NONE, KEEP_FAULT_WORD_SHIFTED, keep_matrix

        kf = {BWD_FAULT_KEEP_BIT_REVERSED: KEEP_FAULT_BIT_REVERSED,
              BWD_FAULT_KEEP_WORD_SHIFTED: KEEP_FAULT_WORD_SHIFTED}.get(fault, KEEP_FAULT_NONE)
        Mdrop = keep_matrix(keep_bits, Nkv, fault=kf) / (1.0 - float(np.float32(dropout_p)))  # [B, Hq, Nq, Nkv]
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            if fault == BWD_FAULT_GQA_LAST_HEAD and h % G != G - 1:
                continue
            s = scale * (Q[b, h] @ K[b, hk].T) + bias[b, h]
            mx = s.max(axis=1, keepdims=True)
            live = np.isfinite(mx[:, 0])
            mx[~live] = 0.0
            e = np.exp(s - mx)
            P = e / np.where(live, e.sum(axis=1), 1.0)[:, None]
            P[~live] = 0.0
            Md = 1.0 if Mdrop is None else Mdrop[b, h]
            dP = (dO[b, h] @ V[b, hk].T) * Md
            dS = P * dP if fault == BWD_FAULT_NO_DELTA else P * (dP - (P * dP).sum(axis=1, keepdims=True))
            if want_dmask:
                dS_all[b, h] = scale * dS if fault == BWD_FAULT_DMASK_SCALED else dS
            dQ[b, h] = scale * (dS @ K[b, hk])
            dK[b, hk] += (1.0 if fault == BWD_FAULT_DK_UNSCALED else scale) * (dS.T @ Q[b, h])
            dV[b, hk] += (P * Md).T @ dO[b, h]
    if not want_dmask:
        return dQ, dK, dV
    if mask is None or mask.dtype == torch.bool:
        raise ValueError("the mask's gradient needs an additive floating mask")
    mshape = tuple(mask.shape)
    full = (1,) * (4 - len(mshape)) + mshape
    # sum over the broadcast dimensions (size 1 in the mask's shape)
    axes = tuple(i for i in range(4) if full[i] == 1 and (B, Hq, Nq, Nkv)[i] != 1)
    if fault == BWD_FAULT_DMASK_ONE_HEAD and full[1] == 1 and Hq > 1:
        dS_all = dS_all[:, :1] * 1.0
        axes = tuple(a for a in axes if a != 1)
    dM = dS_all.sum(axis=axes, keepdims=True) if axes else dS_all
    return dQ, dK, dV, dM.reshape(mshape)


# Planted-mistake switches of the dropout form (tests of the pins only).
DROP_FAULT_NONE = 0
DROP_FAULT_SCALE_BY_KEEP = 1   # kept weights scaled by (1 - p) instead of 1 / (1 - p)
DROP_FAULT_BIT_REVERSED = 2    # key i of a word read from bit 31 - i
DROP_FAULT_LSE_DROPPED = 3     # LSE taken over the kept weights only


def attention_dropout_rows(q, k, v, rows: Sequence[int], keep_bits, p: float, mask=None,
                           scale: Optional[float] = None, is_causal: bool = False, fault: int = DROP_FAULT_NONE):
    """Selected rows of attention with SDPA-style dropout on the attention weights, in fp64.

    The weights are the softmax of the logits (as in ``attention_rows``); dropout keeps weight
    (r, k) where the keep bitmask says so and multiplies the kept ones by 1 / (1 - p); the output is
    the dropped-out weights times V.  The LSE is that of the logits, untouched by dropout.
    ``keep_bits`` is [B, Hq, Nq, ceil(Nkv / 32)] uint32: bit i of word w keeps key 32 w + i
    (``oracle.philox`` draws it).  p is taken as its float32 value, the precision of the C ABI.
    Returns (O [n, D] float64, LSE [n] float64).
    """
    B, Hq, Nq, D = (int(x) for x in q.shape)
    Hkv, Nkv = int(k.shape[1]), int(k.shape[2])
    G = Hq // Hkv
    O_plain, L, P = attention_rows(q, k, v, rows, mask=mask, scale=scale, is_causal=is_causal, want_probs=True)
    kb = np.asarray(keep_bits, dtype=np.uint64).reshape(B * Hq * Nq, -1)
    rows_arr = np.asarray(rows, dtype=np.int64)
    key = np.arange(Nkv)
    bit = (31 - key % 32) if fault == DROP_FAULT_BIT_REVERSED else key % 32
    Z = ((kb[rows_arr][:, key // 32] >> bit.astype(np.uint64)) & np.uint64(1)).astype(np.float64)
    p64 = float(np.float32(p))
    factor = (1.0 - p64) if fault == DROP_FAULT_SCALE_BY_KEEP else 1.0 / (1.0 - p64)
    V = v.detach().cpu().double().numpy()
    O = np.zeros((rows_arr.size, D))
    for i, idx in enumerate(rows_arr):
        b, h = int(idx) // (Nq * Hq), (int(idx) // Nq) % Hq
        O[i] = ((P[i] * Z[i]) @ V[b, h // G]) * factor
    if fault == DROP_FAULT_LSE_DROPPED:
        with np.errstate(divide="ignore"):
            L = L + np.log((P * Z).sum(axis=1))
    return O, L
