"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI, compare with the oracle."""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import exact_attention_head_amd as ffpa  # noqa: E402
import oracle  # noqa: E402

# Tolerances on O (bf16/fp16 output, fp32 accumulation) against the unrounded fp64 oracle, and on the
# fp32 LSE, as the benchmark spec of this path fixes them.
O_MAX_ABS = 2e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def gpu_available() -> bool:
    return torch.cuda.is_available()


def run_gpu(q, k, v, mask=None, is_causal=False, scale=None, enable_gqa=None):
    """Host tensors in, host tensors out (O in the input dtype, LSE fp32); one kernel launch."""
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    md = mask.to(dev) if mask is not None else None
    if enable_gqa is None:
        enable_gqa = q.shape[1] != k.shape[1]
    o, lse = ffpa.attn(qd, kd, vd, attn_mask=md, is_causal=is_causal, scale=scale, enable_gqa=enable_gqa,
                       return_lse=True)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def compare(o_gpu, lse_gpu, q, k, v, rows=None, mask=None, is_causal=False, scale=None):
    """Element-by-element comparison of the GPU rows with the oracle; returns a metrics dict and asserts
    the tolerances.  rows: flat row indices (None = all)."""
    B, Hq, Nq, D = q.shape
    og = o_gpu.float().reshape(-1, D)
    lg = lse_gpu.reshape(-1)
    # the whole GPU output must be free of NaN and of infinities (LSE may be -inf only where allowed)
    assert torch.isfinite(og).all(), "non-finite values in O"
    assert not torch.isnan(lg).any(), "NaN in LSE"
    assert not (lg == math.inf).any(), "+inf in LSE"
    if rows is None:
        rows = np.arange(B * Hq * Nq)
    rows = np.asarray(rows, dtype=np.int64)
    o_ref, l_ref = oracle.attention_rows(q, k, v, rows, mask=mask, scale=scale, is_causal=is_causal)
    o_g = og.numpy().astype(np.float64)[rows]
    l_g = lg.numpy().astype(np.float64)[rows]
    err = np.abs(o_g - o_ref)
    max_abs = float(err.max()) if err.size else 0.0
    ref_norm = float(np.linalg.norm(o_ref))
    rel_l2 = float(np.linalg.norm(o_g - o_ref) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(o_g))
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_g), fin), "LSE finiteness differs from the oracle"
    assert np.all(l_g[~fin] == l_ref[~fin]), "rows with no visible key must have LSE = -inf"
    lse_err = float(np.abs(l_g[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    m = dict(rows=int(rows.size), o_max_abs=max_abs, o_rel_l2=rel_l2, lse_max_abs=lse_err)
    assert max_abs <= O_MAX_ABS, m
    assert rel_l2 <= O_REL_L2, m
    assert lse_err <= LSE_MAX_ABS, m
    return m


def run_gpu_varlen(q, k, v, cu_q, cu_k, max_q=None, max_k=None, causal=False, scale=None):
    """Packed host tensors in, host tensors out: O [Tq, Hq, D] and LSE [Hq, Tq]; one kernel launch."""
    dev = torch.device("cuda:0")
    lq = (cu_q[1:] - cu_q[:-1]).tolist()
    lk = (cu_k[1:] - cu_k[:-1]).tolist()
    max_q = max(lq) if max_q is None else max_q
    max_k = max(lk) if max_k is None else max_k
    o, lse = ffpa.attn_varlen(q.to(dev), k.to(dev), v.to(dev), cu_q.to(dev), cu_k.to(dev), max_q, max_k,
                              softmax_scale=scale, causal=causal, enable_gqa=q.shape[1] != k.shape[1],
                              return_lse=True)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def compare_varlen(o_gpu, lse_gpu, q, k, v, cu_q, cu_k, tokens=None, causal=False, scale=None):
    """Element-by-element comparison of packed GPU rows with the oracle, to the tolerances above; rows
    that see no key must be O = 0 and LSE = -inf exactly."""
    Tq, Hq, D = q.shape
    og = o_gpu.float()
    lg = lse_gpu
    assert torch.isfinite(og).all(), "non-finite values in O"
    assert not torch.isnan(lg).any() and not (lg == math.inf).any(), "NaN or +inf in LSE"
    toks = np.arange(Tq) if tokens is None else np.asarray(tokens, dtype=np.int64)
    o_ref, l_ref = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale=scale, is_causal=causal, tokens=toks)
    o_g = og.numpy().astype(np.float64)[toks]
    l_g = lg.numpy().astype(np.float64)[:, toks]
    dead = ~np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_g), ~dead), "LSE finiteness differs from the oracle"
    assert np.all(l_g[dead] == -math.inf)
    assert np.all(o_g.transpose(1, 0, 2)[dead] == 0), "rows with no visible key must be 0"
    err = np.abs(o_g - o_ref)
    max_abs = float(err.max()) if err.size else 0.0
    ref_norm = float(np.linalg.norm(o_ref))
    rel_l2 = float(np.linalg.norm(o_g - o_ref) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(o_g))
    lse_err = float(np.abs(l_g[~dead] - l_ref[~dead]).max()) if (~dead).any() else 0.0
    m = dict(tokens=int(toks.size), o_max_abs=max_abs, o_rel_l2=rel_l2, lse_max_abs=lse_err,
             dead_rows=int(dead.sum()))
    assert max_abs <= O_MAX_ABS, m
    assert rel_l2 <= O_REL_L2, m
    assert lse_err <= LSE_MAX_ABS, m
    return m
