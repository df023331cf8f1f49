"""Parity of the packed variable-length path (ffpa_fwd_varlen, through the C ABI) with the fp64 oracle.

Small batches compare every row.  Their length mixes put sequence boundaries inside and at the edges
of the kernels' 64-key and 64/128-row tiles, and include empty sequences, sequences without keys,
and causal sequences with fewer keys than queries.  The full-size packed workload runs in the
benchmark's launch configuration and is compared on seeded sampled tokens.
"""
import json
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import compare_varlen, run_gpu_varlen

pytestmark = pytest.mark.gpu


def _packed(lens_q, lens_k, Hq, Hkv, D, dtype=torch.bfloat16, seed=0):
    w = W.VarlenWorkload("t", tuple(lens_q), tuple(lens_k), Hq, Hkv, D, dtype=dtype, seed=seed)
    return W.make_varlen_inputs(w)


def _log(name, m):
    print(f"[varlen] {name}: {json.dumps(m)}", flush=True)


SELF_LENS = (1, 63, 64, 65, 130, 0, 257)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [64, 128, 256, 320, 512, 576, 640, 1024])
def test_varlen_self_every_kernel(D, causal):
    q, k, v, cu_q, cu_k = _packed(SELF_LENS, SELF_LENS, 2, 2, D, seed=D + causal)
    o, l = run_gpu_varlen(q, k, v, cu_q, cu_k, causal=causal)
    _log(f"self D={D} causal={causal}", compare_varlen(o, l, q, k, v, cu_q, cu_k, causal=causal))


CROSS_Q = (100, 5, 64, 0, 300, 1)
CROSS_K = (30, 200, 64, 7, 129, 0)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [128, 512, 1024])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (3, 1)])
def test_varlen_cross_gqa(Hq, Hkv, D, causal):
    """Different query and key lengths per sequence (causal: sequences 0 and 4 have fewer keys than
    queries, so their first rows see none; sequence 5 has no key at all), GQA and MQA heads."""
    q, k, v, cu_q, cu_k = _packed(CROSS_Q, CROSS_K, Hq, Hkv, D, seed=7 * D + Hq + causal)
    o, l = run_gpu_varlen(q, k, v, cu_q, cu_k, causal=causal)
    m = compare_varlen(o, l, q, k, v, cu_q, cu_k, causal=causal)
    assert m["dead_rows"] >= Hq  # the query of sequence 5 sees no key
    _log(f"cross Hq={Hq} Hkv={Hkv} D={D} causal={causal}", m)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.02])
@pytest.mark.parametrize("D", [256, 1024])
def test_varlen_explicit_scales(scale, D):
    """Zero and negative scales take the kernels' explicit-logit variant, a positive one the split one."""
    q, k, v, cu_q, cu_k = _packed((70, 129, 64), (64, 200, 1), 2, 2, D, seed=D + 3)
    for causal in (False, True):
        o, l = run_gpu_varlen(q, k, v, cu_q, cu_k, causal=causal, scale=scale)
        _log(f"scale {scale} D={D} causal={causal}",
             compare_varlen(o, l, q, k, v, cu_q, cu_k, causal=causal, scale=scale))


@pytest.mark.parametrize("D", [64, 512, 1024])
def test_varlen_fp16(D):
    q, k, v, cu_q, cu_k = _packed(SELF_LENS, SELF_LENS, 2, 1, D, dtype=torch.float16, seed=D + 11)
    o, l = run_gpu_varlen(q, k, v, cu_q, cu_k, causal=True)
    _log(f"fp16 D={D}", compare_varlen(o, l, q, k, v, cu_q, cu_k, causal=True))


def test_varlen_larger_max_seqlen_and_bounds():
    """A max_seqlen above every length only adds workgroups that leave at once; nothing outside O and
    LSE is written, every row of O is written, and two launches agree bitwise."""
    import exact_attention_head_amd as ffpa

    dev = torch.device("cuda:0")
    lens_q, lens_k = (33, 0, 190), (40, 5, 150)
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, 4, 2, 512, seed=21)
    qd, kd, vd, cqd, ckd = (t.to(dev) for t in (q, k, v, cu_q, cu_k))
    Tq, Hq, D = q.shape
    n, pad = Tq * Hq * D, 4096
    big = torch.full((n + 2 * pad,), float("nan"), dtype=q.dtype, device=dev)
    lbig = torch.full((Hq * Tq + 2 * pad,), 12345.0, dtype=torch.float32, device=dev)
    o = big[pad:pad + n].view(Tq, Hq, D)
    lse = lbig[pad:pad + Hq * Tq].view(Hq, Tq)
    outs = []
    for _ in range(2):
        st = ffpa.ffpa_fwd_varlen(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), cqd.data_ptr(), ckd.data_ptr(),
                                  o.data_ptr(), lse.data_ptr(), 3, Hq, 2, Tq, k.shape[0], 700, 300, D,
                                  float("nan"), True, ffpa.FFPA_BF16, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(o.float()).all(), "some output element was not written"
    assert torch.isnan(big[:pad].float()).all() and torch.isnan(big[pad + n:].float()).all(), "O guard band written"
    assert (lbig[:pad] == 12345.0).all() and (lbig[pad + Hq * Tq:] == 12345.0).all(), "LSE guard band written"
    _log("max_seqlen 700/300", compare_varlen(o.cpu(), lse.cpu(), q, k, v, cu_q, cu_k, causal=True))


def test_varlen_equal_lengths_match_dense_path():
    """Equal lengths in packed form and in the dense [B, H, N, D] form describe the same problem: both
    paths meet the oracle, and they agree with each other to the same bar."""
    import exact_attention_head_amd as ffpa

    B, H, N, D = 3, 2, 200, 512
    q, k, v = W.random_qkv(B, H, H, N, N, D, seed=31)
    dev = torch.device("cuda:0")
    od, ld = ffpa.attn(q.to(dev), k.to(dev), v.to(dev), is_causal=True, return_lse=True)
    pack = lambda t: t.permute(0, 2, 1, 3).reshape(B * N, H, D).contiguous()
    cu = torch.arange(0, B * N + 1, N, dtype=torch.int32)
    o, l = run_gpu_varlen(pack(q), pack(k), pack(v), cu, cu, causal=True)
    assert (o.float() - pack(od.cpu()).float()).abs().max() <= 2e-2
    assert (l - ld.cpu().permute(1, 0, 2).reshape(H, B * N)).abs().max() <= 1e-3
    _log("packed vs dense", compare_varlen(o, l, pack(q), pack(k), pack(v), cu, cu, causal=True))


def test_varlen_full_size_workload():
    w = W.varlen_causal()
    q, k, v, cu_q, cu_k = W.make_varlen_inputs(w)
    o, l = run_gpu_varlen(q, k, v, cu_q, cu_k, causal=w.causal)
    toks = W.sample_tokens(w.lens_q, seed=w.seed)
    _log(w.name, compare_varlen(o, l, q, k, v, cu_q, cu_k, tokens=toks, causal=w.causal))
