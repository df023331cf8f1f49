"""Parity of the fused backward (ffpa_bwd, through the C ABI) with the fp64 oracle's gradients, on the GPU.

The forward runs first (its O and LSE feed the backward, as in training); the gradients are compared
element by element with the oracle's exact gradients of the same inputs.  The bar, derived from the
arithmetic: P and dS are rounded once to 16 bits for the products (2^-9 relative in bf16) and the
outputs once more, so each gradient is expected near 3-4e-3 relative L2; the test allows rel-L2
<= 1e-2 and a largest element error <= 2e-2 of the largest reference magnitude.
"""
import json

import numpy as np
import pytest
import torch

import exact_attention_head_amd as ffpa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
REL_L2 = 1e-2
MAX_REL = 2e-2


def _grads_gpu(q, k, v, do, mask=None, is_causal=False, scale=None):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    md = mask.to(DEV) if mask is not None else None
    o, lse = ffpa.attn(qd, kd, vd, attn_mask=md, is_causal=is_causal, scale=scale,
                       enable_gqa=q.shape[1] != k.shape[1], return_lse=True)
    dq, dk, dv = ffpa.attn_backward(qd, kd, vd, o, dod, lse, attn_mask=md, is_causal=is_causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _compare(got, q, k, v, do, **kw):
    want = oracle.attention_backward(q, k, v, do, **kw)
    m = {}
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        g = g.double().numpy()
        assert np.isfinite(g).all(), f"non-finite values in {name}"
        rel = float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30))
        mx = float(np.abs(g - w).max() / max(np.abs(w).max(), 1e-30))
        m[name] = dict(rel_l2=round(rel, 6), max_rel=round(mx, 6))
        assert rel <= REL_L2 and mx <= MAX_REL, (name, m)
    return m


def _case(B, Hq, Hkv, Nq, Nkv, D, dtype=torch.bfloat16, seed=0):
    q, k, v = W.random_qkv(B, Hq, Hkv, Nq, Nkv, D, dtype=dtype, seed=seed)
    do = torch.randn(B, Hq, Nq, D, generator=torch.Generator().manual_seed(seed + 1)).to(dtype)
    return q, k, v, do


def _log(name, m):
    print(f"[bwd] {name}: {json.dumps(m)}", flush=True)


# every kernel head dim of the fused backward, and the head dims that run a larger one with the
# columns past D skipped (576, 704, 832, 960)
@pytest.mark.parametrize("D", [64, 128, 192, 256, 320, 384, 448, 512, 576, 640, 704, 768, 832, 896, 960, 1024])
def test_backward_head_dims(D):
    q, k, v, do = _case(1, 2, 2, 130, 200, D, seed=D)
    _log(f"D={D}", _compare(_grads_gpu(q, k, v, do), q, k, v, do))


# head dims that are multiples of 8 but not of 64: the next kernel head dim, columns past D skipped
@pytest.mark.parametrize("D", [8, 40, 72, 80, 96, 120, 136, 200, 264, 328, 456, 520, 600, 712, 776, 840, 1000, 1016])
def test_backward_head_dims_by_8(D):
    q, k, v, do = _case(1, 2, 1, 97, 150, D, seed=D + 7)
    _log(f"D={D}", _compare(_grads_gpu(q, k, v, do), q, k, v, do))


@pytest.mark.parametrize("D", [24, 248, 968])
def test_backward_head_dims_by_8_causal_mask(D):
    q, k, v, do = _case(2, 4, 2, 70, 133, D, seed=D + 9)
    mask = torch.randn(2, 1, 70, 133, generator=torch.Generator().manual_seed(D))
    _log(f"D={D} causal+mask", _compare(_grads_gpu(q, k, v, do, mask=mask, is_causal=True), q, k, v, do, mask=mask,
                                        is_causal=True))


@pytest.mark.parametrize("D", [128, 576, 1024])
def test_backward_fp16_head_dims(D):
    q, k, v, do = _case(2, 2, 1, 97, 161, D, dtype=torch.float16, seed=D + 1)
    _log(f"fp16 D={D}", _compare(_grads_gpu(q, k, v, do, is_causal=True), q, k, v, do, is_causal=True))


def test_backward_tiny_and_single_rows():
    for (Nq, Nkv) in [(1, 40), (2, 3), (33, 33), (31, 95)]:
        q, k, v, do = _case(1, 3, 1, Nq, Nkv, 128, seed=Nq + Nkv)
        _log(f"Nq={Nq} Nkv={Nkv}", _compare(_grads_gpu(q, k, v, do), q, k, v, do))


def test_backward_single_key():
    """One key: the softmax is constant, so dQ and dK are exactly zero (the kernels leave rounding
    noise of Delta's 16-bit O) and dV = sum over the group of dO."""
    q, k, v, do = _case(1, 3, 1, 5, 1, 128, seed=3)
    dq, dk, dv = _grads_gpu(q, k, v, do)
    want = oracle.attention_backward(q, k, v, do)
    assert np.abs(want[0]).max() == 0 and np.abs(want[1]).max() == 0
    scale_v = float(np.abs(want[2]).max())
    assert float(dq.abs().max()) <= 1e-3 * scale_v and float(dk.abs().max()) <= 1e-3 * scale_v
    g = dv.double().numpy()
    assert np.linalg.norm(g - want[2]) <= REL_L2 * np.linalg.norm(want[2])


def test_backward_full_size_self_attention():
    """The D=512 self-attention workload (B=1, H=8, N=4096) that the bench times, all gradients."""
    w = W.large_d_self()
    q, k, v = W.random_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, seed=101)
    do = torch.randn(w.B, w.Hq, w.Nq, w.D, generator=torch.Generator().manual_seed(102)).to(torch.bfloat16)
    _log("B1 H8 N4096 D512", _compare(_grads_gpu(q, k, v, do), q, k, v, do))


@pytest.mark.parametrize("Nq,Nkv", [(64, 64), (100, 333), (257, 260)])
@pytest.mark.parametrize("D", [128, 512])
def test_backward_causal_gqa(Nq, Nkv, D):
    q, k, v, do = _case(2, 4, 2, Nq, Nkv, D, seed=Nq + D)
    _log(f"causal GQA Nq={Nq} Nkv={Nkv} D={D}",
         _compare(_grads_gpu(q, k, v, do, is_causal=True), q, k, v, do, is_causal=True))


@pytest.mark.parametrize("kind", ["bool", "f32"])
def test_backward_masks(kind):
    q, k, v, do = _case(2, 3, 1, 90, 150, 256, seed=7)
    g = torch.Generator().manual_seed(8)
    bias = torch.randn(2, 1, 90, 150, generator=g)
    bias[torch.rand(2, 1, 90, 150, generator=g) < 0.1] = float("-inf")
    bias[..., 0] = 0.0
    mask = bias > -0.5 if kind == "bool" else bias
    if kind == "bool":
        mask[..., 0] = True
    _log(f"mask {kind}", _compare(_grads_gpu(q, k, v, do, mask=mask), q, k, v, do, mask=mask))


def test_backward_fp16_and_scale():
    q, k, v, do = _case(1, 2, 1, 70, 90, 512, dtype=torch.float16, seed=9)
    _log("fp16 scale 0.05", _compare(_grads_gpu(q, k, v, do, scale=0.05), q, k, v, do, scale=0.05))


def test_autograd_function_matches():
    """attn_with_grad + torch autograd gives the gradients of attn_backward."""
    q, k, v, do = _case(1, 4, 2, 100, 120, 512, seed=11)
    qd, kd, vd = (t.to(DEV).requires_grad_(True) for t in (q, k, v))
    o = ffpa.attn_with_grad(qd, kd, vd, is_causal=True, enable_gqa=True)
    o.backward(do.to(DEV))
    got = (qd.grad.cpu(), kd.grad.cpu(), vd.grad.cpu())
    want = _grads_gpu(q, k, v, do, is_causal=True)
    for g, w in zip(got, want):
        assert torch.equal(g, w)
    _log("autograd", _compare(got, q, k, v, do, is_causal=True))


def test_attn_records_autograd_like_sdpa():
    """attn on inputs that require grad records the call: the same gradients as attn_with_grad, bit for
    bit, with the LSE returned beside O and no gradient of its own; under no_grad nothing is recorded."""
    q, k, v, do = _case(1, 4, 2, 100, 120, 512, seed=12)
    qd, kd, vd = (t.to(DEV).requires_grad_(True) for t in (q, k, v))
    o, lse = ffpa.attn(qd, kd, vd, is_causal=True, enable_gqa=True, return_lse=True)
    assert o.grad_fn is not None and not lse.requires_grad
    o.backward(do.to(DEV))
    got = (qd.grad.cpu(), kd.grad.cpu(), vd.grad.cpu())
    qw, kw, vw = (t.to(DEV).requires_grad_(True) for t in (q, k, v))
    ffpa.attn_with_grad(qw, kw, vw, is_causal=True, enable_gqa=True).backward(do.to(DEV))
    for g, w in zip(got, (qw.grad.cpu(), kw.grad.cpu(), vw.grad.cpu())):
        assert torch.equal(g, w)
    with torch.no_grad():
        assert ffpa.attn(qd, kd, vd, is_causal=True, enable_gqa=True).grad_fn is None
    _log("attn autograd", _compare(got, q, k, v, do, is_causal=True))
