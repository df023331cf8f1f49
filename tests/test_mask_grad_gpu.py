"""Gradient of an additive attention mask (ffpa_bwd_mask_grad, through the C ABI) against the fp64
oracle's, on the GPU.

The logits are scale q.k + mask, so the mask's gradient is the logits' gradient P (dP - Delta) summed
over the dimensions along which the mask broadcasts.  The kernels keep that gradient in fp32 (it is
not rounded to 16 bits as dS is for the products); its error comes from Delta, formed from the
16-bit O of the forward (2^-9 relative in bf16), and from the fp32 products.  The bar is the one of
the other gradients: rel-L2 <= 1e-2 and a largest element error <= 2e-2 of the largest reference
magnitude.  dQ, dK and dV of the same call are held to that bar too.
"""
import json

import numpy as np
import pytest
import torch

import exact_attention_head_amd as ffpa
import oracle
import workloads as W
from oracle.philox import dropout_keep_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
REL_L2 = 1e-2
MAX_REL = 2e-2


def _log(name, m):
    print(f"[mask grad] {name}: {json.dumps(m)}", flush=True)


def _err(g, w):
    g = g.double().numpy() if isinstance(g, torch.Tensor) else g
    assert g.shape == w.shape, (g.shape, w.shape)
    assert np.isfinite(g).all()
    rel = float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30))
    mx = float(np.abs(g - w).max() / max(np.abs(w).max(), 1e-30))
    return dict(rel_l2=rel, max_rel=mx)


def _run(B, Hq, Hkv, Nq, Nkv, D, shape, *, dtype=torch.bfloat16, mdtype=torch.float32, causal=False,
         p=0.0, neg_inf=0.0, seed=0, name="", exact_zero=False):
    print(f"[mask grad] case {name}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} mask={shape} "
          f"dtype={dtype} mdtype={mdtype} causal={causal} p={p}", flush=True)
    q, k, v = W.random_qkv(B, Hq, Hkv, Nq, Nkv, D, dtype=dtype, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(B, Hq, Nq, D, generator=g).to(dtype)
    mask = torch.randn(*shape, generator=g)
    if neg_inf:
        mask[torch.rand(*shape, generator=g) < neg_inf] = float("-inf")
        mask[..., 0] = 0.0
    mask = mask.to(mdtype)
    words = dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=seed + 2) if p else None
    keep = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(DEV) if p else None
    qd, kd, vd, dod, md = (t.to(DEV) for t in (q, k, v, do, mask))
    gqa = Hq != Hkv
    if p:
        o, lse = ffpa.attn(qd, kd, vd, attn_mask=md, is_causal=causal, enable_gqa=gqa, return_lse=True,
                           dropout_p=p, dropout_keep=keep)
    else:
        o, lse = ffpa.attn(qd, kd, vd, attn_mask=md, is_causal=causal, enable_gqa=gqa, return_lse=True)
    got = ffpa.attn_backward(qd, kd, vd, o, dod, lse, attn_mask=md, is_causal=causal, dropout_p=p,
                             dropout_keep=keep, mask_grad=True)
    again = ffpa.attn_backward(qd, kd, vd, o, dod, lse, attn_mask=md, is_causal=causal, dropout_p=p,
                               dropout_keep=keep, mask_grad=True)[3]
    torch.cuda.synchronize()
    full = len(shape) == 4 and tuple(shape) == (B, Hq, Nq, Nkv)
    if full:
        # one writer per element: identical bits on every call
        assert torch.equal(got[3], again), "the mask gradient is not reproducible bit for bit"
    else:
        # broadcast dimensions are summed with atomic adds, in an order that may vary: up to B Hq Nq
        # fp32 terms per element, whose rounding differences stay far below the parity bar below
        assert torch.allclose(got[3], again, rtol=0, atol=1e-3 * float(again.abs().max()) + 1e-30)
    assert got[3].dtype == torch.float32 and tuple(got[3].shape) == tuple(shape)
    want = oracle.attention_backward(q, k, v, do, mask=mask, is_causal=causal, keep_bits=words, dropout_p=p,
                                     want_dmask=True)
    names = ("dq", "dk", "dv") if exact_zero else ("dq", "dk", "dv", "dmask")
    m = {nm: _err(gg.cpu(), w) for nm, gg, w in zip(names, got, want)}
    _log(name, m)
    for nm, e in m.items():
        assert e["rel_l2"] <= REL_L2 and e["max_rel"] <= MAX_REL, (nm, m)
    return got, want


SHAPES = {
    "full": lambda B, H, Nq, Nkv: (B, H, Nq, Nkv),
    "batch-bcast": lambda B, H, Nq, Nkv: (1, H, Nq, Nkv),
    "head-bcast": lambda B, H, Nq, Nkv: (B, 1, Nq, Nkv),
    "2d": lambda B, H, Nq, Nkv: (Nq, Nkv),
    "key-padding": lambda B, H, Nq, Nkv: (B, 1, 1, Nkv),
    "row": lambda B, H, Nq, Nkv: (Nkv,),
    "head-row": lambda B, H, Nq, Nkv: (1, H, 1, Nkv),
}


@pytest.mark.parametrize("kind", list(SHAPES))
@pytest.mark.parametrize("gqa", [False, True], ids=["mha", "gqa"])
def test_mask_grad_shapes(kind, gqa):
    B, Hq, Nq, Nkv, D = 2, 4, 70, 150, 128
    _run(B, Hq, 2 if gqa else Hq, Nq, Nkv, D, SHAPES[kind](B, Hq, Nq, Nkv), seed=len(kind) + gqa,
         name=f"{kind} {'gqa' if gqa else 'mha'}")


@pytest.mark.parametrize("D", [64, 256, 512, 1024])
def test_mask_grad_head_dims_causal(D):
    B, Hq, Nq, Nkv = 1, 2, 96, 130
    _run(B, Hq, 1, Nq, Nkv, D, (B, Hq, Nq, Nkv), causal=True, neg_inf=0.1, seed=D, name=f"causal D={D}")


@pytest.mark.parametrize("dtype,mdtype", [(torch.float16, torch.float16), (torch.bfloat16, torch.bfloat16),
                                          (torch.float16, torch.float32)])
def test_mask_grad_dtypes(dtype, mdtype):
    _run(1, 3, 3, 64, 100, 256, (1, 3, 64, 100), dtype=dtype, mdtype=mdtype, neg_inf=0.05, seed=5,
         name=f"{dtype} mask {mdtype}")


@pytest.mark.parametrize("kind", ["full", "head-bcast"])
def test_mask_grad_dropout(kind):
    B, Hq, Nq, Nkv = 2, 2, 64, 100
    _run(B, Hq, Hq, Nq, Nkv, 256, SHAPES[kind](B, Hq, Nq, Nkv), p=0.3, seed=13, name=f"dropout {kind}")


def test_mask_grad_key_broadcast_is_zero():
    """A mask constant along the keys shifts whole rows of logits: its gradient is exactly zero."""
    got, want = _run(2, 2, 2, 40, 60, 128, (2, 2, 40, 1), seed=17, name="key-broadcast", exact_zero=True)
    assert torch.count_nonzero(got[3]) == 0 and np.abs(want[3]).max() < 1e-12


def test_mask_grad_tiny_and_single_key():
    _run(1, 1, 1, 1, 1, 64, (1, 1, 1, 1), seed=19, name="1x1")
    _run(1, 2, 1, 3, 5, 64, (3, 5), causal=True, seed=20, name="causal 3x5")


@pytest.mark.parametrize("kind", ["batch-bcast", "key-padding"])
def test_mask_grad_large(kind):
    """Nq = Nkv = 4096 over 32 heads: every workgroup of many heads adds into the broadcast mask's
    gradient."""
    B, Hq, N, D = 2, 16, 4096, 64
    _run(B, Hq, Hq, N, N, D, SHAPES[kind](B, Hq, N, N), seed=23, name=f"large {kind}")


def test_autograd_mask_gradient():
    """attn_with_grad with a mask that requires grad: mask.grad is attn_backward's dMask in the mask's
    dtype, and query/key/value gradients are unchanged."""
    B, Hq, Nq, Nkv, D = 1, 4, 50, 90, 256
    q, k, v = W.random_qkv(B, Hq, 2, Nq, Nkv, D, seed=29)
    do = torch.randn(B, Hq, Nq, D, generator=torch.Generator().manual_seed(30)).to(torch.bfloat16)
    for mdtype in (torch.float32, torch.bfloat16):
        mask = torch.randn(1, Hq, Nq, Nkv, generator=torch.Generator().manual_seed(31)).to(mdtype).to(DEV)
        mask.requires_grad_(True)
        qd, kd, vd = (t.to(DEV).requires_grad_(True) for t in (q, k, v))
        o = ffpa.attn_with_grad(qd, kd, vd, attn_mask=mask, enable_gqa=True)
        o.backward(do.to(DEV))
        dq, dk, dv, dm = ffpa.attn_backward(qd.detach(), kd.detach(), vd.detach(), o.detach(), do.to(DEV),
                                            ffpa.attn(qd.detach(), kd.detach(), vd.detach(), attn_mask=mask.detach(),
                                                      enable_gqa=True, return_lse=True)[1],
                                            attn_mask=mask.detach(), mask_grad=True)
        torch.cuda.synchronize()
        assert mask.grad is not None and mask.grad.dtype == mdtype
        assert torch.equal(mask.grad, dm.to(mdtype))
        assert torch.equal(qd.grad, dq) and torch.equal(kd.grad, dk) and torch.equal(vd.grad, dv)
        want = oracle.attention_backward(q, k, v, do, mask=mask.detach().cpu(), want_dmask=True)[3]
        e = _err(mask.grad.float().cpu(), want)
        _log(f"autograd {mdtype}", e)
        assert e["rel_l2"] <= REL_L2 and e["max_rel"] <= MAX_REL


def test_mask_grad_argument_errors():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 1, 8, device=DEV)
    with pytest.raises(ValueError):
        ffpa.attn_backward(q, q, q, q, q, lse, attn_mask=torch.ones(8, 8, dtype=torch.bool, device=DEV),
                           mask_grad=True)
    with pytest.raises(ValueError):
        ffpa.attn_backward(q, q, q, q, q, lse, mask_grad=True)
