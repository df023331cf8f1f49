"""Pins for the oracle's backward (gradients of O with respect to Q, K and V; the mask is a constant).

Each pin checks the fp64 gradients against something other than the formulas they are computed
from: torch's autograd through CPU scaled_dot_product_attention in float64, central finite
differences of that forward, invariants that hold for any inputs (the key gradients of a head sum
to zero, the value gradients sum to the output gradients, keys no row sees get none), and the GQA
gradient as the sum over a group of the ungrouped gradients.  ``test_planted_backward_mistakes``
switches on planted mistakes and requires each to fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import random_qkv

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _inputs(B, Hq, Hkv, Nq, Nkv, D, seed):
    q, k, v = random_qkv(B, Hq, Hkv, Nq, Nkv, D, seed=seed)
    do = torch.randn(B, Hq, Nq, D, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    return q, k, v, do


def _torch_grads(q, k, v, do, mask=None, scale=None):
    """Autograd through torch's CPU SDPA in float64 (GQA through enable_gqa)."""
    qd, kd, vd = (t.double().requires_grad_(True) for t in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask, scale=scale,
                                                         enable_gqa=q.shape[1] != k.shape[1])
    return [g.numpy() for g in torch.autograd.grad(o, (qd, kd, vd), do.double())]


def _causal_mask(Nq, Nkv):
    return torch.arange(Nkv).view(1, Nkv) <= torch.arange(Nq).view(Nq, 1) + (Nkv - Nq)


def pin_bwd_torch_autograd(fault=0):
    """Against torch autograd: plain, bool and additive masks, tail causal with Nq < Nkv (as an
    explicit bool mask for torch), GQA and MQA, an explicit scale."""
    ok = True
    g = torch.Generator().manual_seed(5)
    cases = [
        (_inputs(1, 2, 2, 5, 7, 8, 10), dict()),
        (_inputs(2, 4, 2, 4, 6, 8, 11), dict(mask=torch.rand(2, 1, 4, 6, generator=g) < 0.7)),
        (_inputs(1, 3, 1, 6, 6, 16, 12), dict(mask=torch.randn(1, 3, 6, 6, generator=g))),
        (_inputs(1, 2, 1, 4, 9, 8, 13), dict(is_causal=True)),
        (_inputs(1, 2, 2, 3, 5, 8, 14), dict(scale=0.3)),
    ]
    for (q, k, v, do), kw in cases:
        mask = kw.get("mask")
        if mask is not None:
            mask = mask.clone()
            mask[..., 0] = True if mask.dtype == torch.bool else mask[..., 0]
        tmask = _causal_mask(q.shape[2], k.shape[2]) if kw.get("is_causal") else mask
        want = _torch_grads(q, k, v, do, mask=tmask, scale=kw.get("scale"))
        got = oracle.attention_backward(q, k, v, do, mask=mask, scale=kw.get("scale"),
                                        is_causal=kw.get("is_causal", False), fault=fault)
        ok &= all(bool(np.abs(a - b).max() <= 1e-12) for a, b in zip(got, want))
    return ok


def pin_bwd_finite_differences(fault=0):
    """Central differences of the float64 SDPA forward, along random directions in Q, K and V:
    <dL/dX, E> = (L(X + hE) - L(X - hE)) / 2h with L = <O, dO>."""
    q, k, v, do = _inputs(1, 2, 1, 4, 5, 8, 20)
    grads = oracle.attention_backward(q, k, v, do, is_causal=True, fault=fault)
    base = [t.double() for t in (q, k, v)]
    mask = _causal_mask(4, 5)

    def loss(ts):
        o = torch.nn.functional.scaled_dot_product_attention(*ts, attn_mask=mask, enable_gqa=True)
        return float((o * do.double()).sum())

    ok = True
    gen = torch.Generator().manual_seed(21)
    h = 1e-5
    for i in range(3):
        e = torch.randn(base[i].shape, generator=gen, dtype=torch.float64)
        plus = [t + h * e if j == i else t for j, t in enumerate(base)]
        minus = [t - h * e if j == i else t for j, t in enumerate(base)]
        fd = (loss(plus) - loss(minus)) / (2 * h)
        an = float((torch.from_numpy(grads[i]) * e).sum())
        ok &= abs(fd - an) <= 1e-7 * max(1.0, abs(fd))
    return ok


def pin_bwd_invariants(fault=0):
    """Softmax gradients sum to zero over a row, so each KV head's key gradients sum to zero; the
    probabilities sum to one, so its value gradients sum to the output gradients of its rows; a key
    that no row sees gets no gradient."""
    q, k, v, do = _inputs(2, 4, 2, 6, 9, 8, 30)
    mask = torch.rand(2, 1, 6, 9, generator=torch.Generator().manual_seed(31)) < 0.6
    mask[..., 0] = True
    mask[..., 4] = False  # key 4 is seen by no row
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, mask=mask, fault=fault)
    dOd = do.double().numpy()
    ok = bool(np.abs(dK.sum(axis=2)).max() <= 1e-12)
    want = dOd.reshape(2, 2, 2, 6, 8).sum(axis=(2, 3))  # group heads and rows of each KV head
    ok &= bool(np.abs(dV.sum(axis=2) - want).max() <= 1e-12)
    ok &= bool(np.all(dK[:, :, 4] == 0)) and bool(np.all(dV[:, :, 4] == 0))
    return ok


def pin_bwd_gqa_is_repeat(fault=0):
    """GQA gradients equal the ungrouped gradients with K/V repeated per group, summed over each
    group for K and V."""
    q, k, v, do = _inputs(1, 6, 2, 5, 7, 8, 40)
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, is_causal=True, fault=fault)
    kr, vr = k.repeat_interleave(3, dim=1), v.repeat_interleave(3, dim=1)
    rQ, rK, rV = oracle.attention_backward(q, kr, vr, do, is_causal=True)
    ok = bool(np.abs(dQ - rQ).max() <= 1e-13)
    ok &= bool(np.abs(dK - rK.reshape(1, 2, 3, 7, 8).sum(axis=2)).max() <= 1e-13)
    ok &= bool(np.abs(dV - rV.reshape(1, 2, 3, 7, 8).sum(axis=2)).max() <= 1e-13)
    return ok


BWD_PINS = [pin_bwd_torch_autograd, pin_bwd_finite_differences, pin_bwd_invariants, pin_bwd_gqa_is_repeat]


@pytest.mark.parametrize("pin", BWD_PINS, ids=[p.__name__ for p in BWD_PINS])
def test_backward_pin_holds(pin):
    assert pin(0), pin.__doc__


BWD_FAULTS = {
    oracle.BWD_FAULT_NO_DELTA: "row term of the softmax Jacobian dropped",
    oracle.BWD_FAULT_DK_UNSCALED: "dK without the scale",
    oracle.BWD_FAULT_GQA_LAST_HEAD: "KV gradients from one head of the group",
}


@pytest.mark.parametrize("fault", sorted(BWD_FAULTS), ids=[BWD_FAULTS[f] for f in sorted(BWD_FAULTS)])
def test_planted_backward_mistakes(fault):
    failing = [p.__name__ for p in BWD_PINS if not p(fault)]
    assert failing, f"no pin catches the planted mistake: {BWD_FAULTS[fault]}"


def test_fully_masked_rows_give_no_gradient():
    q, k, v, do = _inputs(1, 1, 1, 3, 4, 8, 50)
    mask = torch.ones(1, 1, 3, 4, dtype=torch.bool)
    mask[0, 0, 1] = False
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, mask=mask)
    assert np.all(dQ[0, 0, 1] == 0) and np.isfinite(dK).all() and np.isfinite(dV).all()
    # the same as dropping that row's output gradient
    do2 = do.clone()
    do2[0, 0, 1] = 0
    _, dK2, dV2 = oracle.attention_backward(q, k, v, do2, mask=mask)
    assert np.array_equal(dK, dK2) and np.array_equal(dV, dV2)


def _torch_grads_with_mask(q, k, v, do, mask, scale, is_causal=False):
    """float64 autograd through softmax(scale q.k + mask) V with the mask a leaf: its gradient."""
    G = q.shape[1] // k.shape[1]
    qd, kd, vd = (t.double() for t in (q, k, v))
    md = mask.double().requires_grad_(True)
    kr, vr = kd.repeat_interleave(G, dim=1), vd.repeat_interleave(G, dim=1)
    s = (qd @ kr.transpose(-1, -2)) * scale + md
    if is_causal:
        Nq, Nkv = q.shape[2], k.shape[2]
        vis = torch.arange(Nkv).view(1, Nkv) <= torch.arange(Nq).view(Nq, 1) + (Nkv - Nq)
        s = s.masked_fill(~vis, -math.inf)
    o = torch.softmax(s, dim=-1) @ vr
    (g,) = torch.autograd.grad(o, (md,), do.double())
    return g.numpy()


def pin_dmask(fault=oracle.BWD_FAULT_NONE):
    ok = True
    g = torch.Generator().manual_seed(71)
    for (B, Hq, Hkv, Nq, Nkv, D, causal, shape) in [(2, 4, 2, 5, 9, 8, False, (2, 1, 5, 9)),
                                                     (1, 3, 3, 6, 6, 4, True, (1, 3, 6, 6)),
                                                     (2, 2, 1, 4, 7, 8, False, (4, 7)),
                                                     (2, 2, 2, 3, 5, 8, False, (1, 2, 1, 5))]:
        q, k, v = random_qkv(B, Hq, Hkv, Nq, Nkv, D, seed=B + Nq)
        do = torch.randn(B, Hq, Nq, D, generator=g).to(torch.bfloat16)
        mask = torch.randn(*shape, generator=g)
        scale = 1.0 / math.sqrt(D)
        want = _torch_grads_with_mask(q, k, v, do, mask, scale, is_causal=causal)
        *_, dm = oracle.attention_backward(q, k, v, do, mask=mask, is_causal=causal, fault=fault, want_dmask=True)
        ok &= dm.shape == tuple(shape)
        ok &= bool(np.all(np.abs(dm - want) <= 1e-10 * max(1.0, np.abs(want).max())))
    return ok


def test_mask_gradient_against_autograd():
    assert pin_dmask()


def test_mask_gradient_rows_sum_to_zero():
    """Softmax is invariant to adding a constant to a row of logits, so each row of the logits'
    gradient, and of a full mask's gradient, sums to zero."""
    q, k, v = random_qkv(1, 2, 2, 4, 9, 8, seed=3)
    do = torch.randn(1, 2, 4, 8, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    mask = torch.randn(1, 2, 4, 9, generator=torch.Generator().manual_seed(4))
    *_, dm = oracle.attention_backward(q, k, v, do, mask=mask, want_dmask=True)
    assert np.all(np.abs(dm.sum(axis=-1)) <= 1e-12)


def test_mask_gradient_planted_mistakes_are_caught():
    for fault in (oracle.BWD_FAULT_DMASK_SCALED, oracle.BWD_FAULT_DMASK_ONE_HEAD, oracle.BWD_FAULT_NO_DELTA):
        assert not pin_dmask(fault), fault
