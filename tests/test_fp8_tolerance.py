"""The fp8 forward's tolerance against a numpy model of its one extra rounding (CPU only).

The kernels compute the logits from e4m3 products in fp32 and round each probability to e4m3 (RNE)
for the P V product, with the reference maximum anywhere up to 8 (log2 units) below the row maximum.
The model does exactly that rounding in fp64 on seeded workloads of the GPU tests' kind and checks that
the errors it produces sit well inside the bar the GPU tests use (rel-L2 <= 0.05, max-abs <= 2^-4
max|V'|): the bar is derived from this rounding, not fitted to the kernels' output.
"""
import math

import numpy as np
import pytest
import torch

F8 = torch.float8_e4m3fn


@pytest.mark.parametrize("N,D,causal,mask", [(256, 128, False, False), (1024, 512, False, False),
                                             (512, 256, False, True), (512, 384, True, False)])
def test_model_of_the_probability_rounding(N, D, causal, mask):
    g = torch.Generator().manual_seed(N + D)
    q, k, v = ((torch.randn(1, 2, N, D, generator=g) * 2).to(F8) for _ in range(3))
    f = [torch.rand(1, 2, generator=g) * 0.4 + 0.2 for _ in range(3)]
    Q, K, V = (x.double() * s.double()[:, :, None, None] for x, s in zip((q, k, v), f))
    s = Q @ K.transpose(-1, -2) / math.sqrt(D)
    if mask:
        s = s + torch.randn(1, 1, N, N, generator=g).double()
    if causal:
        s = s.masked_fill(~(torch.arange(N)[None, :] <= torch.arange(N)[:, None]), -math.inf)
    p = torch.exp(s - s.max(-1, keepdim=True).values)
    l = p.sum(-1, keepdim=True)
    O = (p @ V) / l
    for shift in (0.0, 7.99):
        pt = (p * 2 ** shift).float().to(F8).double() / 2 ** shift
        Om = ((pt @ V) / l).to(torch.bfloat16).double()
        err = Om - O
        rel = float(err.norm() / O.norm())
        assert 0.01 < rel < 0.035, rel                          # the rounding is visible, and well inside 0.05
        assert float(err.abs().max()) < 0.25 * 2.0 ** -4 * float(V.abs().max())
