"""Head dims divisible by 8 without a kernel of their own (the README's "End-to-End Inference"
section: head dims divisible by 8, e.g. 120), on the GPU through the C ABI, against the fp64 oracle.

Such a D runs the row kernel of the next compiled head dim up with the real D as the row stride:
Q's padding columns read as zero and O's are never stored.  The cases cover every padded band from
D = 8 to 1016 in both dtypes with ragged tails, causal, GQA/MQA, boolean and additive masks, the
strided and packed entries, sampled rows of a multi-tile workload, and guard bands around O and LSE
(the padding columns of the last row must not be written past the tensor's end).
"""
import json

import numpy as np
import pytest
import torch

import exact_attention_head_amd as ffpa
import workloads as W
from gpu_helpers import compare, compare_varlen, run_gpu, run_gpu_varlen

pytestmark = pytest.mark.gpu

PADDED = [8, 16, 40, 80, 96, 112, 120, 136, 144, 200, 264, 328, 392, 456, 520, 552, 600, 712, 776, 904, 1000, 1016]


def _log(name, m):
    print(f"[headdim] {name}: {json.dumps(m)}", flush=True)


def test_padded_dims_map_to_the_next_row_kernel():
    for D in PADDED:
        kd = ffpa.kernel_head_dim(D)
        assert kd > D and kd % 64 == 0 and ffpa.kernel_name(D) == "ffpa_fwd_row_kernel", (D, kd)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("D", PADDED)
def test_padded_head_dim(D, dtype):
    q, k, v = W.random_qkv(1, 2, 2, 133, 197, D, dtype=dtype, seed=3000 + D)
    o, l = run_gpu(q, k, v)
    _log(f"D={D} {dtype}", compare(o, l, q, k, v))


@pytest.mark.parametrize("D", [80, 120, 520, 1000])
@pytest.mark.parametrize("Nq,Nkv", [(1, 1), (64, 64), (200, 333), (257, 260)])
def test_padded_causal_gqa(D, Nq, Nkv):
    q, k, v = W.random_qkv(2, 4, 2, Nq, Nkv, D, seed=D + Nq, factor=0.5)
    o, l = run_gpu(q, k, v, is_causal=True)
    _log(f"causal D={D} Nq={Nq} Nkv={Nkv}", compare(o, l, q, k, v, is_causal=True))


@pytest.mark.parametrize("kind", ["bool", "f32", "bf16"])
@pytest.mark.parametrize("D", [96, 200, 712])
def test_padded_masks(kind, D):
    B, H, Nq, Nkv = 2, 3, 130, 256
    q, k, v = W.random_qkv(B, H, 1, Nq, Nkv, D, seed=D + 17)
    g = torch.Generator().manual_seed(D)
    bias = torch.randn(B, 1, Nq, Nkv, generator=g)
    bias[torch.rand(B, 1, Nq, Nkv, generator=g) < 0.1] = float("-inf")
    bias[..., 0] = 0.0
    mask = bias > -0.5 if kind == "bool" else bias.to(torch.float32 if kind == "f32" else torch.bfloat16)
    if kind == "bool":
        mask[..., 0] = True
    o, l = run_gpu(q, k, v, mask=mask)
    _log(f"mask {kind} D={D}", compare(o, l, q, k, v, mask=mask))


@pytest.mark.parametrize("D", [80, 520])
def test_padded_strided_view(D):
    """[B, N, H, D] storage seen as [B, H, N, D]: read in place by the strided entry."""
    B, H, N = 2, 3, 150
    q, k, v = W.random_qkv(B, H, H, N, N, D, seed=D + 5)
    dev = torch.device("cuda:0")
    qs, ks, vs = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for t in (q, k, v))
    assert not qs.is_contiguous()
    o, l = ffpa.attn(qs, ks, vs, is_causal=True, return_lse=True)
    torch.cuda.synchronize()
    _log(f"strided D={D}", compare(o.cpu(), l.cpu(), q, k, v, is_causal=True))


@pytest.mark.parametrize("D", [120, 552])
def test_padded_varlen(D):
    lens_q, lens_k = [70, 1, 200, 0, 129], [90, 5, 200, 3, 129]
    Hq, Hkv = 4, 2
    cu_q = torch.tensor([0] + list(np.cumsum(lens_q)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(lens_k)), dtype=torch.int32)
    g = torch.Generator().manual_seed(D)
    q = torch.randn(int(cu_q[-1]), Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(int(cu_k[-1]), Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(int(cu_k[-1]), Hkv, D, generator=g).to(torch.bfloat16)
    for causal in (False, True):
        o, l = run_gpu_varlen(q, k, v, cu_q, cu_k, causal=causal)
        _log(f"varlen D={D} causal={causal}", compare_varlen(o, l, q, k, v, cu_q, cu_k, causal=causal))


def test_padded_multi_tile_sampled():
    """A multi-tile problem (B1 H8 N2048, D = 120) compared on sampled rows of every head."""
    q, k, v = W.random_qkv(1, 8, 8, 2048, 2048, 120, seed=120)
    o, l = run_gpu(q, k, v)
    rows = W.sample_rows(1, 8, 2048, seed=120)
    _log("B1 H8 N2048 D=120 sampled", compare(o, l, q, k, v, rows=rows))


@pytest.mark.parametrize("D", [40, 200, 1016])
def test_padded_in_bounds_and_deterministic(D):
    """Nothing outside O and LSE is written (the padding columns of the last rows lie past O's end),
    every element of O is written, and two launches agree bit for bit."""
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.random_qkv(1, 4, 2, 300, 333, D, seed=D + 11))
    B, Hq, Nq, _ = q.shape
    n, pad = B * Hq * Nq * D, 4096
    big = torch.full((n + 2 * pad,), float("nan"), dtype=q.dtype, device=dev)
    lbig = torch.full((B * Hq * Nq + 2 * pad,), 12345.0, dtype=torch.float32, device=dev)
    o = big[pad:pad + n].view(B, Hq, Nq, D)
    lse = lbig[pad:pad + B * Hq * Nq]
    outs = []
    for _ in range(2):
        st = ffpa.ffpa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), None, o.data_ptr(), lse.data_ptr(), B, Hq, 2,
                           Nq, 333, D, float("nan"), False, ffpa.FFPA_BF16, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(o.float()).all(), "some output element was not written"
    assert torch.isnan(big[:pad].float()).all() and torch.isnan(big[pad + n:].float()).all(), "O guard band written"
    assert (lbig[:pad] == 12345.0).all() and (lbig[pad + B * Hq * Nq:] == 12345.0).all(), "LSE guard band written"
    _log(f"guard D={D}", compare(o.cpu(), lse.cpu(), q.cpu(), k.cpu(), v.cpu()))
