"""FP8 forward (ffpa_fwd_fp8) on the GPU through the C ABI, against the fp64 oracle over the same e4m3
codes and per-head factors (oracle.attention_rows_fp8).

Tolerance, derived from the arithmetic: the logits are products of e4m3 values, exact in the fp32
accumulators up to the accumulation's rounding, so the LSE keeps the 16-bit forward's 1e-3.  The one
extra rounding is that of each probability to e4m3 (RNE, 3 fraction bits) for the P V product: each
weight moves by at most 2^-4 of itself, so |O_gpu - O| <= 2^-4 max|V'| + the output's own rounding
(2^-8 |O| in bf16), and for independent roundings the relative L2 error is about 2^-4 / sqrt(3) of the
spread of the weighted values; a numpy model of that one rounding on these workloads measures
0.021-0.027 (tests/test_fp8_tolerance.py).  The bar: max-abs <= 2^-4 max|V'| + 2^-8 max|O| and
rel-L2 <= 0.05.
"""
import json
import math

import numpy as np
import pytest
import torch

import exact_attention_head_amd as ffpa
import oracle
import workloads as W

pytestmark = pytest.mark.gpu
F8 = torch.float8_e4m3fn
REL_L2 = 0.05
LSE_MAX_ABS = 1e-3


def _log(name, m):
    print(f"[fp8] {name}: {json.dumps(m)}", flush=True)


def compare_fp8(o_gpu, lse_gpu, q, k, v, dq, dk, dv, rows=None, mask=None, is_causal=False, scale=None):
    B, Hq, Nq, D = q.shape
    og = o_gpu.float().reshape(-1, D)
    lg = lse_gpu.reshape(-1)
    assert torch.isfinite(og).all(), "non-finite values in O"
    assert not torch.isnan(lg).any() and not (lg == math.inf).any(), "NaN or +inf in LSE"
    rows = np.arange(B * Hq * Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    o_ref, l_ref = oracle.attention_rows_fp8(q, k, v, rows, dq, dk, dv, mask=mask, scale=scale, is_causal=is_causal)
    o_g = og.numpy().astype(np.float64)[rows]
    l_g = lg.numpy().astype(np.float64)[rows]
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_g), fin), "LSE finiteness differs from the oracle"
    assert np.all(l_g[~fin] == l_ref[~fin])
    vmax = float((v.double() * (dv.double()[:, :, None, None] if dv is not None else 1.0)).abs().max())
    err = np.abs(o_g - o_ref)
    max_abs = float(err.max()) if err.size else 0.0
    bound = 2.0 ** -4 * vmax + 2.0 ** -8 * float(np.abs(o_ref).max() if o_ref.size else 0.0)
    ref_norm = float(np.linalg.norm(o_ref))
    rel_l2 = float(np.linalg.norm(o_g - o_ref) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(o_g))
    lse_err = float(np.abs(l_g[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    m = dict(rows=int(rows.size), o_max_abs=max_abs, o_bound=bound, o_rel_l2=rel_l2, lse_max_abs=lse_err)
    assert max_abs <= bound, m
    assert rel_l2 <= REL_L2, m
    assert lse_err <= LSE_MAX_ABS, m
    return m


def fp8_inputs(B, Hq, Hkv, Nq, Nkv, D, seed, factors=True):
    """Seeded N(0, 1) tensors quantised per head to e4m3 (scale = head's max |x| / 448), with the
    factors that undo the quantisation (or none: the codes stand for themselves)."""
    q, k, v = W.random_qkv(B, Hq, Hkv, Nq, Nkv, D, dtype=torch.float32, seed=seed)
    out = []
    for x in (q, k, v):
        if factors:
            s = (x.abs().amax(dim=(2, 3)) / 448.0).clamp_min(1e-12)
            out += [(x / s[:, :, None, None]).to(F8), s.float()]
        else:
            out += [x.to(F8), None]
    q8, dq, k8, dk, v8, dv = out
    return q8, k8, v8, dq, dk, dv


def run_fp8(q8, k8, v8, dq, dk, dv, mask=None, is_causal=False, scale=None, out_dtype=torch.bfloat16):
    dev = torch.device("cuda:0")
    t = lambda x: None if x is None else x.to(dev)
    o, lse = ffpa.attn_fp8(t(q8), t(k8), t(v8), t(dq), t(dk), t(dv), attn_mask=t(mask), is_causal=is_causal,
                           scale=scale, enable_gqa=q8.shape[1] != k8.shape[1], return_lse=True, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("D", [128, 256, 384, 512, 768, 1024])
def test_fp8_every_head_dim(D, out_dtype):
    q8, k8, v8, dq, dk, dv = fp8_inputs(1, 2, 2, 133, 197, D, seed=D)
    o, l = run_fp8(q8, k8, v8, dq, dk, dv, out_dtype=out_dtype)
    _log(f"D={D} {out_dtype}", compare_fp8(o, l, q8, k8, v8, dq, dk, dv))


@pytest.mark.parametrize("D", [16, 64, 80, 112, 208, 320, 448, 496, 528, 640, 784, 1008])
def test_fp8_padded_head_dims(D):
    q8, k8, v8, dq, dk, dv = fp8_inputs(1, 2, 1, 150, 170, D, seed=D + 1)
    o, l = run_fp8(q8, k8, v8, dq, dk, dv)
    _log(f"padded D={D}", compare_fp8(o, l, q8, k8, v8, dq, dk, dv))


@pytest.mark.parametrize("Nq,Nkv", [(1, 1), (7, 7), (64, 64), (65, 63), (128, 256), (129, 333), (333, 1), (1, 333)])
@pytest.mark.parametrize("D", [128, 512, 1024])
def test_fp8_sequence_shapes(Nq, Nkv, D):
    q8, k8, v8, dq, dk, dv = fp8_inputs(1, 2, 1, Nq, Nkv, D, seed=Nq * 7 + Nkv)
    o, l = run_fp8(q8, k8, v8, dq, dk, dv)
    _log(f"Nq={Nq} Nkv={Nkv} D={D}", compare_fp8(o, l, q8, k8, v8, dq, dk, dv))


@pytest.mark.parametrize("Nq,Nkv", [(1, 1), (64, 64), (200, 200), (100, 333), (257, 260)])
@pytest.mark.parametrize("D", [128, 384, 512, 768, 1024])
def test_fp8_causal_gqa(Nq, Nkv, D):
    q8, k8, v8, dq, dk, dv = fp8_inputs(2, 4, 2, Nq, Nkv, D, seed=Nq + Nkv + D)
    o, l = run_fp8(q8, k8, v8, dq, dk, dv, is_causal=True)
    _log(f"causal Nq={Nq} Nkv={Nkv} D={D}", compare_fp8(o, l, q8, k8, v8, dq, dk, dv, is_causal=True))


@pytest.mark.parametrize("kind", ["bool", "f32", "bf16", "fp16"])
@pytest.mark.parametrize("D", [128, 512, 1024])
@pytest.mark.parametrize("Nkv", [256, 333])
def test_fp8_masks(kind, D, Nkv):
    B, H, Nq = 2, 3, 130
    q8, k8, v8, dq, dk, dv = fp8_inputs(B, H, H, Nq, Nkv, D, seed=D + Nkv)
    g = torch.Generator().manual_seed(D * 3 + Nkv)
    bias = torch.randn(B, 1, Nq, Nkv, generator=g)
    bias[torch.rand(B, 1, Nq, Nkv, generator=g) < 0.1] = float("-inf")
    bias[..., 0] = 0.0
    if kind == "bool":
        mask = bias > -0.5
        mask[..., 0] = True
    else:
        mask = bias.to({"f32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[kind])
    o, l = run_fp8(q8, k8, v8, dq, dk, dv, mask=mask)
    _log(f"mask {kind} D={D} Nkv={Nkv}", compare_fp8(o, l, q8, k8, v8, dq, dk, dv, mask=mask))


def test_fp8_mask_with_causal_and_fully_masked_rows():
    B, H, N, D = 1, 2, 200, 256
    q8, k8, v8, dq, dk, dv = fp8_inputs(B, H, H, N, N, D, seed=9)
    mask = torch.ones(B, 1, N, N, dtype=torch.bool)
    mask[:, :, 5] = False  # row 5 sees no key at all: O = 0, LSE = -inf
    mask[:, :, 10:20, :3] = False
    o, l = run_fp8(q8, k8, v8, dq, dk, dv, mask=mask, is_causal=True)
    m = compare_fp8(o, l, q8, k8, v8, dq, dk, dv, mask=mask, is_causal=True)
    assert torch.all(o[:, :, 5] == 0) and torch.all(l[:, :, 5] == -math.inf)
    _log("mask+causal with an empty row", m)


def test_fp8_codes_without_factors_and_explicit_scales():
    q8, k8, v8, _, _, _ = fp8_inputs(1, 2, 2, 150, 256, 256, seed=12, factors=False)
    for scale in (None, 0.01, -0.02, 0.0):
        o, l = run_fp8(q8, k8, v8, None, None, None, scale=scale)
        _log(f"no factors scale={scale}", compare_fp8(o, l, q8, k8, v8, None, None, None, scale=scale))


@pytest.mark.parametrize("H,N,D", [(8, 4096, 512), (16, 4096, 1024)])
def test_fp8_full_size_sampled(H, N, D):
    """The fp8 benchmark shapes (per-head factors) on sampled rows of every head."""
    q8, k8, v8, dq, dk, dv = fp8_inputs(1, H, H, N, N, D, seed=2)
    o, l = run_fp8(q8, k8, v8, dq, dk, dv)
    rows = W.sample_rows(1, H, N, seed=2)
    _log(f"B1 H{H} N{N} D{D} sampled", compare_fp8(o, l, q8, k8, v8, dq, dk, dv, rows=rows))


@pytest.mark.parametrize("D", [208, 784])
def test_fp8_in_bounds_and_deterministic(D):
    dev = torch.device("cuda:0")
    q8, k8, v8, dq, dk, dv = fp8_inputs(1, 4, 2, 300, 333, D, seed=11)
    B, Hq, Nq, D = q8.shape
    n, pad = B * Hq * Nq * D, 4096
    big = torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device=dev)
    lbig = torch.full((B * Hq * Nq + 2 * pad,), 12345.0, dtype=torch.float32, device=dev)
    o = big[pad:pad + n].view(B, Hq, Nq, D)
    lse = lbig[pad:pad + B * Hq * Nq]
    qd, kd, vd, dqd, dkd, dvd = (x.to(dev) for x in (q8, k8, v8, dq, dk, dv))
    outs = []
    for _ in range(2):
        st = ffpa.ffpa_fwd_fp8(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), dqd.data_ptr(), dkd.data_ptr(),
                               dvd.data_ptr(), None, o.data_ptr(), lse.data_ptr(), B, Hq, 2, Nq, 333, D, float("nan"),
                               False, ffpa.FFPA_BF16, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(o.float()).all(), "some output element was not written"
    assert torch.isnan(big[:pad].float()).all() and torch.isnan(big[pad + n:].float()).all(), "O guard band written"
    assert (lbig[:pad] == 12345.0).all() and (lbig[pad + B * Hq * Nq:] == 12345.0).all(), "LSE guard band written"
    _log(f"guard D={D}", compare_fp8(o.cpu(), lse.cpu(), q8, k8, v8, dq, dk, dv))
