"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Small cases compare every row and span several tiles plus ragged tails in both sequence
dimensions, for every head-dim band of the kernels.  The five full-size workloads run in the
launch configuration the benchmark times and are compared on seeded sampled rows (one per 64-row
bucket of every head, plus boundary rows), with every output element scanned for NaN/inf.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import compare, run_gpu

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, Nq, Nkv, D, dtype=torch.bfloat16, seed=0, factor=1.0):
    return W.random_qkv(B, Hq, Hkv, Nq, Nkv, D, dtype=dtype, seed=seed, factor=factor)


def _log(name, m):
    print(f"[parity] {name}: {json.dumps(m)}", flush=True)


# ---- every head-dim kernel, both dtypes, with ragged tails (Nq, Nkv not multiples of the tiles)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("D", list(range(64, 1025, 64)))
def test_every_head_dim(D, dtype):
    q, k, v = _case(1, 2, 2, 133, 197, D, dtype=dtype, seed=D)
    o, l = run_gpu(q, k, v)
    _log(f"D={D} {dtype}", compare(o, l, q, k, v))


# ---- shapes: tails, single rows/keys, MQA, GQA, cross-attention
@pytest.mark.parametrize("Nq,Nkv", [(1, 1), (7, 7), (63, 65), (65, 63), (127, 129), (129, 333), (333, 1), (1, 333),
                                    (256, 64), (64, 256)])
@pytest.mark.parametrize("D", [64, 320, 512, 576, 1024])
def test_sequence_shapes(Nq, Nkv, D):
    q, k, v = _case(1, 2, 1, Nq, Nkv, D, seed=Nq * 1000 + Nkv)
    o, l = run_gpu(q, k, v)
    _log(f"Nq={Nq} Nkv={Nkv} D={D}", compare(o, l, q, k, v))


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 2), (6, 3), (3, 3)])
@pytest.mark.parametrize("D", [128, 512, 1024])
def test_gqa_mqa(Hq, Hkv, D):
    q, k, v = _case(2, Hq, Hkv, 150, 210, D, seed=Hq * 10 + Hkv)
    o, l = run_gpu(q, k, v)
    _log(f"Hq={Hq} Hkv={Hkv} D={D}", compare(o, l, q, k, v))


# ---- tail-aligned causal, including Nq < Nkv and single-row edge cases
@pytest.mark.parametrize("Nq,Nkv", [(1, 1), (64, 64), (200, 200), (100, 333), (1, 300), (257, 260)])
@pytest.mark.parametrize("D", [64, 256, 512, 1024])
def test_causal(Nq, Nkv, D):
    q, k, v = _case(1, 4, 2, Nq, Nkv, D, seed=Nq + Nkv, factor=0.5)
    o, l = run_gpu(q, k, v, is_causal=True)
    _log(f"causal Nq={Nq} Nkv={Nkv} D={D}", compare(o, l, q, k, v, is_causal=True))


# ---- masks: bool / additive fp32 / bf16 / fp16, broadcast shapes, unaligned strides, masked rows
def _bias(shape, seed, drop=0.1):
    g = torch.Generator().manual_seed(seed)
    b = torch.randn(*shape, generator=g)
    b[torch.rand(*shape, generator=g) < drop] = float("-inf")
    b[..., 0] = 0.0  # every row keeps a key
    return b


@pytest.mark.parametrize("kind", ["bool", "f32", "bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 320, 512, 1024])
@pytest.mark.parametrize("Nkv", [256, 333, 7])
def test_masks(kind, D, Nkv):
    dtype = torch.float16 if kind == "fp16" else torch.bfloat16
    B, H, Nq = 2, 3, 130
    q, k, v = _case(B, H, H, Nq, Nkv, D, dtype=dtype, seed=D + Nkv)
    bias = _bias((B, 1, Nq, Nkv), seed=D * 7 + Nkv)
    if kind == "bool":
        mask = bias > -0.5
        mask[..., 0] = True
    else:
        mask = bias.to({"f32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[kind])
    o, l = run_gpu(q, k, v, mask=mask)
    _log(f"mask {kind} D={D} Nkv={Nkv}", compare(o, l, q, k, v, mask=mask))


@pytest.mark.parametrize("shape", [(130, 200), (1, 1, 130, 200), (2, 3, 130, 200), (2, 1, 1, 200), (1, 3, 130, 200)])
def test_mask_broadcast(shape):
    q, k, v = _case(2, 3, 3, 130, 200, 256, seed=5)
    mask = _bias(shape, seed=6)
    o, l = run_gpu(q, k, v, mask=mask)
    _log(f"mask shape {shape}", compare(o, l, q, k, v, mask=mask))


@pytest.mark.parametrize("shape", [(130, 256), (1, 1, 130, 256), (2, 1, 1, 256), (1, 3, 1, 256), (2, 3, 130, 256)])
@pytest.mark.parametrize("D", [256, 512, 1024])
def test_fp32_mask_staged_shapes(shape, D):
    """fp32 masks over whole 64-key tiles (staged through LDS by the kernels), with broadcast batch,
    head and row strides and a partial last query tile."""
    q, k, v = _case(2, 3, 3, 130, 256, D, seed=D + len(shape))
    mask = _bias(shape, seed=D * 3 + sum(shape))
    o, l = run_gpu(q, k, v, mask=mask)
    _log(f"staged mask shape {shape} D={D}", compare(o, l, q, k, v, mask=mask))


@pytest.mark.parametrize("shape", [(130, 256), (1, 1, 130, 256), (2, 1, 1, 256), (1, 3, 1, 256), (2, 3, 130, 256)])
@pytest.mark.parametrize("D", [128, 256, 512, 1024])
def test_bool_mask_staged_shapes(shape, D):
    """Boolean byte masks over whole 64-key tiles (staged through LDS by the row kernel), with
    broadcast batch, head and row strides and a partial last query tile."""
    q, k, v = _case(2, 3, 3, 130, 256, D, seed=D + 2 * len(shape))
    mask = _bias(shape, seed=D * 11 + sum(shape), drop=0.3) > -0.5
    mask[..., 0] = True
    o, l = run_gpu(q, k, v, mask=mask)
    _log(f"staged bool mask shape {shape} D={D}", compare(o, l, q, k, v, mask=mask))


@pytest.mark.parametrize("kind", ["bool", "f32"])
@pytest.mark.parametrize("D", [512, 1024])
@pytest.mark.parametrize("Nkv", [64, 128])
def test_mask_staged_few_key_tiles(kind, D, Nkv):
    """Staged masks over one or two key tiles: the ring's first epochs (issued together with the Q
    rows) then cover most or all of the keys, and at D = 1024 the staged-mask variants advance the
    ring in 16-product epochs."""
    q, k, v = _case(2, 2, 2, 130, Nkv, D, seed=D + Nkv + (kind == "bool"))
    bias = _bias((2, 1, 130, Nkv), seed=D * 7 + Nkv)
    if kind == "bool":
        mask = bias > -0.5
        mask[..., 0] = True
    else:
        mask = bias
    o, l = run_gpu(q, k, v, mask=mask)
    _log(f"staged mask {kind} D={D} Nkv={Nkv}", compare(o, l, q, k, v, mask=mask))

@pytest.mark.parametrize("D", [64, 512, 1024])
def test_bool_mask_staged_dead_rows(D):
    """Rows whose mask admits no key get O = 0 and LSE = -inf on the staged path too."""
    q, k, v = _case(1, 2, 2, 100, 128, D, seed=D + 77)
    mask = _bias((1, 2, 100, 128), seed=D + 78, drop=0.3) > -0.5
    mask[:, :, ::7] = False
    o, l = run_gpu(q, k, v, mask=mask)
    _log(f"staged bool mask dead rows D={D}", compare(o, l, q, k, v, mask=mask))
    assert torch.all(l[:, :, ::7] == -math.inf) and torch.all(o[:, :, ::7] == 0)


@pytest.mark.parametrize("kind", ["bool", "f32"])
@pytest.mark.parametrize("D", [64, 256, 512, 1024])
@pytest.mark.parametrize("Nq,Nkv", [(130, 200), (64, 64), (100, 333)])
def test_mask_and_causal(kind, D, Nq, Nkv):
    """A mask together with the tail-aligned causal rule: a key takes part only where both admit it."""
    B, H = 2, 2
    q, k, v = _case(B, H, H, Nq, Nkv, D, seed=D + Nq + (kind == "bool"))
    bias = _bias((B, 1, Nq, Nkv), seed=D * 5 + Nkv)
    if kind == "bool":
        mask = bias > -0.5
        mask[..., 0] = True
    else:
        mask = bias
    o, l = run_gpu(q, k, v, mask=mask, is_causal=True)
    _log(f"mask {kind} + causal D={D} Nq={Nq} Nkv={Nkv}", compare(o, l, q, k, v, mask=mask, is_causal=True))


def test_fully_masked_rows():
    """Rows with every key excluded: O = 0 and LSE = -inf (the convention of the oracle)."""
    q, k, v = _case(1, 2, 2, 70, 90, 512, seed=8)
    keep = torch.rand(1, 2, 70, 90, generator=torch.Generator().manual_seed(9)) < 0.5
    keep[..., 0] = True
    keep[0, 0, 3] = False
    keep[0, 1, 69] = False
    o, l = run_gpu(q, k, v, mask=keep)
    assert torch.all(o[0, 0, 3] == 0) and l[0, 0, 3] == -math.inf
    assert torch.all(o[0, 1, 69] == 0) and l[0, 1, 69] == -math.inf
    _log("fully masked rows", compare(o, l, q, k, v, mask=keep))


def test_explicit_scale_and_large_logits():
    """An explicit scale, and logits large enough that the running maximum moves many times.  Only Q and K
    are scaled up: V stays N(0,1) so that the bf16 rounding of O stays inside the absolute bar."""
    q, k, v = _case(1, 2, 2, 100, 700, 256, seed=10)
    q, k = (q.float() * 3).to(q.dtype), (k.float() * 3).to(k.dtype)
    o, l = run_gpu(q, k, v, scale=0.3)
    _log("scale 0.3, x3 inputs", compare(o, l, q, k, v, scale=0.3))
    # increasing additive bias along the keys forces a rescale on every tile
    ramp = torch.arange(700, dtype=torch.float32).view(1, 1, 1, 700) * 0.2
    o, l = run_gpu(q, k, v, mask=ramp)
    _log("ramp bias", compare(o, l, q, k, v, mask=ramp))


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.05])
@pytest.mark.parametrize("D", [256, 512, 1024])
def test_nonpositive_and_small_scales(scale, D):
    """Whole 64-key tiles without a mask: a positive scale runs the raw-logit variant (row maximum over
    raw dot products), zero and negative scales must take the explicit one."""
    q, k, v = _case(1, 2, 2, 130, 256, D, seed=D + int(scale * 100))
    o, l = run_gpu(q, k, v, scale=scale)
    _log(f"scale {scale} D={D}", compare(o, l, q, k, v, scale=scale))
    o, l = run_gpu(q, k, v, scale=scale, is_causal=True)
    _log(f"scale {scale} D={D} causal", compare(o, l, q, k, v, scale=scale, is_causal=True))


def test_golden_fixtures_on_gpu():
    """The hand-worked fixtures, zero-padded to D = 64 (padding adds nothing to any dot product)."""
    import glob

    from test_golden import load_fixture

    for path in sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json"))):
        fx, q, k, v, mask, O_want, L_want = load_fixture(path, torch.bfloat16)
        D0 = q.shape[-1]
        pad = lambda t: torch.nn.functional.pad(t, (0, 64 - D0))
        scale = fx["scale"] if fx["scale"] is not None else 1.0 / math.sqrt(D0)
        o, l = run_gpu(pad(q), pad(k), pad(v), mask=mask, is_causal=fx["is_causal"], scale=scale)
        assert np.allclose(o[..., :D0].double().numpy(), O_want, atol=1e-2, rtol=0), path
        assert torch.all(o[..., D0:] == 0)
        assert np.allclose(l.double().numpy(), L_want, atol=1e-4, rtol=0), path


def test_deterministic_and_in_bounds():
    """Two launches give bitwise-identical results, and nothing outside O and LSE is written."""
    import exact_attention_head_amd as ffpa

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in _case(1, 4, 2, 300, 333, 512, seed=11))
    B, Hq, Nq, D = q.shape
    n, pad = B * Hq * Nq * D, 4096
    big = torch.full((n + 2 * pad,), float("nan"), dtype=q.dtype, device=dev)
    lbig = torch.full((B * Hq * Nq + 2 * pad,), 12345.0, dtype=torch.float32, device=dev)
    o = big[pad:pad + n].view(B, Hq, Nq, D)
    lse = lbig[pad:pad + B * Hq * Nq]
    outs = []
    for _ in range(2):
        st = ffpa.ffpa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), None, o.data_ptr(), lse.data_ptr(), B, Hq,
                           2, Nq, 333, D, float("nan"), False, ffpa.FFPA_BF16,
                           torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(o.float()).all(), "some output element was not written"
    assert torch.isnan(big[:pad].float()).all() and torch.isnan(big[pad + n:].float()).all(), "O guard band written"
    assert (lbig[:pad] == 12345.0).all() and (lbig[pad + B * Hq * Nq:] == 12345.0).all(), "LSE guard band written"


def test_largest_head_at_the_offset_limit():
    """One K/V head just under the 2 GiB the kernels' 32-bit buffer offsets allow (D = 1024,
    1,048,448 keys, K and V 2 GiB each), with a ragged query count: every key's offset is formed and
    range-checked near the top of the range, and the rows are compared with the oracle."""
    import exact_attention_head_amd as ffpa

    D, Nq, Nkv = 1024, 65, (1 << 20) - 128
    assert Nkv * D * 2 < (1 << 31) and (Nkv + 128) * D * 2 >= (1 << 31)
    q, k, v = _case(1, 1, 1, Nq, Nkv, D, seed=77)
    fake = [(i + 1) << 36 for i in range(4)]  # aligned stand-ins: the check never dereferences them
    assert ffpa.ffpa_check_args(fake[0], fake[1], fake[2], None, fake[3], None, 1, 1, 1, Nq, Nkv + 128, D,
                                float("nan"), False, ffpa.FFPA_BF16) == ffpa.ERR_UNSUPPORTED
    o, l = run_gpu(q, k, v)
    _log(f"offset limit Nkv={Nkv} D={D}", compare(o, l, q, k, v))
    del q, k, v


# ---- the five full-size workloads, in the benchmark's launch configuration, on sampled rows
@pytest.mark.parametrize("name", ["tiny", "large_d_self", "gqa_causal", "cross_mask"])
def test_full_size_workloads(name):
    w = getattr(W, name)()
    q, k, v, mask = W.make_inputs(w)
    o, l = run_gpu(q, k, v, mask=mask, is_causal=w.causal)
    rows = None if name == "tiny" else W.sample_rows(w.B, w.Hq, w.Nq, seed=w.seed)
    _log(w.name, compare(o, l, q, k, v, rows=rows, mask=mask, is_causal=w.causal))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("D", list(W.SWEEP_D))
def test_head_dim_sweep_workload(D, dtype):
    w = W.sweep(D, dtype)
    q, k, v, _ = W.make_inputs(w)
    o, l = run_gpu(q, k, v)
    rows = W.sample_rows(w.B, w.Hq, w.Nq, seed=w.seed, bucket=512)
    _log(w.name, compare(o, l, q, k, v, rows=rows))


def test_pages_function_name_runs_attn():
    """ffpa_attn_func (the "API Reference" name) gives attn's result bit for bit, backend keywords
    and all."""
    import exact_attention_head_amd as ffpa

    q, k, v = _case(1, 4, 2, 100, 130, 512, seed=41)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    want = ffpa.attn(qd, kd, vd, is_causal=True, enable_gqa=True)
    got = ffpa.ffpa_attn_func(qd, kd, vd, is_causal=True, enable_gqa=True, backend="triton")
    assert torch.equal(got, want)
