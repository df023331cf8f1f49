"""Attention dropout on the GPU: the keep-bit generator and the forward with dropout, through the C ABI.

- The generator (ffpa_dropout_keep) must reproduce the oracle's Philox4x32-10 keep words bit for
  bit, for ragged key counts, several seeds, offsets and probabilities.
- The forward with dropout (ffpa_fwd_dropout) takes keep words drawn by the oracle on the CPU (no
  input of the oracle comes from the GPU) and is compared element by element with
  oracle.attention_dropout_rows to the tolerances of the plain forward; the LSE must equal the
  plain forward's (dropout leaves it unchanged).  Every head-dim kernel, causal, GQA, masks, fp16,
  and the D=512 self-attention workload at full size on sampled rows are covered.
"""
import json
import math

import numpy as np
import pytest
import torch

import exact_attention_head_amd as ffpa
import oracle
import workloads as W
from gpu_helpers import LSE_MAX_ABS, O_MAX_ABS, O_REL_L2
from oracle.philox import dropout_keep_bits, dropout_keep_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _log(name, m):
    print(f"[dropout] {name}: {json.dumps(m)}", flush=True)


def _as_int32(words: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32))


@pytest.mark.parametrize("B,Hq,Nq,Nkv", [(1, 1, 1, 1), (2, 3, 17, 70), (1, 2, 64, 256), (1, 1, 5, 33), (2, 1, 9, 95)])
@pytest.mark.parametrize("p", [0.0, 0.1, 0.5, 0.9])
@pytest.mark.parametrize("seed,offset", [(0, 0), (2**40 + 3, 7), (12345, 2**31 + 5)])
def test_keep_bits_match_oracle(B, Hq, Nq, Nkv, p, seed, offset):
    keep = ffpa.dropout_keep(B, Hq, Nq, Nkv, p, seed, offset, DEV)
    torch.cuda.synchronize()
    got = keep.cpu().numpy().view(np.uint32)
    want = dropout_keep_bits(B, Hq, Nq, Nkv, p, seed, offset)
    assert np.array_equal(got, want)


def _check(q, k, v, keep_words, p, mask=None, is_causal=False, rows=None, name=""):
    B, Hq, Nq, D = q.shape
    md = mask.to(DEV) if mask is not None else None
    o, lse = ffpa.attn(q.to(DEV), k.to(DEV), v.to(DEV), attn_mask=md, dropout_p=p, is_causal=is_causal,
                       enable_gqa=q.shape[1] != k.shape[1], return_lse=True,
                       dropout_keep=_as_int32(keep_words).to(DEV))
    torch.cuda.synchronize()
    og = o.cpu().float().reshape(-1, D)
    lg = lse.cpu().reshape(-1)
    assert torch.isfinite(og).all() and not torch.isnan(lg).any()
    if rows is None:
        rows = np.arange(B * Hq * Nq)
    o_ref, l_ref = oracle.attention_dropout_rows(q, k, v, rows, keep_words, p, mask=mask, is_causal=is_causal)
    o_g = og.numpy().astype(np.float64)[rows]
    l_g = lg.numpy().astype(np.float64)[rows]
    max_abs = float(np.abs(o_g - o_ref).max())
    ref = float(np.linalg.norm(o_ref))
    rel = float(np.linalg.norm(o_g - o_ref) / ref) if ref > 0 else float(np.linalg.norm(o_g))
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_g), fin)
    lse_err = float(np.abs(l_g[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    m = dict(rows=int(len(rows)), o_max_abs=max_abs, o_rel_l2=rel, lse_max_abs=lse_err)
    _log(name, m)
    # Dropout multiplies the output by s = 1 / (1 - p): O = s * sum_k P_k Z_k v_k, a sub-sum of the
    # plain output's terms scaled by s.  The rounding of P to 16 bits and of O to the output type
    # scale with |O|, hence with s, so the plain forward's absolute bar is scaled by s; the relative
    # L2 bar and the LSE bar (dropout leaves the LSE alone) are those of the plain forward.
    s = 1.0 / (1.0 - float(np.float32(p)))
    assert max_abs <= O_MAX_ABS * s and rel <= O_REL_L2 and lse_err <= LSE_MAX_ABS, m


# (head dims without a kernel of their own run the next one padded: 8, 80, 200, 520, 576, 704, 832,
# 960 and 1016 here)
@pytest.mark.parametrize("D", [8, 64, 80, 128, 192, 200, 256, 320, 512, 520, 576, 704, 768, 832, 960, 1016, 1024])
def test_dropout_every_kernel(D):
    B, Hq, Hkv, Nq, Nkv, p = 1, 2, 2, 133, 197, 0.3
    q, k, v = W.random_qkv(B, Hq, Hkv, Nq, Nkv, D, seed=D + 1)
    _check(q, k, v, dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=D), p, name=f"D={D}")


@pytest.mark.parametrize("p", [0.0, 0.1, 0.5, 0.9])
@pytest.mark.parametrize("D", [128, 512, 1024])
def test_dropout_probabilities(p, D):
    B, Hq, Nq, Nkv = 1, 2, 96, 160
    q, k, v = W.random_qkv(B, Hq, 1, Nq, Nkv, D, seed=7)
    _check(q, k, v, dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=3), p, name=f"p={p} D={D} MQA")


@pytest.mark.parametrize("D", [64, 200, 256, 512, 640, 904, 1024])
def test_dropout_causal_gqa(D):
    B, Hq, Hkv, Nq, Nkv, p = 2, 4, 2, 100, 229, 0.2
    q, k, v = W.random_qkv(B, Hq, Hkv, Nq, Nkv, D, seed=11)
    _check(q, k, v, dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=5), p, is_causal=True, name=f"causal GQA D={D}")


@pytest.mark.parametrize("kind", ["bool", "f32", "bf16"])
@pytest.mark.parametrize("D", [128, 512, 832])
def test_dropout_with_mask(kind, D):
    B, Hq, Nq, Nkv, p = 2, 2, 70, 131, 0.25
    q, k, v = W.random_qkv(B, Hq, Hq, Nq, Nkv, D, seed=13)
    g = torch.Generator().manual_seed(17)
    if kind == "bool":
        mask = torch.rand(B, 1, Nq, Nkv, generator=g) > 0.2
        mask[..., 0] = True
    else:
        mask = torch.randn(B, 1, Nq, Nkv, generator=g)
        mask = mask if kind == "f32" else mask.to(torch.bfloat16)
    _check(q, k, v, dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=9), p, mask=mask, name=f"mask {kind} D={D}")


@pytest.mark.parametrize("D", [256, 512, 1024])
def test_dropout_fp16(D):
    B, Hq, Nq, Nkv, p = 1, 2, 120, 150, 0.4
    q, k, v = W.random_qkv(B, Hq, Hq, Nq, Nkv, D, dtype=torch.float16, seed=19)
    _check(q, k, v, dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=21), p, name=f"fp16 D={D}")


def test_dropout_arbitrary_bits():
    """Any keep words are accepted: all kept, none kept, and a checkerboard."""
    B, Hq, Nq, Nkv, D, p = 1, 1, 64, 128, 512, 0.5
    q, k, v = W.random_qkv(B, Hq, Hq, Nq, Nkv, D, seed=23)
    Wd = (Nkv + 31) // 32
    for name, word in (("all", 0xFFFFFFFF), ("none", 0), ("alternate", 0x55555555)):
        words = np.full((B, Hq, Nq, Wd), word, dtype=np.uint32)
        _check(q, k, v, words, p, name=f"bits {name}")


def test_dropout_self_attention_full_size():
    """The D=512 self-attention workload (B=1 H=8 N=4096) with p = 0.1, on sampled rows whose keep
    words come from the oracle; the GPU generator is checked on the same rows."""
    w = W.large_d_self()
    q, k, v, _ = W.make_inputs(w)
    p, seed = 0.1, 2024
    rows = np.asarray(W.sample_rows(w.B, w.Hq, w.Nq, seed=w.seed, bucket=256), dtype=np.int64)
    Wd = (w.Nkv + 31) // 32
    words = np.full((w.B * w.Hq * w.Nq, Wd), 0xFFFFFFFF, dtype=np.uint32)
    words[rows] = dropout_keep_rows(rows, w.Nkv, p, seed)
    words = words.reshape(w.B, w.Hq, w.Nq, Wd)
    _check(q, k, v, words, p, rows=rows, name="self B1 H8 N4096 D512 p=0.1")
    gen = ffpa.dropout_keep(w.B, w.Hq, w.Nq, w.Nkv, p, seed, 0, DEV)
    torch.cuda.synchronize()
    got = gen.cpu().numpy().view(np.uint32).reshape(-1, Wd)[rows]
    assert np.array_equal(got, words.reshape(-1, Wd)[rows])


def test_dropout_generated_end_to_end():
    """attn draws its own bits from dropout_seed; the returned words match the oracle's and the output
    matches the oracle on them."""
    B, Hq, Nq, Nkv, D, p, seed = 1, 2, 80, 140, 384, 0.3, 77
    q, k, v = W.random_qkv(B, Hq, Hq, Nq, Nkv, D, seed=29)
    o, keep = ffpa.attn(q.to(DEV), k.to(DEV), v.to(DEV), dropout_p=p, dropout_seed=seed, return_dropout_keep=True)
    torch.cuda.synchronize()
    words = dropout_keep_bits(B, Hq, Nq, Nkv, p, seed)
    assert np.array_equal(keep.cpu().numpy().view(np.uint32), words)
    o_ref, _ = oracle.attention_dropout_rows(q, k, v, np.arange(B * Hq * Nq), words, p)
    err = np.abs(o.cpu().double().numpy().reshape(-1, D) - o_ref)
    assert err.max() <= O_MAX_ABS / (1 - p)


def test_dropout_argument_errors():
    q, k, v = (t.to(DEV) for t in W.random_qkv(1, 1, 1, 8, 8, 64, seed=1))
    with pytest.raises(ValueError):
        ffpa.attn(q, k, v, dropout_p=1.0)
    with pytest.raises(ValueError):
        ffpa.attn(q, k, v, dropout_p=0.5, dropout_keep=torch.zeros(1, 1, 8, 2, dtype=torch.int32, device=DEV))
    st = ffpa.ffpa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), None, torch.empty_like(q).data_ptr(), None,
                               1, 1, 1, 8, 8, 64, math.nan, False, ffpa.FFPA_BF16, None, 0.5, None)
    assert st == 2  # null keep


# ---- the backward of the forward with dropout (ffpa_bwd_dropout), against the oracle's gradients.
# Bar of the plain backward: P and dS rounded once to 16 bits, the outputs once more; rel-L2 <= 1e-2
# and a largest element error <= 2e-2 of the largest reference magnitude.
def _bwd_compare(got, want, name):
    m = {}
    for nm, g, w in zip(("dq", "dk", "dv"), got, want):
        g = g.double().numpy()
        assert np.isfinite(g).all(), f"non-finite values in {nm}"
        rel = float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30))
        mx = float(np.abs(g - w).max() / max(np.abs(w).max(), 1e-30))
        m[nm] = dict(rel_l2=rel, max_rel=mx)
        assert rel <= 1e-2 and mx <= 2e-2, (nm, m)
    _log(name, m)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [72, 128, 512, 576, 1024])
def test_backward_dropout(D, causal):
    B, Hq, Hkv, Nq, Nkv, p = 1, 4, 2, 96, 160, 0.2
    q, k, v = W.random_qkv(B, Hq, Hkv, Nq, Nkv, D, seed=31 + D)
    do = torch.randn(B, Hq, Nq, D, generator=torch.Generator().manual_seed(D)).to(torch.bfloat16)
    words = dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=D + 5)
    keep = _as_int32(words).to(DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = ffpa.attn(qd, kd, vd, dropout_p=p, dropout_keep=keep, is_causal=causal, enable_gqa=True,
                       return_lse=True)
    got = ffpa.attn_backward(qd, kd, vd, o, dod, lse, is_causal=causal, dropout_p=p, dropout_keep=keep)
    torch.cuda.synchronize()
    want = oracle.attention_backward(q, k, v, do, is_causal=causal, keep_bits=words, dropout_p=p)
    _bwd_compare([t.cpu() for t in got], want, f"backward D={D} causal={causal}")


def test_backward_dropout_with_mask():
    B, Hq, Nq, Nkv, D, p = 2, 2, 64, 100, 256, 0.3
    q, k, v = W.random_qkv(B, Hq, Hq, Nq, Nkv, D, seed=41)
    do = torch.randn(B, Hq, Nq, D, generator=torch.Generator().manual_seed(41)).to(torch.bfloat16)
    mask = torch.randn(B, 1, Nq, Nkv, generator=torch.Generator().manual_seed(42))
    words = dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=43)
    keep = _as_int32(words).to(DEV)
    qd, kd, vd, dod, md = (t.to(DEV) for t in (q, k, v, do, mask))
    o, lse = ffpa.attn(qd, kd, vd, attn_mask=md, dropout_p=p, dropout_keep=keep, return_lse=True)
    got = ffpa.attn_backward(qd, kd, vd, o, dod, lse, attn_mask=md, dropout_p=p, dropout_keep=keep)
    torch.cuda.synchronize()
    want = oracle.attention_backward(q, k, v, do, mask=mask, keep_bits=words, dropout_p=p)
    _bwd_compare([t.cpu() for t in got], want, "backward with mask")


@pytest.mark.parametrize("D", [320, 200])
def test_autograd_with_dropout(D):
    """attn_with_grad draws its keep words from the seed; the gradients match the oracle's for the
    oracle's own words of that seed (D = 200: a padded head dim, forward and backward)."""
    B, Hq, Nq, Nkv, p, seed = 1, 2, 80, 130, 0.25, 99
    q, k, v = W.random_qkv(B, Hq, Hq, Nq, Nkv, D, seed=51)
    do = torch.randn(B, Hq, Nq, D, generator=torch.Generator().manual_seed(52)).to(torch.bfloat16)
    qd, kd, vd = (t.to(DEV).requires_grad_(True) for t in (q, k, v))
    o = ffpa.attn_with_grad(qd, kd, vd, dropout_p=p, dropout_seed=seed)
    o.backward(do.to(DEV))
    torch.cuda.synchronize()
    words = dropout_keep_bits(B, Hq, Nq, Nkv, p, seed)
    want = oracle.attention_backward(q, k, v, do, keep_bits=words, dropout_p=p)
    _bwd_compare([qd.grad.cpu(), kd.grad.cpu(), vd.grad.cpu()], want, "autograd with dropout")
