"""Pins of the fp8 oracle (oracle.attention_rows_fp8; CPU only).

The fp8 forward takes e4m3 ("e4m3fn", OCP) inputs with per-head dequantisation factors and is exact
attention over the values they stand for.  What pins what:
- The e4m3 decoding: all 256 codes against torch's float8_e4m3fn conversion (another code base),
  and hand-worked codes (1.0, the largest finite 448, the smallest subnormal 2^-9, the smallest
  normal 2^-6, -0, NaN).
- The whole definition with the factors: torch's CPU scaled_dot_product_attention in float64 on the
  dequantised tensors (each element times its head's factor), with GQA (K/V factors indexed by KV
  head), an additive mask, tail causal and an explicit scale; the LSE against torch.logsumexp.
- A math.fsum brute force on tiny inputs; Q = 0 gives the mean of the dequantised V rows.
``test_fp8_planted_mistakes_are_caught``: the K factor taken at the query head's index, the V factor
dropped, and factors dividing instead of multiplying each fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle

F8 = torch.float8_e4m3fn


def test_e4m3_every_code_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(F8).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(want[fin]))


def test_e4m3_hand_worked_codes():
    assert oracle.e4m3_value(0x38) == 1.0            # exponent 7 = bias, fraction 0
    assert oracle.e4m3_value(0x7E) == 448.0          # 1.75 * 2^8, the largest finite value
    assert oracle.e4m3_value(0x01) == 2.0 ** -9      # smallest subnormal: 1/8 * 2^-6
    assert oracle.e4m3_value(0x08) == 2.0 ** -6      # smallest normal
    assert oracle.e4m3_value(0x3C) == 1.5
    assert oracle.e4m3_value(0xC0) == -2.0
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0 and oracle.e4m3_value(0x80) == 0.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))


def fp8_case(B, Hq, Hkv, Nq, Nkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, Hq, Nq, D, generator=g) * 3).to(F8)
    k = (torch.randn(B, Hkv, Nkv, D, generator=g) * 3).to(F8)
    v = (torch.randn(B, Hkv, Nkv, D, generator=g) * 3).to(F8)
    # distinct factors per (batch, head), not powers of two
    dq = torch.rand(B, Hq, generator=g) * 0.2 + 0.05
    dk = torch.rand(B, Hkv, generator=g) * 0.2 + 0.05
    dv = torch.rand(B, Hkv, generator=g) * 0.2 + 0.05
    return q, k, v, dq, dk, dv


def dequant(x, f):
    return x.to(torch.float64) * f.to(torch.float64)[:, :, None, None]


def pin_sdpa(fault=oracle.FAULT_NONE):
    ok = True
    cases = [(2, 4, 2, 9, 13, 16, False, None, None), (1, 3, 1, 7, 7, 32, True, None, 0.3),
             (2, 2, 2, 5, 11, 8, False, "mask", None)]
    for i, (B, Hq, Hkv, Nq, Nkv, D, causal, m, sc) in enumerate(cases):
        q, k, v, dq, dk, dv = fp8_case(B, Hq, Hkv, Nq, Nkv, D, seed=10 + i)
        mask = torch.randn(B, 1, Nq, Nkv, generator=torch.Generator().manual_seed(i)) if m else None
        G = Hq // Hkv
        Q, K, V = dequant(q, dq), dequant(k, dk), dequant(v, dv)
        Kr, Vr = K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1)
        scale = sc if sc is not None else 1.0 / math.sqrt(D)
        s = (Q @ Kr.transpose(-1, -2)) * scale
        if mask is not None:
            s = s + mask.double()
        am = None
        if causal:
            am = torch.arange(Nkv)[None, :] <= torch.arange(Nq)[:, None] + (Nkv - Nq)
            s = s.masked_fill(~am, -math.inf)
        want_o = torch.nn.functional.scaled_dot_product_attention(
            Q, Kr, Vr, attn_mask=(mask.double() if mask is not None else am), scale=scale).numpy()
        want_l = torch.logsumexp(s, dim=-1).numpy()
        rows = np.arange(B * Hq * Nq)
        O, L = oracle.attention_rows_fp8(q, k, v, rows, dq, dk, dv, mask=mask, scale=sc, is_causal=causal,
                                         fault=fault)
        ok &= bool(np.all(np.abs(O - want_o.reshape(-1, D)) <= 1e-12 * max(1.0, np.abs(want_o).max())))
        ok &= bool(np.all(np.abs(L - want_l.reshape(-1)) <= 1e-12 * max(1.0, np.abs(want_l).max())))
    return ok


def pin_brute(fault=oracle.FAULT_NONE):
    B, Hq, Hkv, Nq, Nkv, D = 1, 2, 1, 3, 5, 4
    q, k, v, dq, dk, dv = fp8_case(B, Hq, Hkv, Nq, Nkv, D, seed=3)
    val = lambda t: [oracle.e4m3_value(int(c)) for c in t.contiguous().view(torch.uint8).reshape(-1)]
    qv = np.array(val(q)).reshape(B, Hq, Nq, D)
    kv = np.array(val(k)).reshape(B, Hkv, Nkv, D)
    vv = np.array(val(v)).reshape(B, Hkv, Nkv, D)
    O, L = oracle.attention_rows_fp8(q, k, v, np.arange(B * Hq * Nq), dq, dk, dv, fault=fault)
    ok = True
    for h in range(Hq):
        fq, fk, fv = float(dq[0, h]), float(dk[0, 0]), float(dv[0, 0])
        for r in range(Nq):
            s = [math.fsum((fq * qv[0, h, r, d]) * (fk * kv[0, 0, j, d]) for d in range(D)) / math.sqrt(D)
                 for j in range(Nkv)]
            m = max(s)
            den = math.fsum(math.exp(x - m) for x in s)
            i = h * Nq + r
            ok &= abs(L[i] - (m + math.log(den))) <= 1e-12
            for d in range(D):
                o = math.fsum(math.exp(s[j] - m) / den * fv * vv[0, 0, j, d] for j in range(Nkv))
                ok &= abs(O[i, d] - o) <= 1e-12
    return bool(ok)


def test_fp8_against_sdpa():
    assert pin_sdpa()


def test_fp8_brute_force():
    assert pin_brute()


def test_fp8_zero_query_gives_mean_of_dequantised_values():
    B, Hq, Hkv, Nq, Nkv, D = 1, 2, 2, 3, 6, 8
    _, k, v, dq, dk, dv = fp8_case(B, Hq, Hkv, Nq, Nkv, D, seed=4)
    q = torch.zeros(B, Hq, Nq, D).to(F8)
    O, L = oracle.attention_rows_fp8(q, k, v, np.arange(B * Hq * Nq), dq, dk, dv)
    Vd = dequant(v, dv).numpy()
    for h in range(Hq):
        for r in range(Nq):
            assert np.allclose(O[h * Nq + r], Vd[0, h].mean(axis=0), atol=1e-13, rtol=0)
    assert np.allclose(L, math.log(Nkv), atol=1e-14, rtol=0)


def test_fp8_without_factors_equals_the_16_bit_oracle():
    """With no factors (and with power-of-two ones) every dequantised value is a bf16 value, so the fp8
    entry must reproduce the bf16 entry on the converted tensors exactly."""
    B, Hq, Hkv, Nq, Nkv, D = 2, 4, 2, 9, 17, 24
    q, k, v, _, _, _ = fp8_case(B, Hq, Hkv, Nq, Nkv, D, seed=5)
    rows = np.arange(B * Hq * Nq)
    O8, L8 = oracle.attention_rows_fp8(q, k, v, rows, is_causal=False)
    O16, L16 = oracle.attention_rows(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), rows)
    assert np.array_equal(O8, O16) and np.array_equal(L8, L16)
    two = lambda n: torch.full((B, n), 0.25)
    O8, L8 = oracle.attention_rows_fp8(q, k, v, rows, two(Hq), two(Hkv), two(Hkv))
    qs, ks, vs = ((t.to(torch.float32) * 0.25).to(torch.bfloat16) for t in (q, k, v))
    O16, L16 = oracle.attention_rows(qs, ks, vs, rows)
    assert np.array_equal(O8, O16) and np.array_equal(L8, L16)


def test_fp8_planted_mistakes_are_caught():
    for fault in (oracle.Q8_FAULT_KSCALE_QHEAD, oracle.Q8_FAULT_NO_VSCALE, oracle.Q8_FAULT_DIVIDE):
        assert not (pin_sdpa(fault) and pin_brute(fault)), fault
