"""Pins for the oracle's packed variable-length form (ffpa-attn "API Reference", ffpa_attn_varlen_func).

Each pin checks the packed result against something other than the per-sequence slicing it is
built from: the dense form over all packed tokens with a block-diagonal mask, torch's CPU
scaled_dot_product_attention in float64 per sequence, brute force with math.fsum, and the closed
forms of sequences with no key or one key.  ``test_planted_varlen_mistakes_are_caught`` switches on
mistakes planted in the packed form and requires each to fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import VarlenWorkload, make_varlen_inputs, sample_tokens, varlen_causal

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _packed(lens_q, lens_k, Hq, Hkv, D, dtype=torch.bfloat16, seed=0):
    w = VarlenWorkload("t", tuple(lens_q), tuple(lens_k), Hq, Hkv, D, dtype=dtype, seed=seed)
    return make_varlen_inputs(w)


def _block_mask(cu_q, cu_k, causal):
    """[Tq, Tk] bool: query token i sees key token j when both belong to sequence b and (causal) the
    key's position in b is at most the query's position + Nkv_b - Nq_b."""
    cq, ck = cu_q.tolist(), cu_k.tolist()
    m = torch.zeros(cq[-1], ck[-1], dtype=torch.bool)
    for b in range(len(cq) - 1):
        nq, nk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        for r in range(nq):
            hi = nk if not causal else min(nk, r + nk - nq + 1)
            if hi > 0:
                m[cq[b] + r, ck[b]:ck[b] + hi] = True
    return m


CASES = [
    # lens_q, lens_k, Hq, Hkv, D, causal
    ((3, 0, 5, 2), (3, 0, 5, 2), 2, 2, 8, False),
    ((3, 0, 5, 2), (3, 0, 5, 2), 2, 2, 8, True),
    ((4, 2, 6), (2, 5, 3), 4, 2, 8, True),       # fewer keys than queries in two sequences
    ((4, 2, 6), (2, 5, 3), 4, 2, 8, False),
    ((1, 7, 3), (6, 0, 9), 2, 1, 16, True),      # MQA, a sequence with no keys
]


def pin_vl_block_diagonal(fault=0):
    """Packed attention equals dense attention over all packed tokens as one sequence, with a mask
    that keeps each token inside its own sequence (and its own causal rule)."""
    ok = True
    for i, (lq, lk, Hq, Hkv, D, causal) in enumerate(CASES):
        q, k, v, cu_q, cu_k = _packed(lq, lk, Hq, Hkv, D, seed=40 + i)
        O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, is_causal=causal, fault=fault)
        mask = _block_mask(cu_q, cu_k, causal)
        Od, Ld = oracle.attention(q.permute(1, 0, 2).unsqueeze(0), k.permute(1, 0, 2).unsqueeze(0),
                                  v.permute(1, 0, 2).unsqueeze(0), mask=mask.view(1, 1, *mask.shape))
        ok &= bool(np.all(np.abs(O - Od[0].transpose(1, 0, 2)) <= 1e-13))
        fin = np.isfinite(Ld[0])
        ok &= bool(np.array_equal(np.isfinite(L), fin)) and bool(np.all(np.abs(L[fin] - Ld[0][fin]) <= 1e-13))
    return ok


def pin_vl_torch_sdpa(fault=0):
    """Per sequence, torch's CPU scaled_dot_product_attention in float64 with an explicit bool mask
    for the tail-aligned causal rule (GQA through enable_gqa); LSE from torch.logsumexp of the masked,
    scaled logits.  Rows that see no key are left to the other pins (SDPA gives NaN there)."""
    ok = True
    for i, (lq, lk, Hq, Hkv, D, causal) in enumerate(CASES):
        q, k, v, cu_q, cu_k = _packed(lq, lk, Hq, Hkv, D, seed=50 + i)
        O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, is_causal=causal, fault=fault)
        cq, ck = cu_q.tolist(), cu_k.tolist()
        for b in range(len(cq) - 1):
            nq, nk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
            if nq == 0 or nk == 0:
                continue
            qs = q[cq[b]:cq[b + 1]].double().permute(1, 0, 2).unsqueeze(0)
            ks = k[ck[b]:ck[b + 1]].double().permute(1, 0, 2).unsqueeze(0)
            vs = v[ck[b]:ck[b + 1]].double().permute(1, 0, 2).unsqueeze(0)
            r = torch.arange(nq).view(nq, 1)
            c = torch.arange(nk).view(1, nk)
            vis = (c <= r + nk - nq) if causal else torch.ones(nq, nk, dtype=torch.bool)
            live = vis.any(dim=1)
            ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=vis, enable_gqa=True)
            kr = ks.repeat_interleave(Hq // Hkv, dim=1)
            logits = (qs @ kr.transpose(-1, -2)) / math.sqrt(D)
            lse = torch.logsumexp(logits.masked_fill(~vis, float("-inf")), dim=-1)[0]   # [Hq, nq]
            got = torch.from_numpy(O[cq[b]:cq[b + 1]]).permute(1, 0, 2)                # [Hq, nq, D]
            ok &= bool((got[:, live] - ref[0][:, live]).abs().max() <= 1e-12)
            gl = torch.from_numpy(L[:, cq[b]:cq[b + 1]])
            ok &= bool((gl[:, live] - lse[:, live]).abs().max() <= 1e-12)
            ok &= bool(torch.all(gl[:, ~live] == float("-inf")))
    return ok


def pin_vl_brute_force(fault=0):
    """math.fsum brute force over the packed layout itself: token t of sequence b, head h."""
    lq, lk, Hq, Hkv, D = (2, 3), (3, 1), 2, 1, 4
    ok = True
    for causal in (False, True):
        q, k, v, cu_q, cu_k = _packed(lq, lk, Hq, Hkv, D, seed=60 + causal)
        O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale=0.7, is_causal=causal, fault=fault)
        qd, kd, vd = q.double().tolist(), k.double().tolist(), v.double().tolist()
        cq, ck = cu_q.tolist(), cu_k.tolist()
        for b in range(len(lq)):
            nq, nk = lq[b], lk[b]
            for r in range(nq):
                t = cq[b] + r
                for h in range(Hq):
                    hk = h // (Hq // Hkv)
                    logits = []
                    for j in range(nk):
                        if causal and j > r + nk - nq:
                            logits.append(-math.inf)
                        else:
                            logits.append(0.7 * math.fsum(qd[t][h][d] * kd[ck[b] + j][hk][d] for d in range(D)))
                    m = max(logits, default=-math.inf)
                    if m == -math.inf:
                        ok &= bool(L[h, t] == -math.inf) and bool(np.all(O[t, h] == 0))
                        continue
                    lse = m + math.log(math.fsum(math.exp(x - m) for x in logits))
                    ok &= abs(L[h, t] - lse) <= 1e-13
                    for d in range(D):
                        want = math.fsum(math.exp(x - lse) * vd[ck[b] + j][hk][d] for j, x in enumerate(logits))
                        ok &= abs(O[t, h, d] - want) <= 1e-13
    return ok


def pin_vl_closed_forms(fault=0):
    """A sequence with no key gives O = 0, LSE = -inf; a sequence with one query and one key gives O = v
    and LSE = scale <q, k>; an empty sequence takes no token."""
    q, k, v, cu_q, cu_k = _packed((2, 1, 0, 3), (0, 1, 0, 4), 2, 2, 8, seed=70)
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale=0.25, fault=fault)
    ok = bool(np.all(O[0:2] == 0)) and bool(np.all(L[:, 0:2] == -math.inf))
    t, kk = 2, 0
    for h in range(2):
        ok &= bool(np.all(O[t, h] == v[kk, h].double().numpy()))
        ok &= abs(L[h, t] - 0.25 * float(torch.dot(q[t, h].double(), k[kk, h].double()))) <= 1e-14
    return ok


VL_PINS = [pin_vl_block_diagonal, pin_vl_torch_sdpa, pin_vl_brute_force, pin_vl_closed_forms]


@pytest.mark.parametrize("pin", VL_PINS, ids=[p.__name__ for p in VL_PINS])
def test_varlen_pin_holds(pin):
    assert pin(0), pin.__doc__


VL_FAULTS = {
    oracle.VL_FAULT_SHARED_OFFSETS: "keys cut with the query offsets",
    oracle.VL_FAULT_TOPLEFT_CAUSAL: "top-left causal rule per sequence",
    oracle.VL_FAULT_LSE_TOKEN_MAJOR: "LSE laid out [Tq, Hq]",
}


@pytest.mark.parametrize("fault", sorted(VL_FAULTS), ids=[VL_FAULTS[f] for f in sorted(VL_FAULTS)])
def test_planted_varlen_mistakes_are_caught(fault):
    failing = [p.__name__ for p in VL_PINS if not p(fault)]
    assert failing, f"no pin catches the planted mistake: {VL_FAULTS[fault]}"


def test_token_subset_matches_full():
    q, k, v, cu_q, cu_k = _packed((5, 9, 1), (7, 9, 3), 4, 2, 16, seed=80)
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, is_causal=True)
    toks = [0, 4, 5, 13, 14]
    Os, Ls = oracle.attention_varlen(q, k, v, cu_q, cu_k, is_causal=True, tokens=toks)
    assert np.array_equal(Os, O[toks]) and np.array_equal(Ls, L[:, toks])


def test_malformed_offsets_are_rejected():
    q, k, v, cu_q, cu_k = _packed((2, 3), (2, 3), 1, 1, 8)
    with pytest.raises(ValueError):
        oracle.attention_varlen(q, k, v, [0, 3, 2], [0, 2, 5])
    with pytest.raises(ValueError):
        oracle.attention_varlen(q, k, v, [1, 2, 5], [0, 2, 5])
    with pytest.raises(ValueError):
        oracle.attention_varlen(q, k, v, [0, 2, 4], [0, 2, 5])


def test_varlen_workload_recipe():
    w = varlen_causal()
    assert len(w.lens_q) == 8 and all(256 <= n <= 8192 for n in w.lens_q) and w.lens_k == w.lens_q
    assert w.flops == sum(2.0 * 16 * n * n * 512 for n in w.lens_q)
    toks = sample_tokens(w.lens_q, seed=w.seed)
    assert toks == sorted(set(toks)) and toks[0] == 0 and toks[-1] == sum(w.lens_q) - 1
