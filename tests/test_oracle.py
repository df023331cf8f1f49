"""Pins for the fp64 oracle: checks against facts the pages and mathematics fix.

None of these re-types the oracle's own loop.  Each pin is a closed form, an
invariant, a special case that reduces to a library routine (torch's CPU
scaled_dot_product_attention in float64), or brute force with math.fsum on
tiny inputs.  ``test_planted_mistakes_are_caught`` switches on mistakes
planted inside the C oracle and requires every one of them to fail at least
one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import random_qkv

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _rows(B, H, N):
    return np.arange(B * H * N)


def _full(q, k, v, fault=0, **kw):
    return oracle.attention(q, k, v, fault=fault, **kw)


# ---------------------------------------------------------------------------------------------
# Pins, written as predicates so that the planted-mistake test can run them on a wrong oracle.
# ---------------------------------------------------------------------------------------------

def pin_probs_sum_to_one(fault=0):
    """Every row of P sums to 1 (softmax normalisation), with masks and causal."""
    q, k, v = random_qkv(2, 4, 2, 5, 7, 8, seed=11)
    g = torch.Generator().manual_seed(12)
    add = torch.randn(2, 1, 5, 7, generator=g)
    add[torch.rand(2, 1, 5, 7, generator=g) < 0.3] = float("-inf")
    add[..., 0] = 0.0
    ok = True
    for kw in (dict(), dict(mask=add), dict(mask=add > -1.0), dict(is_causal=True)):
        _, L, P = oracle.attention_rows(q, k, v, _rows(2, 4, 5), want_probs=True, fault=fault, **kw)
        live = np.isfinite(L)
        ok &= bool(np.all(np.abs(P[live].sum(axis=1) - 1.0) <= 1e-14))
    return ok


def pin_identical_v_rows(fault=0):
    """If every V row of a head is the same vector u, every output row of that head is u."""
    q, k, _ = random_qkv(1, 2, 2, 4, 6, 8, seed=13)
    u = torch.randn(1, 2, 1, 8, generator=torch.Generator().manual_seed(14)).to(torch.bfloat16)
    v = u.expand(1, 2, 6, 8).contiguous()
    O, _ = _full(q, k, v, fault=fault)
    want = u.double().numpy()
    return bool(np.all(np.abs(O - want) <= 1e-14 * np.maximum(1.0, np.abs(want))))


def pin_zero_query_uniform(fault=0):
    """Q = 0: the softmax is uniform over the visible keys, so O is their mean and LSE = ln(count).
    Causal with Nq < Nkv: row r sees keys 0..r+(Nkv-Nq)."""
    _, k, v = random_qkv(1, 1, 1, 3, 5, 8, seed=15)
    q = torch.zeros(1, 1, 3, 8, dtype=torch.bfloat16)
    ok = True
    vv = v.double().numpy()[0, 0]
    for causal in (False, True):
        O, L = _full(q, k, v, fault=fault, is_causal=causal)
        for r in range(3):
            n = r + 3 if causal else 5
            mean = np.array([math.fsum(vv[:n, d]) / n for d in range(8)])
            ok &= bool(np.all(np.abs(O[0, 0, r] - mean) <= 1e-14))
            ok &= abs(L[0, 0, r] - math.log(n)) <= 1e-14
    return ok


def pin_weighted_by_mask(fault=0):
    """Q = 0 with additive bias ln(w_k): the softmax weights are w_k / sum(w), an exact rational
    mixture; LSE = ln(sum w).  The bias enters after scaling, so a scale != 1 must not touch it."""
    D = 16
    _, k, v = random_qkv(1, 1, 1, 1, 4, D, seed=16)
    q = torch.zeros(1, 1, 1, D, dtype=torch.bfloat16)
    w = [1.0, 2.0, 3.0, 4.0]
    bias = torch.tensor([math.log(x) for x in w], dtype=torch.float32).view(1, 1, 1, 4)
    wf = [math.exp(float(b)) for b in bias.view(-1)]  # the fp32-rounded weights actually passed
    O, L = _full(q, k, v, fault=fault, mask=bias, scale=0.25)
    vv = v.double().numpy()[0, 0]
    want = np.array([math.fsum(wf[j] * vv[j, d] for j in range(4)) / math.fsum(wf) for d in range(D)])
    return bool(np.all(np.abs(O[0, 0, 0] - want) <= 1e-13)) and abs(L[0, 0, 0] - math.log(math.fsum(wf))) <= 1e-13


def pin_causal_locality(fault=0):
    """Tail-aligned causal: row r depends only on keys k <= r + (Nkv - Nq).  Changing K and V beyond
    that leaves row r bit-identical; and with Nq = Nkv row 0 sees only key 0, so O = v_0, LSE = s_0."""
    Nq, Nkv, D = 4, 7, 8
    q, k, v = random_qkv(1, 2, 1, Nq, Nkv, D, seed=17)
    O, L = _full(q, k, v, fault=fault, is_causal=True)
    ok = True
    for r in range(Nq):
        last = r + Nkv - Nq
        k2, v2 = k.clone(), v.clone()
        k2[:, :, last + 1:] = torch.randn(k2[:, :, last + 1:].shape).to(k.dtype)
        v2[:, :, last + 1:] = torch.randn(v2[:, :, last + 1:].shape).to(v.dtype)
        O2, L2 = _full(q, k2, v2, fault=fault, is_causal=True)
        ok &= bool(np.array_equal(O[:, :, r], O2[:, :, r])) and bool(np.array_equal(L[:, :, r], L2[:, :, r]))
        # and the keys it may see do matter (guards against a rule that hides too much)
        if last >= 1:
            v3 = v.clone()
            v3[:, :, last] += 1.0
            O3, _ = _full(q, k, v3, fault=fault, is_causal=True)
            ok &= not np.array_equal(O[:, :, r], O3[:, :, r])
    q, k, v = random_qkv(1, 1, 1, 3, 3, D, seed=18)
    O, L = _full(q, k, v, fault=fault, is_causal=True)
    s0 = math.fsum(float(a) * float(b) for a, b in zip(q[0, 0, 0].double(), k[0, 0, 0].double())) / math.sqrt(D)
    ok &= bool(np.array_equal(O[0, 0, 0], v[0, 0, 0].double().numpy()))
    ok &= abs(L[0, 0, 0] - s0) <= 1e-14 * max(1.0, abs(s0))
    return ok


def pin_gqa_is_repeat(fault=0):
    """GQA: Hq = G*Hkv gives exactly what K/V repeated G times per head (repeat_interleave) gives."""
    q, k, v = random_qkv(2, 6, 2, 5, 9, 8, seed=19)
    O, L = _full(q, k, v, fault=fault)
    O2, L2 = _full(q, k.repeat_interleave(3, dim=1), v.repeat_interleave(3, dim=1), fault=fault)
    return bool(np.array_equal(O, O2)) and bool(np.array_equal(L, L2))


def pin_scale(fault=0):
    """scale=None is 1/sqrt(D); and scale multiplies Q K^T: scale 0.5 on Q equals scale 1 on 0.5*Q
    (a power of two, so the bf16 inputs stay exact)."""
    q, k, v = random_qkv(1, 2, 2, 4, 6, 16, seed=20)
    O1, L1 = _full(q, k, v, fault=fault)
    O2, L2 = _full(q, k, v, fault=fault, scale=1.0 / math.sqrt(16))
    O3, L3 = _full(q, k, v, fault=fault, scale=0.5)
    O4, L4 = _full((q.float() * 0.5).to(q.dtype), k, v, fault=fault, scale=1.0)
    return (bool(np.array_equal(O1, O2)) and bool(np.array_equal(L1, L2)) and bool(np.array_equal(O3, O4))
            and bool(np.array_equal(L3, L4)))


def pin_mask_algebra(fault=0):
    """A bool mask equals the additive 0/-inf mask; adding c to a whole mask row leaves O alone and
    shifts LSE by c; permuting keys jointly in K, V and the mask leaves O and LSE alone."""
    B, H, Nq, Nkv, D = 1, 2, 3, 6, 8
    q, k, v = random_qkv(B, H, H, Nq, Nkv, D, seed=21)
    g = torch.Generator().manual_seed(22)
    keep = torch.rand(B, H, Nq, Nkv, generator=g) < 0.6
    keep[..., 2] = True
    add = torch.where(keep, torch.zeros(()), torch.full((), float("-inf")))
    Ob, Lb = _full(q, k, v, fault=fault, mask=keep)
    Oa, La = _full(q, k, v, fault=fault, mask=add)
    ok = bool(np.array_equal(Ob, Oa)) and bool(np.array_equal(Lb, La))
    # bias on a 2^-10 grid so that bias + c is exact in fp32
    bias = torch.round(torch.randn(B, H, Nq, Nkv, generator=g) * 1024.0) / 1024.0
    c = torch.tensor([0.5, -1.25, 2.0]).view(1, 1, Nq, 1)
    O1, L1 = _full(q, k, v, fault=fault, mask=bias)
    O2, L2 = _full(q, k, v, fault=fault, mask=bias + c)
    ok &= bool(np.all(np.abs(O1 - O2) <= 1e-13))
    ok &= bool(np.all(np.abs((L2 - L1) - c.view(1, 1, Nq).double().numpy()) <= 1e-13))
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    O3, L3 = _full(q, k[:, :, perm], v[:, :, perm], fault=fault, mask=bias[..., perm])
    ok &= bool(np.all(np.abs(O1 - O3) <= 1e-13)) and bool(np.all(np.abs(L1 - L3) <= 1e-13))
    return ok


def pin_mask_with_causal(fault=0):
    """A mask together with the causal rule equals that mask combined by hand with the tail-aligned
    causal mask (bool: AND; additive: -inf where the causal rule excludes), Nq < Nkv."""
    B, H, Nq, Nkv, D = 2, 2, 4, 7, 8
    q, k, v = random_qkv(B, H, H, Nq, Nkv, D, seed=71)
    g = torch.Generator().manual_seed(72)
    vis = torch.arange(Nkv).view(1, Nkv) <= torch.arange(Nq).view(Nq, 1) + (Nkv - Nq)
    keep = torch.rand(B, 1, Nq, Nkv, generator=g) < 0.7
    keep[..., 0] = True
    bias = torch.randn(B, 1, Nq, Nkv, generator=g)
    ok = True
    O1, L1 = _full(q, k, v, fault=fault, mask=keep, is_causal=True)
    O2, L2 = _full(q, k, v, fault=fault, mask=keep & vis)
    ok &= bool(np.array_equal(O1, O2)) and bool(np.array_equal(L1, L2))
    O1, L1 = _full(q, k, v, fault=fault, mask=bias, is_causal=True)
    O2, L2 = _full(q, k, v, fault=fault, mask=bias.masked_fill(~vis, float("-inf")))
    ok &= bool(np.array_equal(O1, O2)) and bool(np.array_equal(L1, L2))
    return ok


def pin_one_and_two_keys(fault=0):
    """Nkv = 1: O = v_0, LSE = s_0.  Nkv = 2: O = sigmoid(s0-s1) v0 + sigmoid(s1-s0) v1 and
    LSE = s0 + log(1 + exp(s1 - s0))."""
    D = 8
    ok = True
    q, k, v = random_qkv(1, 1, 1, 2, 1, D, seed=23)
    O, L = _full(q, k, v, fault=fault)
    for r in range(2):
        s0 = math.fsum(float(a) * float(b) for a, b in zip(q[0, 0, r].double(), k[0, 0, 0].double())) / math.sqrt(D)
        ok &= bool(np.array_equal(O[0, 0, r], v[0, 0, 0].double().numpy()))
        ok &= abs(L[0, 0, r] - s0) <= 1e-14 * max(1.0, abs(s0))
    q, k, v = random_qkv(1, 1, 1, 3, 2, D, seed=24)
    O, L = _full(q, k, v, fault=fault)
    for r in range(3):
        s = [math.fsum(float(a) * float(b) for a, b in zip(q[0, 0, r].double(), k[0, 0, j].double())) / math.sqrt(D)
             for j in range(2)]
        w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        w1 = 1.0 / (1.0 + math.exp(s[0] - s[1]))
        want = w0 * v[0, 0, 0].double().numpy() + w1 * v[0, 0, 1].double().numpy()
        ok &= bool(np.all(np.abs(O[0, 0, r] - want) <= 1e-14))
        ok &= abs(L[0, 0, r] - (s[0] + math.log1p(math.exp(s[1] - s[0])))) <= 1e-14
    return ok


def _sdpa64(q, k, v, mask=None, is_causal=False, enable_gqa=False):
    import torch.nn.functional as F

    return F.scaled_dot_product_attention(q.double(), k.double(), v.double(), attn_mask=mask, is_causal=is_causal,
                                          enable_gqa=enable_gqa).numpy()


def pin_torch_sdpa(fault=0):
    """Whole definition against torch's CPU scaled_dot_product_attention in float64 (another code
    base): no mask, bool mask, float mask, causal with Nq = Nkv, GQA via enable_gqa, and tail-aligned
    causal with Nq < Nkv passed to SDPA as an explicit boolean mask."""
    ok = True
    q, k, v = random_qkv(2, 4, 4, 9, 9, 16, seed=25)
    ok &= np.allclose(_full(q, k, v, fault=fault)[0], _sdpa64(q, k, v), atol=1e-12, rtol=0)
    g = torch.Generator().manual_seed(26)
    keep = torch.rand(2, 1, 9, 9, generator=g) < 0.7
    keep[..., 0] = True
    ok &= np.allclose(_full(q, k, v, fault=fault, mask=keep)[0], _sdpa64(q, k, v, mask=keep), atol=1e-12, rtol=0)
    bias = torch.randn(2, 4, 9, 9, generator=g, dtype=torch.float64)
    ok &= np.allclose(_full(q, k, v, fault=fault, mask=bias.float())[0], _sdpa64(q, k, v, mask=bias.float().double()),
                      atol=1e-12, rtol=0)
    ok &= np.allclose(_full(q, k, v, fault=fault, is_causal=True)[0], _sdpa64(q, k, v, is_causal=True), atol=1e-12,
                      rtol=0)
    q, k, v = random_qkv(1, 8, 2, 6, 10, 16, seed=27)
    ok &= np.allclose(_full(q, k, v, fault=fault)[0], _sdpa64(q, k, v, enable_gqa=True), atol=1e-12, rtol=0)
    tail = torch.ones(6, 10, dtype=torch.bool).tril(diagonal=10 - 6)
    ok &= np.allclose(_full(q, k, v, fault=fault, is_causal=True)[0], _sdpa64(q, k, v, mask=tail, enable_gqa=True),
                      atol=1e-12, rtol=0)
    return bool(ok)


def _brute(q, k, v, mask=None, is_causal=False, scale=None):
    """Pure-Python fsum evaluation of the definition on tiny inputs."""
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    qd, kd, vd = q.double().tolist(), k.double().tolist(), v.double().tolist()
    if mask is not None:
        mm = mask.expand(B, Hq, Nq, Nkv)
        md = mm.tolist()
    O = np.zeros((B, Hq, Nq, D))
    L = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for r in range(Nq):
                logits = []
                for j in range(Nkv):
                    if is_causal and j > r + Nkv - Nq:
                        logits.append(-math.inf)
                        continue
                    s = scale * math.fsum(qd[b][h][r][d] * kd[b][hk][j][d] for d in range(D))
                    if mask is not None:
                        mv = md[b][h][r][j]
                        s = (s if mv else -math.inf) if isinstance(mv, bool) else s + mv
                    logits.append(s)
                m = max(logits)
                if m == -math.inf:
                    L[b, h, r] = -math.inf
                    continue
                lse = m + math.log(math.fsum(math.exp(x - m) for x in logits))
                L[b, h, r] = lse
                for d in range(D):
                    O[b, h, r, d] = math.fsum(math.exp(x - lse) * vd[b][hk][j][d] for j, x in enumerate(logits))
    return O, L


def pin_brute_force(fault=0):
    """Brute force with math.fsum on tiny inputs: plain, causal with Nq < Nkv, GQA, both mask kinds, fp16."""
    ok = True
    g = torch.Generator().manual_seed(28)
    cases = [
        (random_qkv(1, 2, 2, 3, 5, 4, seed=29), dict()),
        (random_qkv(2, 2, 1, 3, 6, 8, seed=30), dict(is_causal=True)),
        (random_qkv(1, 4, 2, 4, 4, 4, seed=31), dict(mask=torch.rand(1, 4, 4, 4, generator=g) < 0.7)),
        (random_qkv(2, 2, 2, 2, 5, 6, seed=32), dict(mask=torch.randn(2, 1, 2, 5, generator=g))),
        (random_qkv(1, 2, 2, 4, 4, 8, dtype=torch.float16, seed=33), dict(is_causal=True, scale=0.3)),
    ]
    for (q, k, v), kw in cases:
        Ob, Lb = _brute(q, k, v, **kw)
        Oo, Lo = _full(q, k, v, fault=fault, **kw)
        ok &= bool(np.all(np.abs(Ob - Oo) <= 1e-13)) and bool(np.all(np.abs(Lb - Lo) <= 1e-13))
    return ok


PINS = [pin_probs_sum_to_one, pin_identical_v_rows, pin_zero_query_uniform, pin_weighted_by_mask,
        pin_causal_locality, pin_gqa_is_repeat, pin_scale, pin_mask_algebra, pin_mask_with_causal,
        pin_one_and_two_keys, pin_torch_sdpa, pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_holds(pin):
    assert pin(0), pin.__doc__


FAULTS = {
    oracle.FAULT_TOPLEFT_CAUSAL: "top-left instead of tail-aligned causal",
    oracle.FAULT_HEAD_MODULO: "kv head h % Hkv instead of h // group",
    oracle.FAULT_MASK_BEFORE_SCALE: "bias added before scaling",
    oracle.FAULT_LSE_LOG2: "LSE in base 2",
    oracle.FAULT_DROP_LAST_KEY: "last key dropped from the sums",
    oracle.FAULT_V_TRANSPOSED: "V read transposed",
}


@pytest.mark.parametrize("fault", sorted(FAULTS), ids=[FAULTS[f] for f in sorted(FAULTS)])
def test_planted_mistakes_are_caught(fault):
    failing = [p.__name__ for p in PINS if not p(fault)]
    assert failing, f"no pin catches the planted mistake: {FAULTS[fault]}"


# ---------------------------------------------------------------------------------------------
# Exact widening of the 16-bit inputs and the conventions the pages leave open.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_widening_is_exact(dtype):
    """With one key, O = v_0 exactly, so O exposes the oracle's widening of every finite 16-bit value;
    torch's own conversion to float64 is the reference."""
    bits = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(dtype)
    finite = bits[torch.isfinite(bits.float())]
    D = finite.numel()
    v = finite.view(1, 1, 1, D)
    q = torch.zeros(1, 1, 1, D, dtype=dtype)
    O, L = oracle.attention(q, v.clone(), v)
    assert np.array_equal(O.reshape(-1), finite.double().numpy())
    assert L[0, 0, 0] == 0.0


def test_fully_masked_row_convention():
    """A row whose keys are all excluded has no softmax; the convention is O = 0 and LSE = -inf."""
    q, k, v = random_qkv(1, 1, 1, 3, 4, 8, seed=34)
    keep = torch.ones(1, 1, 3, 4, dtype=torch.bool)
    keep[0, 0, 1] = False
    O, L = oracle.attention(q, k, v, mask=keep)
    assert np.all(O[0, 0, 1] == 0.0) and L[0, 0, 1] == -math.inf
    assert np.all(np.isfinite(O)) and np.isfinite(L[0, 0, 0]) and np.isfinite(L[0, 0, 2])


def test_mask_broadcast_strides():
    """A mask given as [Nq, Nkv], [B, 1, Nq, Nkv] or full [B, Hq, Nq, Nkv] gives the same result."""
    q, k, v = random_qkv(2, 3, 3, 4, 5, 8, seed=35)
    bias = torch.randn(4, 5, generator=torch.Generator().manual_seed(36))
    O1, L1 = oracle.attention(q, k, v, mask=bias)
    O2, L2 = oracle.attention(q, k, v, mask=bias.view(1, 1, 4, 5).expand(2, 1, 4, 5).contiguous())
    O3, L3 = oracle.attention(q, k, v, mask=bias.expand(2, 3, 4, 5).contiguous())
    assert np.array_equal(O1, O2) and np.array_equal(O1, O3)
    assert np.array_equal(L1, L2) and np.array_equal(L1, L3)


def test_row_subset_matches_full():
    """attention_rows on a subset returns exactly the full computation's rows (rows are independent)."""
    q, k, v = random_qkv(2, 2, 1, 6, 7, 8, seed=37)
    O, L = oracle.attention(q, k, v, is_causal=True)
    rows = [0, 5, 7, 13, 23]
    Os, Ls = oracle.attention_rows(q, k, v, rows, is_causal=True)
    assert np.array_equal(Os, O.reshape(-1, 8)[rows]) and np.array_equal(Ls, L.reshape(-1)[rows])


def test_causal_visible_counts():
    assert [oracle.causal_visible(r, 3, 5) for r in range(3)] == [3, 4, 5]
    assert [oracle.causal_visible(r, 4, 4) for r in range(4)] == [1, 2, 3, 4]
