"""Pins of the dropout oracle (CPU only).

What pins what:
- Philox4x32-10 (oracle/philox.py): the known-answer vectors published with the generator's
  definition (Salmon et al., SC 2011, and the Random123 library's test vectors), on both the
  scalar and the array form.
- The keep-bit layout: the fraction of dropped keys against p within a binomial bound, p = 0
  keeping every key, keys past Nkv never kept, rows, words and offsets drawing distinct streams.
- The keep-word decoding (oracle.philox.keep_matrix): against a reader that takes the bits one by
  one, and against a hand-set word (bit 13 of word 1 keeps key 45 alone).  The dropout backward's
  torch reference reads the bits one by one too, so a decoding mistake in the oracle's backward
  fails that pin as well.
- The dropout attention (oracle.attention_dropout_rows): a pure-Python math.fsum evaluation of
  SDPA-style dropout on tiny inputs (bits read one by one from the words); closed forms (every
  key kept gives the plain output over 1 - p; complementary masks add up to the plain output
  times 1 / (1 - p)); a Monte-Carlo check that the expectation over seeds is the plain output
  (inverted dropout is unbiased); and the LSE left untouched.
``test_dropout_planted_mistakes_are_caught`` requires each planted mistake to fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.philox import (KEEP_FAULT_BIT_REVERSED, KEEP_FAULT_NONE, KEEP_FAULT_WORD_SHIFTED, dropout_keep_bits,
                           drop_threshold, keep_matrix, philox4x32_10, philox4x32_10_np)
from workloads import random_qkv

# Published known-answer vectors of Philox4x32 with 10 rounds: (counter, key) -> output.
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    assert philox4x32_10(ctr, key) == want
    out = philox4x32_10_np(*[np.array([c], dtype=np.uint64) for c in ctr], key[0], key[1])
    assert tuple(int(x[0]) for x in out) == want


def test_threshold():
    assert drop_threshold(0.0) == 0
    assert drop_threshold(0.5) == 1 << 31
    assert drop_threshold(0.25) == 1 << 30
    with pytest.raises(ValueError):
        drop_threshold(1.0)
    with pytest.raises(ValueError):
        drop_threshold(-0.1)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_fraction(p):
    B, H, Nq, Nkv = 2, 3, 64, 200
    Z = keep_matrix(dropout_keep_bits(B, H, Nq, Nkv, p, seed=1234), Nkv)
    n = Z.size
    dropped = n - Z.sum()
    sd = math.sqrt(n * p * (1 - p))
    assert abs(dropped - n * p) <= 5 * sd


def test_keep_layout():
    B, H, Nq, Nkv = 1, 2, 5, 70  # three words per row, the last one partial
    kb = dropout_keep_bits(B, H, Nq, Nkv, 0.0, seed=7)
    assert kb.shape == (1, 2, 5, 3) and kb.dtype == np.uint32
    assert np.all(kb[..., :2] == 0xFFFFFFFF) and np.all(kb[..., 2] == (1 << 6) - 1)
    kb = dropout_keep_bits(B, H, Nq, Nkv, 0.3, seed=7)
    assert np.all(kb[..., 2] >> 6 == 0)  # keys past Nkv are never kept
    # bit i of word w is decided by output i % 4 of block (i // 4) of counter (8 w + i // 4, R, 0, offset)
    R, w, i = 3 * 1 + 0, 1, 13  # (b=0, h=0, r=3), key 45
    u = philox4x32_10((8 * w + i // 4, R, 0, 0), (7, 0))[i % 4]
    assert ((int(kb[0, 0, 3, w]) >> i) & 1) == int(u >= drop_threshold(0.3))


def test_streams_differ():
    a = dropout_keep_bits(1, 2, 64, 256, 0.5, seed=99)
    b = dropout_keep_bits(1, 2, 64, 256, 0.5, seed=99, offset=1)
    c = dropout_keep_bits(1, 2, 64, 256, 0.5, seed=100)
    flat = a.reshape(-1, a.shape[-1])
    # no two rows, no two words repeat (128-bit blocks are distinct counters)
    assert len({tuple(r) for r in flat.tolist()}) == flat.shape[0]
    assert len(set(flat.reshape(-1).tolist())) > 0.99 * flat.size
    for other in (b, c):
        agree = 1.0 - np.mean(keep_matrix(a, 256) != keep_matrix(other, 256))
        assert 0.45 < agree < 0.55


def brute_dropout(q, k, v, Z, p, mask=None, is_causal=False):
    """math.fsum evaluation of softmax(scale q.k + bias) with dropout, one weight at a time."""
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd = q.double().tolist(), k.double().tolist(), v.double().tolist()
    pf = float(np.float32(p))
    O = np.zeros((B, Hq, Nq, D))
    L = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for r in range(Nq):
                s = []
                for j in range(Nkv):
                    x = scale * math.fsum(qd[b][h][r][d] * kd[b][hk][j][d] for d in range(D))
                    if mask is not None:
                        x += float(mask[b, 0, r, j])  # [B, 1, Nq, Nkv]: shared by the heads
                    if is_causal and j > r + Nkv - Nq:
                        x = -math.inf
                    s.append(x)
                m = max(s)
                den = math.fsum(math.exp(x - m) for x in s)
                L[b, h, r] = m + math.log(den)
                for d in range(D):
                    O[b, h, r, d] = math.fsum(math.exp(s[j] - m) / den * Z[b][h][r][j] / (1.0 - pf) * vd[b][hk][j][d]
                                              for j in range(Nkv))
    return O, L


def bits_one_by_one(kb, B, Hq, Nq, Nkv):
    """Keep flags read bit by bit from the words (independent of keep_matrix)."""
    return [[[[(int(kb[b, h, r, j // 32]) >> (j % 32)) & 1 for j in range(Nkv)] for r in range(Nq)]
             for h in range(Hq)] for b in range(B)]


def pin_brute(fault=oracle.DROP_FAULT_NONE):
    ok = True
    for (B, Hq, Hkv, Nq, Nkv, D, causal, p, seed) in [(1, 2, 1, 5, 37, 4, False, 0.3, 1), (2, 2, 2, 4, 6, 3, True, 0.5, 2)]:
        q, k, v = random_qkv(B, Hq, Hkv, Nq, Nkv, D, seed=seed)
        kb = dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=seed + 50)
        mask = torch.randn(B, 1, Nq, Nkv, generator=torch.Generator().manual_seed(seed)) if not causal else None
        Ob, Lb = brute_dropout(q, k, v, bits_one_by_one(kb, B, Hq, Nq, Nkv), p, mask=mask, is_causal=causal)
        O, L = oracle.attention_dropout_rows(q, k, v, np.arange(B * Hq * Nq), kb, p, mask=mask, is_causal=causal,
                                             fault=fault)
        ok &= bool(np.all(np.abs(O - Ob.reshape(-1, D)) <= 1e-12))
        ok &= bool(np.all(np.abs(L - Lb.reshape(-1)) <= 1e-12))
    return ok


def pin_closed_forms(fault=oracle.DROP_FAULT_NONE):
    B, Hq, Nq, Nkv, D, p = 1, 2, 9, 45, 16, 0.25
    q, k, v = random_qkv(B, Hq, 1, Nq, Nkv, D, seed=5)
    rows = np.arange(B * Hq * Nq)
    O0, L0 = oracle.attention_rows(q, k, v, rows)
    W = (Nkv + 31) // 32
    ones = np.full((B, Hq, Nq, W), 0xFFFFFFFF, dtype=np.uint32)
    O1, L1 = oracle.attention_dropout_rows(q, k, v, rows, ones, p, fault=fault)
    ok = bool(np.all(np.abs(O1 * (1 - p) - O0) <= 1e-13)) and bool(np.all(np.abs(L1 - L0) <= 1e-13))
    kb = dropout_keep_bits(B, Hq, Nq, Nkv, 0.5, seed=11)
    Oa, La = oracle.attention_dropout_rows(q, k, v, rows, kb, p, fault=fault)
    Ob, _ = oracle.attention_dropout_rows(q, k, v, rows, ~kb, p, fault=fault)
    ok &= bool(np.all(np.abs((Oa + Ob) * (1 - p) - O0) <= 1e-13))
    ok &= bool(np.all(np.abs(La - L0) <= 1e-13))
    return ok


def pin_unbiased(fault=oracle.DROP_FAULT_NONE):
    B, Hq, Nq, Nkv, D, p, n = 1, 1, 4, 64, 8, 0.5, 400
    q, k, v = random_qkv(B, Hq, 1, Nq, Nkv, D, seed=8)
    rows = np.arange(Nq)
    O0, _ = oracle.attention_rows(q, k, v, rows)
    acc = np.zeros_like(O0)
    sq = np.zeros_like(O0)
    for s in range(n):
        O, _ = oracle.attention_dropout_rows(q, k, v, rows, dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=1000 + s), p,
                                             fault=fault)
        acc += O
        sq += O * O
    mean = acc / n
    sem = np.sqrt(np.maximum(sq / n - mean * mean, 0) / n)
    return bool(np.all(np.abs(mean - O0) <= 5 * sem + 1e-12))


def test_dropout_brute_force():
    assert pin_brute()


def test_dropout_closed_forms():
    assert pin_closed_forms()


def test_dropout_unbiased():
    assert pin_unbiased()


def test_dropout_planted_mistakes_are_caught():
    for fault in (oracle.DROP_FAULT_SCALE_BY_KEEP, oracle.DROP_FAULT_BIT_REVERSED, oracle.DROP_FAULT_LSE_DROPPED):
        assert not (pin_brute(fault) and pin_closed_forms(fault) and pin_unbiased(fault)), fault


def _torch_dropout_grads(q, k, v, do, words, p, mask=None, is_causal=False):
    """Autograd in float64 through softmax(scale q.k + bias) * keep / (1 - p) @ V (keep a constant),
    with K/V repeated per group (repeat_interleave) for GQA."""
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qd, kd, vd = (t.double().requires_grad_(True) for t in (q, k, v))
    kr, vr = kd.repeat_interleave(G, dim=1), vd.repeat_interleave(G, dim=1)
    s = (qd @ kr.transpose(-1, -2)) / math.sqrt(D)
    if mask is not None:
        s = s + mask.double()
    if is_causal:
        vis = torch.arange(Nkv).view(1, Nkv) <= torch.arange(Nq).view(Nq, 1) + (Nkv - Nq)
        s = s.masked_fill(~vis, -math.inf)
    # keep flags read bit by bit from the words, not through keep_matrix, which this pins
    Z = torch.tensor(bits_one_by_one(words, B, Hq, Nq, Nkv), dtype=torch.float64)
    o = (torch.softmax(s, dim=-1) * Z / (1.0 - float(np.float32(p)))) @ vr
    return [g.numpy() for g in torch.autograd.grad(o, (qd, kd, vd), do.double())]


def pin_backward_dropout(fault=oracle.BWD_FAULT_NONE):
    ok = True
    g = torch.Generator().manual_seed(31)
    for (B, Hq, Hkv, Nq, Nkv, D, causal, p, seed) in [(1, 2, 2, 5, 40, 8, False, 0.3, 1),
                                                      (2, 4, 2, 4, 9, 8, True, 0.5, 2)]:
        q, k, v = random_qkv(B, Hq, Hkv, Nq, Nkv, D, seed=seed)
        do = torch.randn(B, Hq, Nq, D, generator=g).to(torch.bfloat16)
        words = dropout_keep_bits(B, Hq, Nq, Nkv, p, seed=seed + 3)
        mask = None if causal else torch.randn(B, 1, Nq, Nkv, generator=g)
        want = _torch_dropout_grads(q, k, v, do, words, p, mask=mask, is_causal=causal)
        got = oracle.attention_backward(q, k, v, do, mask=mask, is_causal=causal, fault=fault, keep_bits=words,
                                        dropout_p=p)
        for a, b in zip(got, want):
            ok &= bool(np.all(np.abs(a - b) <= 1e-10 * max(1.0, np.abs(b).max())))
    return ok


def test_backward_dropout_against_autograd():
    assert pin_backward_dropout()


def test_backward_dropout_all_kept_at_zero_p():
    q, k, v = random_qkv(1, 2, 1, 6, 70, 16, seed=4)
    do = torch.randn(1, 2, 6, 16, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    ones = np.full((1, 2, 6, 3), 0xFFFFFFFF, dtype=np.uint32)
    plain = oracle.attention_backward(q, k, v, do)
    drop = oracle.attention_backward(q, k, v, do, keep_bits=ones, dropout_p=0.0)
    for a, b in zip(plain, drop):
        assert np.array_equal(a, b)


def test_backward_dropout_planted_mistakes_are_caught():
    for fault in (oracle.BWD_FAULT_NO_DELTA, oracle.BWD_FAULT_DK_UNSCALED, oracle.BWD_FAULT_GQA_LAST_HEAD,
                  oracle.BWD_FAULT_KEEP_BIT_REVERSED, oracle.BWD_FAULT_KEEP_WORD_SHIFTED):
        assert not pin_backward_dropout(fault), fault


def pin_keep_matrix(fault=KEEP_FAULT_NONE):
    """keep_matrix against the bit-by-bit reader on random words (ragged Nkv, several words per row)
    and on one hand-set word: word 1 = 1 << 13 keeps key 45 and nothing else of keys 32..63."""
    ok = True
    rng = np.random.default_rng(5)
    for shape, Nkv in [((2, 3, 4, 3), 70), ((1, 1, 2, 4), 128), ((1, 2, 3, 1), 9)]:
        words = rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32)
        want = np.array(bits_one_by_one(words, *shape[:3], Nkv), dtype=np.float64)
        ok &= bool(np.array_equal(keep_matrix(words, Nkv, fault=fault), want))
    hand = np.array([[[[0, 1 << 13, 0]]]], dtype=np.uint32)
    z = keep_matrix(hand, 96, fault=fault)[0, 0, 0]
    ok &= bool(z[45] == 1.0 and z[44] == 0.0 and z.sum() == 1.0)
    return ok


def test_keep_matrix_bit_order():
    assert pin_keep_matrix()


def test_keep_matrix_planted_mistakes_are_caught():
    for fault in (KEEP_FAULT_BIT_REVERSED, KEEP_FAULT_WORD_SHIFTED):
        assert not pin_keep_matrix(fault), fault
