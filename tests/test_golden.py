"""Hand-worked examples (tests/golden/*.json) against the oracle.

Each fixture holds tiny exact inputs and the expected O and LSE as closed-form
expressions; see tests/golden/README.md for the passage each one exercises.
"""
import glob
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json")))
_MATH = {"exp": math.exp, "log": math.log, "sqrt": math.sqrt, "__builtins__": {}}


def closed_form(expr) -> float:
    if isinstance(expr, (int, float)):
        return float(expr)
    return float(eval(expr, dict(_MATH), {}))  # fixture text is ours: numbers, + - * / and exp/log/sqrt


def load_fixture(path, dtype):
    with open(path) as f:
        fx = json.load(f)
    t = lambda key: torch.tensor(fx[key], dtype=torch.float64).to(dtype)
    mask = None
    if fx.get("mask"):
        m = fx["mask"]
        mask = torch.tensor(m["value"], dtype=torch.bool if m["dtype"] == "bool" else torch.float32)
    O = np.vectorize(closed_form, otypes=[float])(np.array(fx["O"], dtype=object))
    L = np.vectorize(closed_form, otypes=[float])(np.array(fx["LSE"], dtype=object))
    return fx, t("q"), t("k"), t("v"), mask, O, L


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_golden_oracle(path, dtype):
    fx, q, k, v, mask, O_want, L_want = load_fixture(path, dtype)
    O, L = oracle.attention(q, k, v, mask=mask, scale=fx["scale"], is_causal=fx["is_causal"])
    assert O.shape == O_want.shape and L.shape == L_want.shape
    assert np.allclose(O, O_want, rtol=0, atol=1e-14), (O, O_want)
    assert np.allclose(L, L_want, rtol=0, atol=1e-14), (L, L_want)
