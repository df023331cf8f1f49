"""ffpa_bwd_noalloc (the backward entry that allocates nothing) against ffpa_bwd, through the C ABI.

Both run the same kernels on the same inputs, so their gradients must agree bit for bit; two calls
in a row, the second smaller, check that the built-in Delta buffer is rewritten, not reused stale.
"""
import pytest
import torch

import exact_attention_head_amd as ffpa
import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _grads(entry, q, k, v, o, do, lse, is_causal):
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), None,
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nkv, D, float("nan"), is_causal, ffpa.FFPA_BF16)
    if entry == "noalloc":
        st = ffpa.ffpa_bwd_noalloc(*args, stream)
    else:
        nbytes = ffpa.ffpa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        st = ffpa.ffpa_bwd(*args, ws.data_ptr(), nbytes, stream)
    assert st == 0, ffpa.library().ffpa_last_error_detail()
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_workspace_entry(causal):
    for (B, Hq, Hkv, N, D, seed) in [(2, 4, 2, 300, 512, 1), (1, 2, 1, 70, 128, 2)]:
        print(f"[noalloc] B={B} Hq={Hq} Hkv={Hkv} N={N} D={D} causal={causal}", flush=True)
        q, k, v = (t.to(DEV) for t in W.random_qkv(B, Hq, Hkv, N, N, D, seed=seed))
        do = torch.randn(B, Hq, N, D, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16).to(DEV)
        o, lse = ffpa.attn(q, k, v, is_causal=causal, enable_gqa=Hq != Hkv, return_lse=True)
        want = _grads("workspace", q, k, v, o, do, lse, causal)
        got = _grads("noalloc", q, k, v, o, do, lse, causal)
        for g, w in zip(got, want):
            assert torch.equal(g, w)


def test_noalloc_rejects_sizes_beyond_its_buffer():
    q = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    p = q.data_ptr()
    rows = (1 << 22) + 1
    st = ffpa.ffpa_bwd_noalloc(p, p, p, p, p, p, None, p, p, p, 1, 1, 1, rows, 64, 64, float("nan"), 0,
                               ffpa.FFPA_BF16, None)
    assert st == 3  # FFPA_ERR_UNSUPPORTED, before any GPU work
