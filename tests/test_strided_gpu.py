"""Parity of the strided (zero-copy) layouts with the fp64 oracle, on the GPU.

The binding hands non-contiguous views straight to ffpa_fwd_strided.  The cases cover [B, N, H, D]
storage seen as [B, H, N, D], heads sliced out of a fused projection, K/V broadcast over the batch,
and a strided output.  Each is checked element by element against the oracle on the same logical
tensors, and each view is checked to reach the kernels without a copy.
"""
import json

import pytest
import torch

import exact_attention_head_amd as ffpa
import workloads as W
from gpu_helpers import compare

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _log(name, m):
    print(f"[strided] {name}: {json.dumps(m)}", flush=True)


def _run(q, k, v, **kw):
    o, lse = ffpa.attn(q, k, v, enable_gqa=q.shape[1] != k.shape[1], return_lse=True, **kw)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [64, 256, 512, 576, 1024])
def test_nhd_views(D, causal):
    """[B, N, H, D] storage, transposed views: GQA, ragged lengths."""
    B, Hq, Hkv, Nq, Nkv = 2, 4, 2, 130, 200
    q, k, v = W.random_qkv(B, Hq, Hkv, Nq, Nkv, D, seed=D + causal)
    qn = q.transpose(1, 2).contiguous().to(DEV)   # [B, N, H, D]
    kn = k.transpose(1, 2).contiguous().to(DEV)
    vn = v.transpose(1, 2).contiguous().to(DEV)
    qv, kv_, vv = qn.transpose(1, 2), kn.transpose(1, 2), vn.transpose(1, 2)
    assert not qv.is_contiguous() and ffpa._strides3(qv) is not None
    o, lse = _run(qv, kv_, vv, is_causal=causal)
    _log(f"NHD D={D} causal={causal}", compare(o.cpu(), lse.cpu(), q, k, v, is_causal=causal))


@pytest.mark.parametrize("D", [128, 512, 1024])
def test_fused_projection_slices_and_mask(D):
    """Q, K, V as slices of one [B, N, 3, H, D] tensor (different bases, shared strides), with a bool
    mask, and a strided output laid out [B, N, H, D]."""
    B, H, N = 2, 2, 150
    g = torch.Generator().manual_seed(D)
    qkv = torch.randn(B, N, 3, H, D, generator=g).to(torch.bfloat16)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))   # logical [B, H, N, D]
    mask = torch.rand(B, 1, N, N, generator=g) < 0.8
    mask[..., 0] = True
    qkv_d = qkv.to(DEV)
    qd, kd, vd = (qkv_d[:, :, i].transpose(1, 2) for i in range(3))
    out_store = torch.empty(B, N, H, D, dtype=torch.bfloat16, device=DEV)
    out = out_store.transpose(1, 2)
    o, lse = _run(qd, kd, vd, attn_mask=mask.to(DEV), out=out)
    assert o.data_ptr() == out_store.data_ptr()
    _log(f"fused slices D={D}", compare(out.cpu(), lse.cpu(), q.contiguous(), k.contiguous(), v.contiguous(),
                                       mask=mask))


def test_kv_broadcast_over_batch():
    """K/V expanded over the batch (batch stride 0) with MQA; a K/V expanded along N (row stride 0)
    cannot be read in place and is copied by the binding."""
    B, Hq, N, D = 3, 4, 100, 512
    q, k1, v1 = W.random_qkv(B, Hq, 1, N, 90, D, seed=5)
    k1, v1 = k1[:1], v1[:1]
    kd, vd = k1.to(DEV).expand(B, -1, -1, -1), v1.to(DEV).expand(B, -1, -1, -1)
    assert ffpa._strides3(kd) == [0, 0, D]
    assert ffpa._strides3(kd[:, :, :1].expand(B, 1, 90, D)) is None
    o, lse = _run(q.to(DEV), kd, vd)
    _log("K/V broadcast over batch", compare(o.cpu(), lse.cpu(), q, k1.expand(B, -1, -1, -1).contiguous(),
                                            v1.expand(B, -1, -1, -1).contiguous()))


def test_strided_matches_contiguous():
    """The same logical problem through the contiguous and the strided entries: the runtime-layout
    variant meets the oracle and agrees with the contiguous result to the same bar."""
    B, H, N, D = 1, 4, 256, 512
    q, k, v = W.random_qkv(B, H, H, N, N, D, seed=9)
    oc, lc = _run(q.to(DEV), k.to(DEV), v.to(DEV))
    qn, kn, vn = (t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, k, v))
    os_, ls = _run(qn, kn, vn)
    assert (oc.float() - os_.float()).abs().max() <= 2e-2 and (lc - ls).abs().max() <= 1e-3
    _log("strided vs contiguous", compare(os_.cpu(), ls.cpu(), q, k, v))
