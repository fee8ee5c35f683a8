"""FP8 (OCP E4M3) K/V on the GPU (rp_run_fp8kv, rp_run_paged_fp8kv), head_dim 128 and 256.

Parity against the fp64 FP8 oracle (dequantised K/V, attention by its
definition) with the standard gates; with unit scales the FP8 path must give
the same bits as rp_run on the decoded values stored as bf16 (E4M3 values are
bf16 values and the kernel converts exactly); the paged FP8 path must give
the same bits as the contiguous one.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import bf16_to_f64, compare, default_scale
from workloads import make_batch, make_fp8_kv, make_paged

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_prefill_amd as vp
    assert vp.available(), "the gfx950 library did not load or the device is not a gfx950"


def _plan(b, causal, **kw):
    import varlen_prefill_amd as vp
    return vp.Plan(b.q_indptr, b.kv_indptr, b.num_qo_heads, b.num_kv_heads, b.head_dim, causal, **kw)


def _outs(b):
    q = b.q.to(DEV)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device=DEV)
    return q, o, lse


CASES = [
    # qo, kv, Hq, Hkv, causal, k_scale, v_scale, kv_chunk
    ([1, 130, 257, 64], [1, 130, 257, 64], 32, 8, True, 0.5, 1.25, 0),
    ([33, 129, 7], [500, 129, 2], 16, 2, True, 1.0, 1.0, 0),
    ([100, 3, 0], [0, 3, 5], 4, 2, True, 2.0, 0.25, 0),
    ([40, 200], [90, 200], 8, 1, False, 0.125, 3.0, 0),
    ([50, 300, 9], [700, 300, 1000], 8, 2, True, 0.75, 0.5, 128),   # split KV
    ([1, 1, 1], [3000, 45, 2100], 32, 8, True, 0.5, 0.5, 0),        # decode
]


# head_dim 256 runs the cases whose oracle stays quick at twice the width
CASES_256 = [0, 2, 3, 4]


@pytest.mark.parametrize("d,case", [(128, c) for c in range(len(CASES))] + [(256, c) for c in CASES_256])
def test_fp8_parity(d, case):
    qo, kv, hq, hkv, causal, ks, vs, chunk = CASES[case]
    b = make_batch(qo, kv, hq, hkv, d, seed=5000 + case + d, q_base=2)
    k8, v8 = make_fp8_kv(b, ks, vs)
    sm = default_scale(d)
    plan = _plan(b, causal, kv_chunk=chunk)
    q, o, lse = _outs(b)
    plan.run_fp8kv(q, k8.to(DEV), v8.to(DEV), ks, vs, out=o, lse=lse, sm_scale=sm)
    torch.cuda.synchronize()
    plan.close()
    ro, rl = oracle.fp8_kv_attention(b.q, k8.numpy(), v8.numpy(), ks, vs, b.q_indptr, b.kv_indptr,
                                     hq, hkv, causal, sm)
    rows = slice(2, None)
    print(compare(bf16_to_f64(o.cpu())[rows], lse.double().cpu().numpy()[rows], ro[rows], rl[rows]))
    assert torch.isnan(o[:2]).all() and torch.isnan(lse[:2]).all()


@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (256, True), (256, False)])
def test_fp8_unit_scales_equal_bf16_kernel_bitwise(d, causal):
    b = make_batch([1, 130, 257, 64, 40], [1, 300, 257, 64, 900], 32, 8, d, seed=5100 + d)
    k8, v8 = make_fp8_kv(b, 1.0, 1.0)
    kb = k8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    vb = v8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    sm = default_scale(d)
    plan = _plan(b, causal, kv_chunk=256)
    q, o, lse = _outs(b)
    plan.run_fp8kv(q, k8.to(DEV), v8.to(DEV), 1.0, 1.0, out=o, lse=lse, sm_scale=sm)
    ob, lb = plan.run(q, kb.to(DEV), vb.to(DEV), sm_scale=sm)
    torch.cuda.synchronize()
    plan.close()
    assert torch.equal(o.view(torch.int16), ob.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lb.view(torch.int32))


@pytest.mark.parametrize("d,page_size", [(128, 16), (128, 64), (256, 16)])
def test_fp8_paged_equals_contiguous_bitwise(d, page_size):
    b = make_batch([33, 129, 7, 1], [500, 129, 2, 2000], 16, 2, d, seed=5200 + page_size + d)
    k8, v8 = make_fp8_kv(b, 0.5, 2.0)
    pk = make_paged(b, page_size, seed=5200 + page_size, k=k8, v=v8)
    sm = default_scale(d)
    plan = _plan(b, True)
    q, o, lse = _outs(b)
    plan.run_paged_fp8kv(q, pk.k_pages.to(DEV), pk.v_pages.to(DEV),
                         torch.from_numpy(pk.block_table).to(DEV), 0.5, 2.0, out=o, lse=lse,
                         sm_scale=sm)
    oc, lc = plan.run_fp8kv(q, k8.to(DEV), v8.to(DEV), 0.5, 2.0, sm_scale=sm)
    torch.cuda.synchronize()
    plan.close()
    assert torch.equal(o.view(torch.int16), oc.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lc.view(torch.int32))


def test_fp8_argument_errors():
    import varlen_prefill_amd as vp
    b = make_batch([20], [40], 4, 2, 256, seed=5300)
    plan = _plan(b, True)
    q = b.q.to(DEV)
    k8 = torch.zeros(40, 2, 128, dtype=torch.uint8, device=DEV)   # head_dim of another plan
    with pytest.raises(ValueError, match="256"):
        plan.run_fp8kv(q, k8, k8, 1.0, 1.0)
    plan.close()
    b = make_batch([20], [40], 4, 2, 128, seed=5301)
    plan = _plan(b, True)
    q = b.q.to(DEV)
    k8 = torch.zeros(40, 2, 128, dtype=torch.uint8, device=DEV)
    with pytest.raises(vp.RaggedPrefillError, match="finite"):
        plan.run_fp8kv(q, k8, k8, float("inf"), 1.0)
    plan.close()
