"""Decode-like requests (few query rows, long KV) and mixed prefill + decode
batches on the GPU.

Requests with at most 32 query rows (qo_len x group) are cut into KV chunks
of at most 2048 keys; the tests cover lengths around the chunk edges, every
GQA group size's decode threshold, both mask settings, and that a decode
request's bits do not depend on the batch around it.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import bf16_to_f64, compare, default_scale
from workloads import make_batch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_prefill_amd as vp
    assert vp.available(), "the gfx950 library did not load or the device is not a gfx950"


def _run(b, causal, **kw):
    import varlen_prefill_amd as vp
    plan = vp.Plan(b.q_indptr, b.kv_indptr, b.num_qo_heads, b.num_kv_heads, b.head_dim, causal, **kw)
    q = b.q.to(DEV)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device=DEV)
    plan.run(q, b.k.to(DEV), b.v.to(DEV), out=o, lse=lse, sm_scale=default_scale(b.head_dim))
    torch.cuda.synchronize()
    info = plan.info
    plan.close()
    return o.cpu(), lse.cpu(), info


def _check(b, causal, o, lse):
    ro, rl = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, b.num_qo_heads,
                                     b.num_kv_heads, causal, default_scale(b.head_dim))
    print(compare(bf16_to_f64(o), lse.double().numpy(), ro, rl))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 1, 128), (4, 4, 128), (16, 4, 256)])
def test_decode_lengths_around_chunk_edges(causal, hq, hkv, d):
    kv = [0, 1, 31, 32, 2047, 2048, 2049, 4096, 4097, 6000]
    b = make_batch([1] * len(kv), kv, hq, hkv, d, seed=900 + hq + d)
    o, lse, info = _run(b, causal)
    _check(b, causal, o, lse)
    assert info["num_merge_items"] == hkv * sum(1 for x in kv if x > 2048)


def test_decode_threshold_by_group():
    """qo_len x group <= 32 rows is decode-like: with g = 4, 8 query tokens split
    at 2048 keys, 9 tokens use the 8192-key chunk."""
    for qo, merges in ((8, 2), (9, 0)):
        b = make_batch([qo], [5000], 8, 2, 128, seed=950 + qo)
        o, lse, info = _run(b, True)
        assert info["num_merge_items"] == merges
        _check(b, True, o, lse)


def test_mixed_batch_and_decode_invariance():
    qo = [700, 1, 1, 300, 1, 0, 1]
    kv = [700, 9000, 3000, 2500, 1, 40, 12000]
    b = make_batch(qo, kv, 32, 8, 128, seed=990)
    o, lse, _ = _run(b, True)
    _check(b, True, o, lse)
    # each decode request alone gives the same bits as inside the batch
    for r in (1, 2, 6):
        one = make_batch([1], [kv[r]], 32, 8, 128, seed=990, request_ids=[r])
        o1, l1, _ = _run(one, True)
        row = int(b.q_indptr[r])
        assert torch.equal(o1[0].view(torch.int16), o[row].view(torch.int16))
        assert torch.equal(l1[0].view(torch.int32), lse[row].view(torch.int32))
