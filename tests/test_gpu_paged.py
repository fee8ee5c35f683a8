"""Paged-KV append prefill (rp_run_paged) on the GPU.

The K/V of each case are scattered into a page pool by ``workloads.make_paged``
(random page order, NaN in unused slots and spare pages, -1 / 0 / stale
padding columns).  Every case is checked against the fp64 oracle over the
keys the oracle gathers from the pages, and bit for bit against rp_run on the
same keys stored contiguously.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import bf16_to_f64, compare, default_scale
from workloads import make_batch, make_paged

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_prefill_amd as vp
    assert vp.available(), "the gfx950 library did not load or the device is not a gfx950"


CASES = [
    # (qo_lens, kv_lens, Hq, Hkv, D, causal, page_size)
    ([1, 130, 257, 64], [1, 130, 257, 64], 8, 2, 128, True, 16),
    ([33, 129, 7], [500, 129, 2], 16, 2, 128, True, 32),        # append (qo < kv), qo > kv rows
    ([100, 3, 0], [0, 3, 5], 4, 2, 128, True, 64),               # kv = 0, empty request
    ([40, 200], [90, 200], 8, 1, 128, False, 128),               # g = 8, non-causal
    ([70, 150], [300, 150], 4, 2, 256, False, 16),               # hd256 non-causal
    ([1, 130, 64], [1, 130, 64], 8, 2, 256, True, 32),           # hd256 causal
]


def _runs(b, causal, page_size, seed, **plan_kw):
    import varlen_prefill_amd as vp
    sm = default_scale(b.head_dim)
    pk = make_paged(b, page_size, seed)
    q = b.q.to(DEV)
    plan = vp.Plan(b.q_indptr, b.kv_indptr, b.num_qo_heads, b.num_kv_heads, b.head_dim, causal,
                   **plan_kw)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device=DEV)
    plan.run_paged(q, pk.k_pages.to(DEV), pk.v_pages.to(DEV),
                   torch.from_numpy(pk.block_table).to(DEV), out=o, lse=lse, sm_scale=sm)
    oc = torch.full_like(q, float("nan"))
    lc = torch.full_like(lse, float("nan"))
    plan.run(q, b.k.to(DEV), b.v.to(DEV), out=oc, lse=lc, sm_scale=sm)
    torch.cuda.synchronize()
    plan.close()
    return pk, o.cpu(), lse.cpu(), oc.cpu(), lc.cpu()


@pytest.mark.parametrize("case", range(len(CASES)))
def test_paged_parity_and_bitwise(case):
    qo, kv, hq, hkv, d, causal, ps = CASES[case]
    b = make_batch(qo, kv, hq, hkv, d, seed=4000 + case, q_base=2)
    pk, o, lse, oc, lc = _runs(b, causal, ps, seed=4000 + case)
    # bit for bit the contiguous result
    assert torch.equal(o.view(torch.int16), oc.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lc.view(torch.int32))
    # and the oracle over the keys gathered from the pages
    k, v, ind = oracle.paged_kv_gather(pk.k_pages, pk.v_pages, pk.block_table, b.kv_lens, ps)
    ro, rl = oracle.ragged_attention(b.q, k, v, b.q_indptr, ind, hq, hkv, causal, default_scale(d))
    rows = np.zeros(b.q.shape[0], dtype=bool)
    for r in range(b.batch):
        rows[int(b.q_indptr[r]):int(b.q_indptr[r + 1])] = True
    rep = compare(bf16_to_f64(o)[rows], lse.double().numpy()[rows], ro[rows], rl[rows])
    print(rep)
    assert torch.isnan(o[~torch.from_numpy(rows)]).all()


@pytest.mark.parametrize("d", [128, 256])
def test_paged_split_kv_bitwise(d):
    b = make_batch([50, 300, 9], [700, 300, 1000], 8, 2, d, seed=4100 + d)
    for causal in (True, False):
        _, o, lse, oc, lc = _runs(b, causal, 32, seed=4100 + d, kv_chunk=128)
        assert torch.equal(o.view(torch.int16), oc.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lc.view(torch.int32))


def test_paged_argument_errors():
    import varlen_prefill_amd as vp
    b = make_batch([20], [40], 4, 2, 128, seed=4200)
    plan = vp.Plan(b.q_indptr, b.kv_indptr, 4, 2, 128, True)
    q = b.q.to(DEV)
    pool = torch.zeros(8, 8, 2, 128, dtype=torch.bfloat16, device=DEV)   # page_size 8
    table = torch.zeros(1, 8, dtype=torch.int32, device=DEV)
    with pytest.raises(vp.RaggedPrefillError, match="page_size"):
        plan.run_paged(q, pool, pool, table)
    pool16 = torch.zeros(8, 16, 2, 128, dtype=torch.bfloat16, device=DEV)
    short = torch.zeros(1, 2, dtype=torch.int32, device=DEV)               # 40 keys need 3 pages
    with pytest.raises(vp.RaggedPrefillError, match="max_blocks"):
        plan.run_paged(q, pool16, pool16, short)
    plan.close()
