"""rp_run_noalloc (split-KV partial states in the library's fixed device
array) against rp_run with a caller workspace: the same kernels, so the same
bits.  Two calls in a row, the second with a smaller input, then a head_dim
256 call; each compares bit for bit with rp_run on the same plan."""

from __future__ import annotations

import pytest
import torch

from parity import default_scale
from workloads import make_batch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_prefill_amd as vp
    assert vp.available(), "the gfx950 library did not load or the device is not a gfx950"


CALLS = [
    # qo_lens, kv_lens, Hq, Hkv, head_dim, kv_chunk, seed
    ([50, 300, 9], [700, 300, 1000], 8, 2, 128, 128, 61),
    ([20, 5], [400, 5], 8, 2, 128, 128, 62),
    ([33, 1], [900, 2500], 4, 2, 256, 256, 63),
]


def test_noalloc_matches_rp_run_bitwise():
    import varlen_prefill_amd as vp
    for qo, kv, hq, hkv, d, chunk, seed in CALLS:
        b = make_batch(qo, kv, hq, hkv, d, seed=seed)
        q, k, v = b.q.to(DEV), b.k.to(DEV), b.v.to(DEV)
        plan = vp.Plan(b.q_indptr, b.kv_indptr, hq, hkv, d, True, kv_chunk=chunk)
        assert plan.info["num_partial_items"] > 0 and plan.workspace_bytes > 0
        sm = default_scale(d)
        ro, rl = plan.run(q, k, v, sm_scale=sm)
        no = torch.full_like(q, float("nan"))
        nl = torch.full((q.shape[0], hq), float("nan"), dtype=torch.float32, device=DEV)
        plan.run_noalloc(q, k, v, out=no, lse=nl, sm_scale=sm)
        torch.cuda.synchronize()
        print(f"qo={qo} kv={kv} d={d}: workspace {plan.workspace_bytes} bytes, "
              f"{plan.info['num_partial_items']} partial items")
        assert torch.equal(no.view(torch.int16), ro.view(torch.int16))
        assert torch.equal(nl.view(torch.int32), rl.view(torch.int32))
        plan.close()
