"""The oracle's paged-KV gather, pinned against things other than itself.

* A hand-built pool whose every key value names its own page and slot, with a
  table that uses pages out of order, a negative entry (read as page 0, the
  clamp of page "vllm-rlt PR #112", design notes) and padding columns: the
  gathered keys are written out by hand.
* Round trip: the seeded scatter of ``workloads.make_paged`` (independent
  code, random page order, NaN in unused slots and spare pages, -1 / 0 /
  stale padding columns) gathered back gives every request's original keys,
  bit for bit, for every page size.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_batch, make_paged


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def test_hand_built_table():
    ps, hkv, d = 16, 1, 8
    # key value = 16 * page + slot, the same in every (head, d) position;
    # integers below 256 are exact in bf16
    pool = torch.tensor([[[[float(16 * p + s)] * d] * hkv for s in range(ps)] for p in range(3)],
                        dtype=torch.bfloat16)
    vpool = -pool
    table = np.array([[2, 0, -1], [1, -1, 7], [-1, 5, 5]], dtype=np.int32)
    kv_lens = [20, 5, 3]
    k, v, ind = oracle.paged_kv_gather(pool, vpool, table, kv_lens, ps)
    # request 0: keys 0..15 in page 2, keys 16..19 in page 0 slots 0..3
    # request 1: keys 0..4 in page 1; request 2: entry -1 is read as page 0
    want = [32 + j for j in range(16)] + [j for j in range(4)] + [16 + j for j in range(5)] + [0, 1, 2]
    assert list(ind) == [0, 20, 25, 28]
    got_k = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).float()[:, 0, 0].tolist()
    got_v = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).float()[:, 0, 0].tolist()
    assert got_k == [float(x) for x in want]
    assert got_v == [-float(x) for x in want]


@pytest.mark.parametrize("page_size", [16, 32, 64, 128])
@pytest.mark.parametrize("d", [128, 256])
def test_scatter_gather_round_trip(page_size, d):
    qo = [5, 0, 33, 1, 70]
    kv = [page_size * 2, 7, 0, 1, 3 * page_size + 5]
    b = make_batch(qo, kv, 8, 2, d, seed=61 + page_size)
    pk = make_paged(b, page_size, seed=61)
    assert pk.block_table.shape[1] >= max(-(-x // page_size) for x in kv)
    k, v, ind = oracle.paged_kv_gather(pk.k_pages, pk.v_pages, pk.block_table, b.kv_lens, page_size)
    assert np.array_equal(ind, b.kv_indptr)
    assert np.array_equal(k, _bits(b.k)) and np.array_equal(v, _bits(b.v))
    # the scatter really permuted the pages and left padding behind
    used = set()
    for r, n in enumerate(kv):
        used |= set(pk.block_table[r, : -(-n // page_size)].tolist())
    assert len(used) == sum(-(-n // page_size) for n in kv)
