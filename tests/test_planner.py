"""Planner properties on host-only plans (no GPU needed).

* coverage: for every request, kv head and query token, the work items cover
  exactly the visible keys [0, limit of the tile's last row) once, in
  canonical request-relative chunks (kv_chunk keys; at most 2048 for
  decode-like requests of at most 32 query rows);
* split tiles have one merge item whose slots hold chunks 0..n-1 in order;
* the plan of a request does not depend on the rest of the batch;
* items are ordered longest-first; algorithmic flops/bytes follow the counting
  rule 4 * D * Hq * visible pairs and Q,K,V read + O,LSE written once.
"""

import numpy as np
import pytest

import varlen_prefill_amd as vp
from workloads import CONFIGS
from workloads.gen import indptr_from_lens

F = {name: i for i, name in enumerate(vp.ITEM_FIELDS)}


def _limit(i, qo, kv, causal):
    if not causal:
        return kv
    return min(max(i + kv - qo + 1, 0), kv)


def _check_plan(qo_lens, kv_lens, hq, hkv, d, causal, kv_chunk=0, q_base=0, kv_base=0,
                num_xcds=0):
    qi = indptr_from_lens(qo_lens, q_base)
    ki = indptr_from_lens(kv_lens, kv_base)
    p = vp.Plan(qi, ki, hq, hkv, d, causal, kv_chunk=kv_chunk, host_only=True, num_xcds=num_xcds)
    info = p.info
    launch = p.items()
    xcds = num_xcds or 8
    # longest-first within each XCD's share of the launch order (workgroup b
    # runs on XCD b % xcds); padding items (n_tok = 0) carry no work
    for x in range(xcds):
        mine = launch[x::xcds]
        mine = mine[mine[:, F["n_tok"]] > 0]
        assert np.all(mine[:-1, F["cost"]] >= mine[1:, F["cost"]])
    pad = launch[launch[:, F["n_tok"]] == 0]
    assert np.all(pad[:, F["key_end"]] <= pad[:, F["key_begin"]])
    items = launch[launch[:, F["n_tok"]] > 0]
    chunk = info["kv_chunk"]
    g = hq // hkv
    tt = 128 // g
    assert info["tile_tokens"] == tt
    # coverage
    seen = {}
    slots = set()
    for it in items:
        key = (it[F["request"]], it[F["kv_head"]], it[F["t0"]])
        seen.setdefault(key, []).append((it[F["key_begin"]], it[F["key_end"]], it[F["slot"]],
                                         it[F["chunk"]]))
        if it[F["slot"]] >= 0:
            assert it[F["slot"]] not in slots
            slots.add(it[F["slot"]])
    n_expected = 0
    for b, (qo, kv) in enumerate(zip(qo_lens, kv_lens)):
        # decode-like requests (at most 32 query rows) use chunks of at most 2048 keys
        cb = min(chunk, 2048) if qo * g <= 32 else chunk
        for t0 in range(0, qo, tt):
            n_tok = min(tt, qo - t0)
            lim_last = _limit(t0 + n_tok - 1, qo, kv, causal)
            for kvh in range(hkv):
                n_expected += 1
                ranges = sorted(seen.pop((b, kvh, t0)))
                if len(ranges) == 1:
                    kb, ke, slot, _ = ranges[0]
                    assert (kb, ke, slot) == (0, lim_last, -1)
                else:
                    assert all(r[2] >= 0 for r in ranges)
                    assert ranges[0][0] == 0 and ranges[-1][1] == lim_last
                    for c, (kb, ke, slot, ch) in enumerate(ranges):
                        assert ch == c and kb == c * cb
                        assert ke == min((c + 1) * cb, lim_last)
                        assert slot == ranges[0][2] + c
    assert not seen, f"items outside every tile: {list(seen)[:3]}"
    # the rows each item names lie in its request
    for it in items:
        b = it[F["request"]]
        assert it[F["q_tok0"]] == qi[b] + it[F["t0"]]
        assert it[F["kv_row0"]] == ki[b]
        assert it[F["t0"]] + it[F["n_tok"]] <= qo_lens[b]
    # algorithmic work
    pairs = sum(_limit(i, qo, kv, causal) for qo, kv in zip(qo_lens, kv_lens) for i in range(qo))
    assert info["flops"] == pytest.approx(4.0 * d * hq * pairs, rel=1e-12)
    tq, tk = sum(qo_lens), sum(kv_lens)
    assert info["bytes"] == pytest.approx(2.0 * d * (2 * hq * tq + 2 * hkv * tk) + 4.0 * hq * tq,
                                          rel=1e-12)
    return p, items


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (32, 8, 128), (4, 4, 256), (12, 4, 128),
                                      (64, 8, 128)])
def test_coverage_random(causal, hq, hkv, d):
    rng = np.random.default_rng(hq * 7 + d + causal)
    for _ in range(3):
        n = int(rng.integers(1, 9))
        qo = rng.integers(0, 700, n).tolist()
        kv = rng.integers(0, 1500, n).tolist()
        qo[0] = 0
        _check_plan(qo, kv, hq, hkv, d, causal, kv_chunk=256, q_base=int(rng.integers(0, 5)))


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_coverage_configs(name):
    c = CONFIGS[name]
    _check_plan(c.qo_lens, c.kv_lens, c.num_qo_heads, c.num_kv_heads, c.head_dim, c.causal)


def test_plan_of_a_request_is_independent_of_the_batch():
    qo = [130, 0, 1, 257, 64, 600]
    kv = [130, 7, 1, 400, 64, 3000]
    _, full = _check_plan(qo, kv, 8, 2, 128, True, kv_chunk=256)
    rel = ["n_tok", "t0", "qo_len", "kv_len", "kv_head", "key_begin", "key_end", "chunk",
           "lim_first", "cost"]
    idx = [F[r] for r in rel]
    for b in range(len(qo)):
        _, alone = _check_plan([qo[b]], [kv[b]], 8, 2, 128, True, kv_chunk=256)
        mine = full[full[:, F["request"]] == b][:, idx]
        other = alone[:, idx]
        order = lambda a: a[np.lexsort(a.T[::-1])]
        assert np.array_equal(order(mine), order(other))
        # partial items keep partial placement
        assert (np.sum(full[full[:, F["request"]] == b][:, F["slot"]] >= 0)
                == np.sum(alone[:, F["slot"]] >= 0))


def test_plan_is_deterministic():
    c = CONFIGS["ragged64"]
    _, a = _check_plan(c.qo_lens, c.kv_lens, 32, 8, 128, True)
    _, b = _check_plan(c.qo_lens, c.kv_lens, 32, 8, 128, True)
    assert np.array_equal(a, b)


def test_workspace_size_counts_partial_states():
    p, items = _check_plan([64], [5000], 8, 2, 128, True, kv_chunk=1024)
    n_slots = int(np.sum(items[:, F["slot"]] >= 0))
    assert n_slots == 2 * 2 * 5  # two 32-token tiles x two kv heads x five chunks
    assert p.workspace_bytes >= n_slots * 128 * (128 + 1) * 4


def test_xcd_grouping_keeps_tiles_of_one_kv_head_together():
    c = CONFIGS["hd128_gqa_causal"]
    p, _ = _check_plan(c.qo_lens, c.kv_lens, 32, 8, 128, True)
    launch = p.items()
    homes = {}
    costs = np.zeros(8)
    for b, it in enumerate(launch):
        if it[F["n_tok"]] == 0:
            continue
        homes.setdefault((it[F["request"]], it[F["kv_head"]]), set()).add(b % 8)
        costs[b % 8] += it[F["cost"]]
    # most (request, kv head) groups live on a single XCD; loads are balanced
    single = sum(1 for v in homes.values() if len(v) == 1)
    assert single >= 0.6 * len(homes)
    assert costs.max() <= 1.02 * costs.mean() + launch[:, F["cost"]].max()


def test_single_xcd_order_is_plain_longest_first():
    c = CONFIGS["ragged64"]
    p, _ = _check_plan(c.qo_lens, c.kv_lens, 32, 8, 128, True, num_xcds=1)
    launch = p.items()
    assert np.all(launch[:, F["n_tok"]] > 0)
    assert np.all(launch[:-1, F["cost"]] >= launch[1:, F["cost"]])
