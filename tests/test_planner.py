"""Planner properties on host-only plans (no GPU needed).

* coverage: for every request, kv head and query token, the work items cover
  exactly the visible keys [0, limit of the tile's last row) once, in
  canonical request-relative chunks (kv_chunk keys; at most 2048 for
  decode-like requests of at most 32 query rows);
* split tiles have one merge item whose slots hold chunks 0..n-1 in order;
  folded tiles have one item over all their keys with its own slot, the
  chunk count and the chunk size;
* the split mode: NEVER folds every multi-chunk tile, ALWAYS splits it, the
  automatic mode folds at head_dim 128 when the longest folded tile costs no
  more than 1/512 of the whole plan;
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
                num_xcds=0, split_mode=vp.RP_SPLIT_AUTO):
    qi = indptr_from_lens(qo_lens, q_base)
    ki = indptr_from_lens(kv_lens, kv_base)
    p = vp.Plan(qi, ki, hq, hkv, d, causal, kv_chunk=kv_chunk, host_only=True, num_xcds=num_xcds,
                split_mode=split_mode)
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
                                         it[F["chunk"]], it[F["fold_keys"]]))
        if it[F["slot"]] >= 0:
            assert it[F["slot"]] not in slots
            slots.add(it[F["slot"]])
    n_expected = 0
    n_fold = n_split = 0
    for b, (qo, kv) in enumerate(zip(qo_lens, kv_lens)):
        # decode-like requests (at most 32 query rows) use chunks of at most 2048 keys
        cb = min(chunk, 2048) if qo * g <= 32 else chunk
        for t0 in range(0, qo, tt):
            n_tok = min(tt, qo - t0)
            lim_last = _limit(t0 + n_tok - 1, qo, kv, causal)
            for kvh in range(hkv):
                n_expected += 1
                ranges = sorted(seen.pop((b, kvh, t0)))
                n_chunks = -(-lim_last // cb)
                if len(ranges) == 1 and ranges[0][4] > 0:
                    # folded tile: all its keys, its own slot, chunk count and size
                    kb, ke, slot, ch, fk = ranges[0]
                    assert (kb, ke, ch, fk) == (0, lim_last, n_chunks, cb) and n_chunks > 1
                    assert slot >= 0
                    n_fold += 1
                elif len(ranges) == 1:
                    kb, ke, slot, _, _ = ranges[0]
                    assert (kb, ke, slot) == (0, lim_last, -1) and n_chunks <= 1
                else:
                    assert all(r[2] >= 0 and r[4] == 0 for r in ranges)
                    assert ranges[0][0] == 0 and ranges[-1][1] == lim_last
                    for c, (kb, ke, slot, ch, _) in enumerate(ranges):
                        assert ch == c and kb == c * cb
                        assert ke == min((c + 1) * cb, lim_last)
                        assert slot == ranges[0][2] + c
                    n_split += 1
    assert not seen, f"items outside every tile: {list(seen)[:3]}"
    assert info["num_fold_items"] == n_fold
    assert info["num_merge_items"] == n_split
    if split_mode == vp.RP_SPLIT_NEVER:
        assert n_split == 0
    if split_mode == vp.RP_SPLIT_ALWAYS:
        assert n_fold == 0
    if split_mode == vp.RP_SPLIT_AUTO and (n_fold or n_split):
        assert n_fold == 0 or n_split == 0     # one placement for the whole plan
        tile_cost = {}
        for it in items:
            key = (it[F["request"]], it[F["kv_head"]], it[F["t0"]])
            tile_cost[key] = tile_cost.get(key, 0) + it[F["cost"]]
        multi = {(it[F["request"]], it[F["kv_head"]], it[F["t0"]]) for it in items if it[F["slot"]] >= 0}
        longest = max(tile_cost[k] for k in multi)
        folds = d == 128 and longest * 512 <= sum(tile_cost.values())
        assert (n_fold > 0) == folds
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


@pytest.mark.parametrize("split_mode", [vp.RP_SPLIT_AUTO, vp.RP_SPLIT_NEVER, vp.RP_SPLIT_ALWAYS])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (32, 8, 128), (4, 4, 256), (12, 4, 128),
                                      (64, 8, 128)])
def test_coverage_random(causal, hq, hkv, d, split_mode):
    rng = np.random.default_rng(hq * 7 + d + causal)
    for _ in range(3):
        n = int(rng.integers(1, 9))
        qo = rng.integers(0, 700, n).tolist()
        kv = rng.integers(0, 1500, n).tolist()
        qo[0] = 0
        _check_plan(qo, kv, hq, hkv, d, causal, kv_chunk=256, q_base=int(rng.integers(0, 5)),
                    split_mode=split_mode)


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_coverage_configs(name):
    c = CONFIGS[name]
    _check_plan(c.qo_lens, c.kv_lens, c.num_qo_heads, c.num_kv_heads, c.head_dim, c.causal)


@pytest.mark.parametrize("split_mode", [vp.RP_SPLIT_NEVER, vp.RP_SPLIT_ALWAYS])
def test_plan_of_a_request_is_independent_of_the_batch(split_mode):
    # (in the automatic mode the placement is chosen per plan; the bits are
    # the same either way, which the GPU tests check)
    qo = [130, 0, 1, 257, 64, 600]
    kv = [130, 7, 1, 400, 64, 3000]
    _, full = _check_plan(qo, kv, 8, 2, 128, True, kv_chunk=256, split_mode=split_mode)
    rel = ["n_tok", "t0", "qo_len", "kv_len", "kv_head", "key_begin", "key_end", "chunk",
           "lim_first", "cost", "fold_keys"]
    idx = [F[r] for r in rel]
    for b in range(len(qo)):
        _, alone = _check_plan([qo[b]], [kv[b]], 8, 2, 128, True, kv_chunk=256, split_mode=split_mode)
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
    p, items = _check_plan([64], [5000], 8, 2, 128, True, kv_chunk=1024, split_mode=vp.RP_SPLIT_ALWAYS)
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


def test_fold_items_take_one_slot_each():
    p, items = _check_plan([64], [5000], 8, 2, 128, True, kv_chunk=1024, split_mode=vp.RP_SPLIT_NEVER)
    assert len(items) == 2 * 2 and np.all(items[:, F["fold_keys"]] == 1024)
    assert sorted(items[:, F["slot"]].tolist()) == [0, 1, 2, 3]
    assert p.info["num_merge_items"] == 0 and p.info["num_partial_items"] == 0
    assert p.workspace_bytes >= 4 * 128 * (128 + 1) * 4
    # cost of a folded tile: the sum of its chunks' costs as split items
    q = _check_plan([64], [5000], 8, 2, 128, True, kv_chunk=1024, split_mode=vp.RP_SPLIT_ALWAYS)[1]
    for kvh in range(2):
        for t0 in (0, 32):
            sel = lambda a: a[(a[:, F["kv_head"]] == kvh) & (a[:, F["t0"]] == t0)]
            assert sel(items)[:, F["cost"]].sum() == sel(q)[:, F["cost"]].sum()


@pytest.mark.parametrize("name,folds", [("append_prefix", True), ("decode64", False),
                                        ("decode_few", False), ("mixed", False),
                                        ("hd256_gqa", False)])
def test_automatic_placement_of_the_workloads(name, folds):
    """The automatic mode folds where the grid fills the GPU without split-KV
    (long-prefix append at head_dim 128) and splits where it would not (decode
    batches); at head_dim 256 it always splits."""
    c = CONFIGS[name]
    p, items = _check_plan(c.qo_lens, c.kv_lens, c.num_qo_heads, c.num_kv_heads, c.head_dim, c.causal)
    info = p.info
    if folds:
        assert info["num_fold_items"] > 0 and info["num_merge_items"] == 0
    else:
        assert info["num_fold_items"] == 0
