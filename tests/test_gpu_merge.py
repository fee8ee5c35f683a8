"""Attention-state merging and shared-prefix attention on the GPU.

merge_state / merge_state_in_place / merge_states are checked against the
fp64 oracle's merge of the same (bf16 v, fp32 lse) inputs.  The kernel sums
k weighted terms in fp32 and rounds once to bf16, so each output must lie
within one bf16 spacing of the fp64 value (a faithful rounding) plus the fp32
summation bound (k + 4) 2^-24 sum_i w_i |v_i| (k fma roundings, the
exponential, the normalisation); the scale sum_i w_i |v_i| is the oracle's
merge of |v|.  The LSE must agree within fp32 rounding.  Shared-prefix attention is
checked against the oracle's attention over the concatenated keys with the
usual parity gates, bit for bit against rp_run when the prefix is empty, and
with the own keys in a paged cache bit for bit against the contiguous run.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import _bf16_neighbours, bf16_to_f64, compare, default_scale
from workloads import make_batch, make_paged, request_tensors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_prefill_amd as vp
    assert vp.available(), "the gfx950 library did not load or the device is not a gfx950"


def _states(rows, k, h, d, seed, empty_frac=0.1):
    """k random states per (row, head): v bf16 ~ N(0,1) * 2, lse fp32 spread
    over ~[-30, 30] around a per-row offset, some states empty (-inf)."""
    rng = np.random.default_rng(seed)
    v = torch.from_numpy((2 * rng.standard_normal((rows, k, h, d))).astype(np.float32)).to(torch.bfloat16)
    off = rng.uniform(-60, 60, (rows, 1, h))
    lse = (off + rng.uniform(-30, 30, (rows, k, h))).astype(np.float32)
    lse[rng.random((rows, k, h)) < empty_frac] = -np.inf
    lse[0, :, 0] = -np.inf                      # a row-head with every state empty
    return v, torch.from_numpy(lse)


def _check_faithful(v_gpu, s_gpu, v_ref, s_ref, scale, k):
    vg = bf16_to_f64(v_gpu)
    sg = s_gpu.double().cpu().numpy()
    empty = np.isneginf(s_ref)
    assert np.array_equal(np.isneginf(sg), empty)
    assert np.all(vg[empty] == 0.0)
    lo, hi = _bf16_neighbours(v_ref)
    ok = np.abs(vg - v_ref) <= (hi - lo) + (k + 4) * 2.0**-24 * np.nan_to_num(scale)
    ok[empty] = True
    if not ok.all():
        idx = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{int((~ok).sum())} outputs not a faithful rounding; first at {idx}: "
                             f"gpu={vg[idx]!r} ref={v_ref[idx]!r}")
    live = ~empty
    err = np.abs(sg[live] - s_ref[live])
    assert np.all(err <= 2e-5 + 2e-6 * np.abs(s_ref[live])), f"lse error {err.max():.3e}"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_merge_state_and_in_place(d):
    import varlen_prefill_amd as vp
    rows, h = 333, 5
    v, s = _states(rows, 2, h, d, seed=d)
    va, vb = v[:, 0].contiguous().to(DEV), v[:, 1].contiguous().to(DEV)
    sa, sb = s[:, 0].contiguous().to(DEV), s[:, 1].contiguous().to(DEV)
    vo, so = vp.merge_state(va, sa, vb, sb)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_state(bf16_to_f64(v[:, 0]), s[:, 0].double().numpy(),
                                bf16_to_f64(v[:, 1]), s[:, 1].double().numpy())
    scale, _ = oracle.merge_state(np.abs(bf16_to_f64(v[:, 0])), s[:, 0].double().numpy(),
                                  np.abs(bf16_to_f64(v[:, 1])), s[:, 1].double().numpy())
    _check_faithful(vo.cpu(), so.cpu(), ro, rl, scale, 2)
    # in place gives the same bits
    vi, si = va.clone(), sa.clone()
    vp.merge_state_in_place(vi, si, vb, sb)
    torch.cuda.synchronize()
    assert torch.equal(vi.view(torch.int16), vo.view(torch.int16))
    assert torch.equal(si.view(torch.int32), so.view(torch.int32))


@pytest.mark.parametrize("k,d", [(1, 128), (3, 128), (7, 64), (4, 256), (16, 128)])
def test_merge_states(k, d):
    import varlen_prefill_amd as vp
    rows, h = 129, 8
    v, s = _states(rows, k, h, d, seed=100 + k)
    vo, so = vp.merge_states(v.to(DEV), s.to(DEV))
    torch.cuda.synchronize()
    vs, ss = np.moveaxis(bf16_to_f64(v), 1, 2), np.moveaxis(s.double().numpy(), 1, 2)
    ro, rl = oracle.merge_states(vs, ss)
    scale, _ = oracle.merge_states(np.abs(vs), ss)
    _check_faithful(vo.cpu(), so.cpu(), ro, rl, scale, k)
    if k == 1:
        live = ~torch.isneginf(s[:, 0])
        assert torch.equal(vo.cpu()[live].view(torch.int16), v[:, 0][live].view(torch.int16))
        assert torch.equal(so.cpu()[live], s[:, 0][live])


def test_merge_of_two_runs_equals_attention_over_union():
    """rp_run over key sets A and B of the same queries, merged, against the
    oracle over A ++ B."""
    import varlen_prefill_amd as vp
    hq, hkv, d = 8, 2, 128
    qo, ka, kb = [40, 1, 77], [100, 3, 0], [60, 250, 30]
    a = make_batch(qo, ka, hq, hkv, d, seed=501)
    b = make_batch(qo, kb, hq, hkv, d, seed=502)
    sm = default_scale(d)
    q = a.q.to(DEV)
    outs = []
    for bt in (a, b):
        plan = vp.Plan(bt.q_indptr, bt.kv_indptr, hq, hkv, d, causal=False)
        outs.append(plan.run(q, bt.k.to(DEV), bt.v.to(DEV), sm_scale=sm))
    vo, so = vp.merge_state(outs[0][0], outs[0][1], outs[1][0], outs[1][1])
    torch.cuda.synchronize()
    k_cat, v_cat, lens = [], [], []
    for r in range(len(qo)):
        sl_a = slice(int(a.kv_indptr[r]), int(a.kv_indptr[r + 1]))
        sl_b = slice(int(b.kv_indptr[r]), int(b.kv_indptr[r + 1]))
        k_cat += [a.k[sl_a], b.k[sl_b]]
        v_cat += [a.v[sl_a], b.v[sl_b]]
        lens.append(ka[r] + kb[r])
    ind = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ro, rl = oracle.ragged_attention(a.q, torch.cat(k_cat), torch.cat(v_cat), a.q_indptr, ind, hq,
                                     hkv, False, sm)
    print(compare(bf16_to_f64(vo.cpu()), so.double().cpu().numpy(), ro, rl))


def _shared_prefix_case(qo, kv, p, hq, hkv, d, causal, seed):
    import varlen_prefill_amd as vp
    b = make_batch(qo, kv, hq, hkv, d, seed=seed, q_base=3)
    _, ks, vs = request_tensors(seed, 10**6, 0, p, hq, hkv, d)   # the shared prefix keys
    sm = default_scale(d)
    plan = vp.SharedPrefixPlan(b.q_indptr, b.kv_indptr, p, hq, hkv, d, causal)
    q = b.q.to(DEV)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], hq), float("nan"), dtype=torch.float32, device=DEV)
    plan.run(q, ks.to(DEV), vs.to(DEV), b.k.to(DEV), b.v.to(DEV), out=o, lse=lse, sm_scale=sm)
    torch.cuda.synchronize()
    info = plan.info
    plan.close()
    # the definition: attention over [shared keys, own keys] per request
    k_cat, v_cat = [], []
    for r in range(b.batch):
        sl = slice(int(b.kv_indptr[r]), int(b.kv_indptr[r + 1]))
        k_cat += [ks, b.k[sl]]
        v_cat += [vs, b.v[sl]]
    ind = np.concatenate([[0], np.cumsum([p + x for x in kv])]).astype(np.int32)
    ro, rl = oracle.ragged_attention(b.q, torch.cat(k_cat), torch.cat(v_cat), b.q_indptr, ind, hq,
                                     hkv, causal, sm)
    rows = slice(3, None)
    rep = compare(bf16_to_f64(o.cpu())[rows], lse.double().cpu().numpy()[rows], ro[rows], rl[rows])
    print(rep)
    assert torch.isnan(o[:3].cpu()).all() and torch.isnan(lse[:3].cpu()).all()
    return b, o, lse, info


@pytest.mark.parametrize("case", [
    # qo, own kv, shared len, Hq, Hkv, D, causal
    ([30, 130, 1, 0, 64], [30, 200, 5, 9, 64], 700, 32, 8, 128, True),
    ([30, 130, 7], [60, 130, 0], 257, 8, 8, 128, False),
    ([17, 90], [17, 300], 1000, 16, 4, 256, True),
    ([5, 64], [0, 64], 33, 4, 1, 256, False),
    ([40, 40], [40, 50], 9000, 8, 2, 128, True),          # long prefix: split-KV in level 1
])
def test_shared_prefix_parity(case):
    qo, kv, p, hq, hkv, d, causal = case
    _shared_prefix_case(qo, kv, p, hq, hkv, d, causal, seed=600 + p)


def test_shared_prefix_empty_prefix_is_rp_run_bitwise():
    import varlen_prefill_amd as vp
    qo, kv = [30, 130, 1], [30, 200, 5]
    b, o, lse, _ = _shared_prefix_case(qo, kv, 0, 8, 2, 128, True, seed=700)
    plan = vp.Plan(b.q_indptr, b.kv_indptr, 8, 2, 128, True)
    oc, lc = plan.run(b.q.to(DEV), b.k.to(DEV), b.v.to(DEV), sm_scale=default_scale(128))
    torch.cuda.synchronize()
    assert torch.equal(o[3:].view(torch.int16), oc[3:].view(torch.int16))
    assert torch.equal(lse[3:].view(torch.int32), lc[3:].view(torch.int32))


@pytest.mark.parametrize("case", [
    # qo, own kv, shared len, Hq, Hkv, D, causal, kv_chunk, split mode
    ([30, 130, 1, 0, 64], [30, 200, 5, 9, 64], 700, 32, 8, 128, True, 0, "auto"),
    ([17, 90], [17, 300], 1000, 16, 4, 256, True, 0, "auto"),
    ([40, 300, 3], [700, 300, 1000], 500, 8, 2, 128, True, 128, "always"),   # merge kernel path
    ([40, 300, 3], [700, 300, 1000], 500, 8, 2, 128, True, 128, "never"),    # fold items
    ([40, 100], [700, 1000], 300, 8, 2, 256, False, 128, "always"),
])
def test_shared_prefix_equals_two_runs_and_merge_bitwise(case):
    """Shared-prefix attention is bit-identical to running both levels as
    ordinary plans and merging them with merge_state, whatever the own
    level's placement (final items, split items + merge kernel, fold items),
    with and without the LSE output."""
    import varlen_prefill_amd as vp
    qo, kv, p, hq, hkv, d, causal, chunk, mode = case
    split_mode = {"auto": vp.RP_SPLIT_AUTO, "always": vp.RP_SPLIT_ALWAYS,
                  "never": vp.RP_SPLIT_NEVER}[mode]
    b = make_batch(qo, kv, hq, hkv, d, seed=900 + p, q_base=2)
    _, ks, vs = request_tensors(900 + p, 10**6, 0, p, hq, hkv, d)
    sm = default_scale(d)
    q, ksd, vsd = b.q.to(DEV), ks.to(DEV), vs.to(DEV)
    kd, vd = b.k.to(DEV), b.v.to(DEV)
    sp = vp.SharedPrefixPlan(b.q_indptr, b.kv_indptr, p, hq, hkv, d, causal, kv_chunk=chunk,
                             split_mode=split_mode)
    of, lf = sp.run(q, ksd, vsd, kd, vd, sm_scale=sm)
    of, lf = of.clone(), lf.clone()
    on, ln = sp.run(q, ksd, vsd, kd, vd, sm_scale=sm, return_lse=False)   # no LSE output
    assert ln is None
    q0, q1 = int(b.q_indptr[0]), int(b.q_indptr[-1])
    assert torch.equal(on[q0:q1].view(torch.int16), of[q0:q1].view(torch.int16))
    lvl1 = vp.Plan([0, q1 - q0], [0, p], hq, hkv, d, False, kv_chunk=chunk, split_mode=split_mode)
    o1, l1 = lvl1.run(q[q0:q1].contiguous(), ksd, vsd, sm_scale=sm)
    lvl2 = vp.Plan(b.q_indptr, b.kv_indptr, hq, hkv, d, causal, kv_chunk=chunk, split_mode=split_mode)
    o2, l2 = lvl2.run(q, kd, vd, sm_scale=sm)
    om, lm = vp.merge_state(o1, l1, o2[q0:q1].contiguous(), l2[q0:q1].contiguous())
    torch.cuda.synchronize()
    for x in (sp, lvl1, lvl2):
        x.close()
    assert torch.equal(of[q0:q1].view(torch.int16), om.view(torch.int16))
    assert torch.equal(lf[q0:q1].view(torch.int32), lm.view(torch.int32))


@pytest.mark.parametrize("case", [
    # qo, own kv, shared len, Hq, Hkv, D, causal, page size
    ([30, 130, 1, 0, 64], [30, 200, 5, 9, 64], 700, 32, 8, 128, True, 16),
    ([17, 90], [17, 300], 1000, 16, 4, 256, True, 64),
    ([5, 64, 40], [0, 64, 333], 33, 8, 2, 128, False, 32),
])
def test_shared_prefix_paged_equals_contiguous_bitwise(case):
    """Own keys in a paged cache (random page order, padded table) give the
    same bits as the contiguous own keys."""
    import varlen_prefill_amd as vp
    qo, kv, p, hq, hkv, d, causal, ps = case
    b = make_batch(qo, kv, hq, hkv, d, seed=800 + p)
    _, ks, vs = request_tensors(800 + p, 10**6, 0, p, hq, hkv, d)
    pk = make_paged(b, ps, seed=800 + ps)
    sm = default_scale(d)
    plan = vp.SharedPrefixPlan(b.q_indptr, b.kv_indptr, p, hq, hkv, d, causal)
    q, ksd, vsd = b.q.to(DEV), ks.to(DEV), vs.to(DEV)
    oc, lc = plan.run(q, ksd, vsd, b.k.to(DEV), b.v.to(DEV), sm_scale=sm)
    oc, lc = oc.clone(), lc.clone()
    op, lp = plan.run_paged(q, ksd, vsd, pk.k_pages.to(DEV), pk.v_pages.to(DEV),
                            torch.from_numpy(pk.block_table).to(DEV), sm_scale=sm)
    torch.cuda.synchronize()
    plan.close()
    assert torch.equal(op.view(torch.int16), oc.view(torch.int16))
    assert torch.equal(lp.view(torch.int32), lc.view(torch.int32))


def test_argument_errors():
    import varlen_prefill_amd as vp
    v = torch.zeros(4, 2, 96, dtype=torch.bfloat16, device=DEV)
    s = torch.zeros(4, 2, dtype=torch.float32, device=DEV)
    with pytest.raises(vp.RaggedPrefillError, match="head_dim"):
        vp.merge_state(v, s, v, s)
    # causal shared prefix with more queries than own keys is rejected
    with pytest.raises(vp.RaggedPrefillError, match="qo_len <= kv_len"):
        vp.SharedPrefixPlan([0, 10], [0, 5], 100, 4, 2, 128, causal=True)
    plan = vp.SharedPrefixPlan([0, 10], [0, 5], 100, 4, 2, 128, causal=False)
    q = torch.zeros(10, 4, 128, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(5, 2, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(vp.RaggedPrefillError, match="shared-prefix plan"):
        vp.Plan.run(plan, q, kv, kv)
    plan.close()
