"""GPU path against the fp64 oracle (needs an MI355X).

Every case draws its inputs from the seeded generator in ``workloads``, runs
the HIP library through its C ABI (via the ctypes binding), and checks the
result element by element against ``oracle`` (see tests/parity.py for the
gates).  Invariant and determinism cases compare GPU results with each other
bit for bit.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from parity import bf16_to_f64, compare, default_scale
from workloads import get_config, make_batch, make_config_batch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import varlen_prefill_amd as vp
    assert vp.available(), "the gfx950 library did not load or the device is not a gfx950"


def _gpu(batch, causal, sm_scale, fill=float("nan"), **plan_kw):
    """Run one batch through a fresh plan; outputs pre-filled with `fill`."""
    import varlen_prefill_amd as vp
    q, k, v = batch.q.to(DEV), batch.k.to(DEV), batch.v.to(DEV)
    out = torch.full_like(q, fill)
    lse = torch.full((q.shape[0], batch.num_qo_heads), fill, dtype=torch.float32, device=DEV)
    plan = vp.Plan(batch.q_indptr, batch.kv_indptr, batch.num_qo_heads, batch.num_kv_heads,
                   batch.head_dim, causal, **plan_kw)
    plan.run(q, k, v, out=out, lse=lse, sm_scale=sm_scale)
    torch.cuda.synchronize()
    plan.close()
    return out.cpu(), lse.cpu()


def _oracle(batch, causal, sm_scale):
    return oracle.ragged_attention(batch.q, batch.k, batch.v, batch.q_indptr, batch.kv_indptr,
                                   batch.num_qo_heads, batch.num_kv_heads, causal, sm_scale)


def _rows_in_requests(batch):
    rows = np.zeros(batch.q.shape[0], dtype=bool)
    for r in range(batch.batch):
        rows[int(batch.q_indptr[r]):int(batch.q_indptr[r + 1])] = True
    return rows


def _check_full(batch, causal, sm_scale, **plan_kw):
    o, lse = _gpu(batch, causal, sm_scale, **plan_kw)
    ro, rl = _oracle(batch, causal, sm_scale)
    rows = _rows_in_requests(batch)
    rep = compare(bf16_to_f64(o)[rows], lse.double().numpy()[rows], ro[rows], rl[rows])
    # rows outside every request are never written
    assert torch.isnan(o[~torch.from_numpy(rows)]).all()
    assert torch.isnan(lse[~torch.from_numpy(rows)]).all()
    print(rep)
    return o, lse, rep


def test_tiny_config():
    cfg = get_config("tiny")
    b = make_config_batch(cfg)
    _check_full(b, cfg.causal, default_scale(cfg.head_dim))


CASES = [
    # (qo_lens, kv_lens, Hq, Hkv, D, causal)
    ([1, 130, 257, 64], [1, 130, 257, 64], 8, 2, 128, True),          # several tiles, ragged tails
    ([300, 5, 77], [300, 5, 77], 4, 4, 128, True),                      # MHA (g = 1), 128-token tiles
    ([40, 0, 1, 200], [90, 3, 1, 200], 8, 1, 128, False),               # g = 8, non-causal, qo != kv
    ([33, 129, 7], [500, 129, 2], 16, 2, 128, True),                    # append (qo < kv), qo > kv rows
    ([100, 3, 0], [0, 3, 5], 4, 2, 128, True),                          # kv = 0, zero-length request
    ([1, 130, 257, 64], [1, 130, 257, 64], 8, 2, 256, True),            # hd256
    ([70, 150], [300, 150], 4, 2, 256, False),                          # hd256 non-causal
    ([45, 12], [45, 300], 12, 4, 128, True),                            # g = 3 (padding rows)
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_small_ragged(case):
    qo, kv, hq, hkv, d, causal = CASES[case]
    b = make_batch(qo, kv, hq, hkv, d, seed=1000 + case, q_base=3, kv_base=5)
    _check_full(b, causal, default_scale(d))


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("mode", ["always", "never"])
def test_split_kv_chunks(d, mode):
    # a small canonical chunk makes multi-chunk tiles: split items + the merge
    # kernel ("always") or items that fold their chunks in the workgroup ("never")
    import varlen_prefill_amd as vp
    split_mode = vp.RP_SPLIT_ALWAYS if mode == "always" else vp.RP_SPLIT_NEVER
    b = make_batch([50, 300, 9], [700, 300, 1000], 8, 2, d, seed=2000 + d)
    for causal in (True, False):
        _check_full(b, causal, default_scale(d), kv_chunk=128, split_mode=split_mode)
    # non-positive scales take the other kernel branch
    for sm in (0.0, -0.05):
        o, lse = _gpu(b, True, sm, kv_chunk=128, split_mode=split_mode)
        ro, rl = _oracle(b, True, sm)
        rows = _rows_in_requests(b)
        compare(bf16_to_f64(o)[rows], lse.double().numpy()[rows], ro[rows], rl[rows])


def _run_variant(batch, variant, **plan_kw):
    """One batch through a fresh plan with contiguous bf16 K/V ("bf16"),
    FP8 (E4M3) K/V ("fp8") or a paged bf16 cache of 16-key pages ("paged")."""
    import varlen_prefill_amd as vp
    from workloads import make_fp8_kv, make_paged
    q = batch.q.to(DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], batch.num_qo_heads), float("nan"), dtype=torch.float32, device=DEV)
    plan = vp.Plan(batch.q_indptr, batch.kv_indptr, batch.num_qo_heads, batch.num_kv_heads,
                   batch.head_dim, True, **plan_kw)
    sm = default_scale(batch.head_dim)
    if variant == "bf16":
        plan.run(q, batch.k.to(DEV), batch.v.to(DEV), out=out, lse=lse, sm_scale=sm)
    elif variant == "fp8":
        k8, v8 = make_fp8_kv(batch, 0.5, 0.75)
        plan.run_fp8kv(q, k8.to(DEV), v8.to(DEV), 0.5, 0.75, out=out, lse=lse, sm_scale=sm)
    else:
        pg = make_paged(batch, 16, seed=batch.seed + len(batch.qo_lens))
        plan.run_paged(q, pg.k_pages.to(DEV), pg.v_pages.to(DEV),
                       torch.from_numpy(pg.block_table).to(DEV), out=out, lse=lse, sm_scale=sm)
    torch.cuda.synchronize()
    plan.close()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("d,variant", [(128, "bf16"), (256, "bf16"), (128, "fp8"), (256, "fp8"),
                                       (128, "paged"), (256, "paged")])
def test_batch_composition_bitwise(d, variant):
    """Each request's bits do not depend on the batch: the request alone, in
    the batch and in a permuted batch, with and without split KV, for every
    kernel instance (head_dim 128 / 256; bf16, FP8 and paged K/V)."""
    lens_q = [130, 0, 1, 257, 64, 600]
    lens_kv = [130, 7, 1, 400, 64, 600]
    for kv_chunk in (0, 192):
        full = make_batch(lens_q, lens_kv, 8, 2, d, seed=77)
        fo, fl = _run_variant(full, variant, kv_chunk=kv_chunk)
        perm = [5, 3, 0, 2, 4, 1]
        pb = make_batch([lens_q[i] for i in perm], [lens_kv[i] for i in perm], 8, 2, d, seed=77,
                        request_ids=perm)
        po, pl = _run_variant(pb, variant, kv_chunk=kv_chunk)
        for r in range(len(lens_q)):
            alone = make_batch([lens_q[r]], [lens_kv[r]], 8, 2, d, seed=77, request_ids=[r])
            ao, al = _run_variant(alone, variant, kv_chunk=kv_chunk)
            q0, q1 = int(full.q_indptr[r]), int(full.q_indptr[r + 1])
            pos = perm.index(r)
            p0, p1 = int(pb.q_indptr[pos]), int(pb.q_indptr[pos + 1])
            assert torch.equal(ao.view(torch.int16), fo[q0:q1].view(torch.int16))
            assert torch.equal(al.view(torch.int32), fl[q0:q1].view(torch.int32))
            assert torch.equal(po[p0:p1].view(torch.int16), fo[q0:q1].view(torch.int16))
            assert torch.equal(pl[p0:p1].view(torch.int32), fl[q0:q1].view(torch.int32))


def test_split_mode_always_matches_auto_bitwise():
    import varlen_prefill_amd as vp
    b = make_batch([200, 31], [3000, 31], 8, 2, 128, seed=5)
    ao, al = _gpu(b, True, default_scale(128), kv_chunk=1024)
    so, sl = _gpu(b, True, default_scale(128), kv_chunk=1024, split_mode=vp.RP_SPLIT_ALWAYS)
    assert torch.equal(ao.view(torch.int16), so.view(torch.int16))
    assert torch.equal(al.view(torch.int32), sl.view(torch.int32))


@pytest.mark.parametrize("d,variant", [(128, "bf16"), (256, "bf16"), (128, "fp8"), (256, "fp8"),
                                       (128, "paged"), (256, "paged")])
def test_split_modes_bitwise(d, variant):
    """In-workgroup chunk folding (NEVER), split items + merge kernel
    (ALWAYS) and the automatic choice give the same bits, for every kernel
    instance; the canonical chunk of 192 keys gives tiles of 2..11 chunks,
    a ragged last chunk, and chunks a tile's causal rows only partly see."""
    import varlen_prefill_amd as vp
    qo, kv = [50, 300, 9, 1, 130, 64], [700, 300, 1000, 2100, 2000, 64]
    b = make_batch(qo, kv, 8, 2, d, seed=3000 + d)
    info = vp.Plan(b.q_indptr, b.kv_indptr, 8, 2, d, True, kv_chunk=192,
                   split_mode=vp.RP_SPLIT_NEVER, host_only=True).info
    assert info["num_fold_items"] > 0 and info["num_merge_items"] == 0
    ref_o, ref_l = _run_variant(b, variant, kv_chunk=192, split_mode=vp.RP_SPLIT_ALWAYS)
    for mode in (vp.RP_SPLIT_NEVER, vp.RP_SPLIT_AUTO):
        o, l = _run_variant(b, variant, kv_chunk=192, split_mode=mode)
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), mode
        assert torch.equal(l.view(torch.int32), ref_l.view(torch.int32)), mode


def test_repeat_runs_bitwise():
    import varlen_prefill_amd as vp
    b = make_batch([300, 45], [300, 1000], 8, 2, 128, seed=6)
    q, k, v = b.q.to(DEV), b.k.to(DEV), b.v.to(DEV)
    plan = vp.Plan(b.q_indptr, b.kv_indptr, 8, 2, 128, True, kv_chunk=256)
    o0, l0 = plan.run(q, k, v)
    o0, l0 = o0.clone(), l0.clone()
    for _ in range(10):
        o1, l1 = plan.run(q, k, v)
        assert torch.equal(o1.view(torch.int16), o0.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l0.view(torch.int32))
    plan.close()


def test_closed_forms_on_gpu():
    import varlen_prefill_amd as vp
    d = 128
    # kv_len = 1 -> O = V[0] exactly; causal qo = kv -> row 0 = V[0] exactly
    b = make_batch([5, 70], [1, 70], 8, 2, d, seed=8)
    o, _ = _gpu(b, False, default_scale(d))
    assert torch.equal(o[0:5].float(), b.v[0:1].float().repeat_interleave(4, 1).expand(5, 8, d))
    o, _ = _gpu(b, True, default_scale(d))
    assert torch.equal(o[5].float(), b.v[1].float().repeat_interleave(4, 0))
    # sm_scale = 0 -> mean of the visible V rows; LSE = ln(#visible)
    b = make_batch([9, 200], [9, 300], 4, 2, d, seed=9)
    o, lse = _gpu(b, True, 0.0)
    ro, rl = _oracle(b, True, 0.0)
    compare(bf16_to_f64(o), lse.double().numpy(), ro, rl)
    # negative scale goes through the same definition
    o, lse = _gpu(b, True, -0.05)
    ro, rl = _oracle(b, True, -0.05)
    compare(bf16_to_f64(o), lse.double().numpy(), ro, rl)


def test_one_shot_entry_point_and_streams():
    import varlen_prefill_amd as vp
    cfg = get_config("tiny")
    b = make_config_batch(cfg)
    q, k, v = b.q.to(DEV), b.k.to(DEV), b.v.to(DEV)
    ro, rl = _oracle(b, True, default_scale(128))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = vp.ragged_prefill(q, k, v, b.q_indptr, b.kv_indptr, causal=True)
    s.synchronize()
    compare(bf16_to_f64(o.cpu()), lse.cpu().double().numpy(), ro, rl)
    o2, lse2 = vp.ragged_prefill(q, k, v, torch.from_numpy(b.q_indptr).to(DEV),
                                 torch.from_numpy(b.kv_indptr).to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu().view(torch.int16), o.cpu().view(torch.int16))
    # empty batch: returns without launching
    e = torch.empty(0, 4, 128, dtype=torch.bfloat16, device=DEV)
    ek = torch.empty(0, 2, 128, dtype=torch.bfloat16, device=DEV)
    vp.ragged_prefill(e, ek, ek, [0], [0])


def test_one_shot_two_streams_split_bitwise():
    """Two one-shot calls whose plans split KV (decode-like requests, 2048-key
    chunks), enqueued back to back on two streams with no synchronisation in
    between, give the bits of the two-phase API: each stream has its own
    partial-state workspace."""
    import varlen_prefill_amd as vp
    b1 = make_batch([1, 1, 3], [5000, 3000, 4500], 8, 2, 128, seed=41)
    b2 = make_batch([1, 2], [6100, 2500], 8, 2, 128, seed=42)
    refs = [_gpu(b, True, default_scale(128), fill=0.0) for b in (b1, b2)]
    dev = [(b.q.to(DEV), b.k.to(DEV), b.v.to(DEV)) for b in (b1, b2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    results = []
    for _ in range(4):
        for i, (b, (q, k, v)) in enumerate(zip((b1, b2), dev)):
            with torch.cuda.stream(streams[i]):
                results.append((i, vp.ragged_prefill(q, k, v, b.q_indptr, b.kv_indptr, causal=True)))
    torch.cuda.synchronize()
    for i, (o, lse) in results:
        ro, rl = refs[i]
        assert torch.equal(o.cpu().view(torch.int16), ro.view(torch.int16))
        assert torch.equal(lse.cpu().view(torch.int32), rl.view(torch.int32))


def test_one_shot_graph_capture():
    """A one-shot call captured into a HIP graph after a warm-up call on the
    capturing stream replays to the eager bits; under capture, offsets with
    no cached plan are refused before anything is enqueued."""
    import varlen_prefill_amd as vp
    b = make_batch([1, 2], [6100, 2500], 8, 2, 128, seed=43)
    q, k, v = b.q.to(DEV), b.k.to(DEV), b.v.to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], 8, dtype=torch.float32, device=DEV)
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        vp.ragged_prefill(q, k, v, b.q_indptr, b.kv_indptr, causal=True, out=out, lse=lse)
    s_.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s_):
        vp.ragged_prefill(q, k, v, b.q_indptr, b.kv_indptr, causal=True, out=out, lse=lse)
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32))
    other = make_batch([1, 3], [7000, 900], 8, 2, 128, seed=44)
    oq, ok_, ov = other.q.to(DEV), other.k.to(DEV), other.v.to(DEV)
    x = torch.zeros(1, device=DEV)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s_):
        x.add_(1.0)
        with pytest.raises(vp.RaggedPrefillError):
            vp.ragged_prefill(oq, ok_, ov, other.q_indptr, other.kv_indptr, causal=True)
    g2.replay()
    torch.cuda.synchronize()
    assert float(x.item()) == 1.0


def test_injected_allocation_failure_leaves_outputs_untouched(monkeypatch):
    """RP_FAULT_INJECT=alloc makes the library's device allocations fail: plan
    creation and a one-shot call that needs a new plan return RP_ENOMEM and
    leave the outputs as they were; the next call without it works."""
    import varlen_prefill_amd as vp
    from varlen_prefill_amd import _lib
    b = make_batch([1, 40], [5300, 5400], 8, 2, 128, seed=45)
    q, k, v = b.q.to(DEV), b.k.to(DEV), b.v.to(DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], 8), float("nan"), dtype=torch.float32, device=DEV)
    monkeypatch.setenv("RP_FAULT_INJECT", "alloc")
    with pytest.raises(vp.RaggedPrefillError) as ei:
        vp.Plan(b.q_indptr, b.kv_indptr, 8, 2, 128, True)
    assert ei.value.status == _lib.RP_ENOMEM
    with pytest.raises(vp.RaggedPrefillError) as ei:
        vp.ragged_prefill(q, k, v, b.q_indptr, b.kv_indptr, causal=True, out=out, lse=lse)
    assert ei.value.status == _lib.RP_ENOMEM
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all()
    monkeypatch.delenv("RP_FAULT_INJECT")
    vp.ragged_prefill(q, k, v, b.q_indptr, b.kv_indptr, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = _oracle(b, True, default_scale(128))
    compare(bf16_to_f64(out.cpu()), lse.cpu().double().numpy(), ro, rl)


@pytest.mark.parametrize("mode", ["auto", "never"])
def test_graph_capture_replays(mode):
    """A captured rp_run replays bit-identically (split items + merge kernel,
    or fold items whose running state lives in the workspace), with eager
    work and synchronisations between the replays."""
    import varlen_prefill_amd as vp
    split_mode = vp.RP_SPLIT_NEVER if mode == "never" else vp.RP_SPLIT_AUTO
    b = make_batch([150, 20], [900, 20], 8, 2, 128, seed=12)
    q, k, v = b.q.to(DEV), b.k.to(DEV), b.v.to(DEV)
    plan = vp.Plan(b.q_indptr, b.kv_indptr, 8, 2, 128, True, kv_chunk=256, split_mode=split_mode)
    assert (plan.info["num_fold_items"] > 0) == (mode == "never")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], 8, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    plan.run(q, k, v, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            plan.run(q, k, v, out=out, lse=lse, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xA5)   # stale workspace contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32))
    plan.close()


# Full-size workloads whose every row the oracle computes in seconds to tens of
# seconds: (workload, causal)
FULL_ROWS = [
    ("hd128_gqa_causal", True),
    ("ragged64", True),
    ("hd256_gqa", True),
    ("hd256_gqa", False),
]


@pytest.mark.parametrize("case", FULL_ROWS, ids=[f"{n}{'' if c else '_noncausal'}" for n, c in FULL_ROWS])
def test_full_size_config_all_rows(case):
    """Full-size workloads in the benchmark's launch configuration (one-shot
    plan with default chunking), every (token, qo head) row against the
    oracle."""
    name, causal = case
    cfg = get_config(name)
    b = make_config_batch(cfg)
    sm = default_scale(cfg.head_dim)
    o, lse = _gpu(b, causal, sm)
    ro, rl = _oracle(b, causal, sm)
    rep = compare(bf16_to_f64(o), lse.double().numpy(), ro, rl)
    print(f"{name} causal={causal}: {rep}")


# (workload, causal, edge tokens per request end, random rows); the append
# workload's rows see up to 16K keys and the decode workloads up to 32K, so
# their rows are sampled
FULL_SIZE = [
    ("decode64", True, 40, 3000),
    ("decode_few", True, 40, 3000),
    ("mixed", True, 40, 3000),
    ("append_prefix", True, 4, 2000),
]


@pytest.mark.parametrize("case", FULL_SIZE, ids=[f"{n}{'' if c else '_noncausal'}" for n, c, _, _ in FULL_SIZE])
def test_full_size_config_sampled(case):
    """Full-size workloads in the benchmark's launch configuration: every head
    of the first/last `edge` tokens of each request and `nrand` random rows
    are checked against the oracle row by row."""
    name, causal, edge, nrand = case
    cfg = get_config(name)
    b = make_config_batch(cfg)
    sm = default_scale(cfg.head_dim)
    o, lse = _gpu(b, causal, sm)
    rng = np.random.default_rng(123)
    toks = []
    for r in range(b.batch):
        q0, q1 = int(b.q_indptr[r]), int(b.q_indptr[r + 1])
        toks += list(range(q0, min(q1, q0 + edge))) + list(range(max(q0, q1 - edge), q1))
    toks = np.unique(np.array(toks, dtype=np.int64))
    tt = np.repeat(toks, cfg.num_qo_heads)
    hh = np.tile(np.arange(cfg.num_qo_heads), toks.size)
    total = int(b.q_indptr[-1])
    rt = rng.integers(0, total, nrand)
    rh = rng.integers(0, cfg.num_qo_heads, nrand)
    tt = np.concatenate([tt, rt])
    hh = np.concatenate([hh, rh])
    ro, rl = oracle.ragged_attention_rows(b.q, b.k, b.v, b.q_indptr, b.kv_indptr,
                                          cfg.num_qo_heads, cfg.num_kv_heads, causal, sm,
                                          tt, hh)
    og = bf16_to_f64(o)[tt, hh]
    lg = lse.double().numpy()[tt, hh]
    print(compare(og, lg, ro, rl))
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()


def _scale_keys(batch, factor):
    """Multiply key j of every request by factor(j) (request-relative), in
    place, keeping bf16 inputs: both sides then see the same scaled keys."""
    for r in range(batch.batch):
        k0, k1 = int(batch.kv_indptr[r]), int(batch.kv_indptr[r + 1])
        if k1 > k0:
            f = factor(torch.arange(k1 - k0, dtype=torch.float32))
            batch.k[k0:k1] = (batch.k[k0:k1].float() * f[:, None, None]).to(torch.bfloat16)


STRESS = ["growing", "sink", "wide_scale", "growing_split", "growing_hd256", "sink_hd256",
          "wide_scale_hd256", "wide_scale_split", "growing_fold", "wide_scale_fold"]


@pytest.mark.parametrize("mode", STRESS)
def test_reference_max_moves(mode):
    """Score profiles that move the running reference max of the online
    softmax often and by large steps (keys that grow along the sequence, a
    large sm_scale), or never (one dominant first key).  Random N(0,1)
    inputs almost never move it after a tile's first key block, so these
    cases drive the update paths that keep or move the reference (and the
    rescale of the accumulator) that the other tests rarely reach.  Their
    softmax is dominated by a few keys anywhere in a row, which is what the
    kernel's split of P into bf16 hi + lo parts is for: they are held to the
    same gates as every other case."""
    d = 256 if mode.endswith("_hd256") else 128
    b = make_batch([200, 64, 700, 33], [200, 64, 700, 900], 8, 2, d, seed=3100)
    sm = default_scale(d)
    plan_kw = {}
    if mode.startswith("growing"):
        _scale_keys(b, lambda j: 1.0 + j / 48.0)
    elif mode.startswith("sink"):
        _scale_keys(b, lambda j: torch.where(j == 0, 6.0, 1.0))
    elif mode.startswith("wide_scale"):
        sm = 1.0
    if mode.endswith("_split"):
        plan_kw["kv_chunk"] = 128
    if mode.endswith("_fold"):
        import varlen_prefill_amd as vp
        plan_kw.update(kv_chunk=128, split_mode=vp.RP_SPLIT_NEVER)
    _check_full(b, True, sm, **plan_kw)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_every_placement(seed):
    """Seeded random ragged batches (request count, lengths with qo <= kv and
    qo > kv, empty requests, GQA group 1..8, head_dim 128/256, causal or
    not, canonical chunks of 64..320 keys): the fold placement (NEVER)
    against the oracle at the standard gates, and NEVER, ALWAYS and AUTO
    bit for bit."""
    import varlen_prefill_amd as vp
    rng = np.random.default_rng(4000 + seed)
    n = int(rng.integers(1, 6))
    qo = [int(x) for x in rng.integers(0, 200, n)]
    kv = [int(x) if rng.random() < 0.8 else int(q) for x, q in zip(rng.integers(0, 900, n), qo)]
    g = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2]))
    d = int(rng.choice([128, 256]))
    causal = bool(rng.random() < 0.7)
    chunk = int(rng.choice([64, 128, 192, 320]))
    b = make_batch(qo, kv, g * hkv, hkv, d, seed=4000 + seed, q_base=int(rng.integers(0, 3)))
    sm = default_scale(d)
    print(f"qo={qo} kv={kv} g={g} hkv={hkv} d={d} causal={causal} chunk={chunk}", flush=True)
    o, lse, _ = _check_full(b, causal, sm, kv_chunk=chunk, split_mode=vp.RP_SPLIT_NEVER)
    for mode in (vp.RP_SPLIT_ALWAYS, vp.RP_SPLIT_AUTO):
        o2, l2 = _gpu(b, causal, sm, kv_chunk=chunk, split_mode=mode)
        assert torch.equal(o2.view(torch.int16), o.view(torch.int16)), mode
        assert torch.equal(l2.view(torch.int32), lse.view(torch.int32)), mode


EXTREME = [
    # qo, kv, Hq, Hkv, D, causal
    ([3, 1, 2], [70000, 1, 0], 128, 1, 128, True),     # GQA group 128 (one token per tile), 35 decode chunks
    ([300], [70000], 8, 1, 128, True),                 # 9 canonical chunks of 8192 keys per tile
    ([64, 5, 40], [64, 300, 9000], 64, 4, 256, True),  # group 16 at head_dim 256 (8 tokens per tile)
    ([33], [20000], 16, 2, 256, False),                # non-causal, 3 chunks at head_dim 256
]


@pytest.mark.parametrize("case", range(len(EXTREME)))
def test_extreme_shapes(case):
    """Largest GQA groups, very long KV (tens of canonical chunks) and
    non-causal long KV: every row against the oracle in the fold placement,
    and split and fold placements bit for bit."""
    import varlen_prefill_amd as vp
    qo, kv, hq, hkv, d, causal = EXTREME[case]
    b = make_batch(qo, kv, hq, hkv, d, seed=5000 + case)
    sm = default_scale(d)
    o, lse, _ = _check_full(b, causal, sm, split_mode=vp.RP_SPLIT_NEVER)
    o2, l2 = _gpu(b, causal, sm, split_mode=vp.RP_SPLIT_ALWAYS)
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16))
    assert torch.equal(l2.view(torch.int32), lse.view(torch.int32))
