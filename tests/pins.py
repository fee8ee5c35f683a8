"""Pins of the fp64 oracle to things other than itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle bound by
``lib`` (``None`` = the real build) disagrees with:

* a library routine that the method reduces to: torch's fp64
  ``scaled_dot_product_attention`` (non-causal, square causal through the
  library's own ``is_causal``, bottom-right causal through an explicit mask);
  the log-sum-exp is recovered from the same routine by adding one extra key
  of score 0 whose value is a one-hot in an extra dimension, whose output is
  ``1 / (1 + sum_j exp(s_j))``;
* closed forms (one key, identical keys, zero scale, constant values, row 0 of
  a square causal request, fully masked rows);
* invariants (batch composition, GQA as replicated MHA, value scaling, score
  shift, key permutation without a mask, rows outside every request);
* the merge identity (two disjoint key windows merged equal the whole).

The mutation test runs these against deliberately broken oracle builds and
requires every mutant to fail at least one pin.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from workloads import make_batch

SM = float(np.float32(1.0 / math.sqrt(64)))


def _bf16(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _f64(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.float64)


def _visible_mask(qo: int, kv: int, causal: bool) -> torch.Tensor:
    """Boolean [qo, kv]; bottom-right causal alignment (key j visible to row i
    iff j <= i + kv - qo)."""
    if not causal:
        return torch.ones(qo, kv, dtype=torch.bool)
    i = torch.arange(qo).unsqueeze(1)
    j = torch.arange(kv).unsqueeze(0)
    return j <= i + (kv - qo)


def _sdpa_request(q, k, v, causal, sm_scale, group):
    """Library attention for one request: q [qo,Hq,D], k/v [kv,Hkv,D] (fp64).
    Returns O [qo,Hq,D], LSE [qo,Hq] for rows with >= 1 visible key, plus the
    boolean row mask of such rows."""
    qo, hq, d = q.shape
    kv = k.shape[0]
    kr = k.repeat_interleave(group, dim=1)  # kv head of qo head h is h // group
    vr = v.repeat_interleave(group, dim=1)
    qh, kh, vh = q.transpose(0, 1), kr.transpose(0, 1), vr.transpose(0, 1)
    if causal and qo == kv:
        o = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True, scale=sm_scale)
    else:
        o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=_visible_mask(qo, kv, causal),
                                           scale=sm_scale)
    # log-sum-exp through one extra key of score 0 and a one-hot value
    q_aug = torch.cat([qh, torch.zeros(hq, qo, 1, dtype=q.dtype)], -1)
    k_aug = torch.cat([torch.cat([kh, torch.zeros(hq, kv, 1, dtype=q.dtype)], -1),
                       torch.zeros(hq, 1, d + 1, dtype=q.dtype)], 1)
    v_extra = torch.zeros(hq, 1, d + 1, dtype=q.dtype)
    v_extra[..., d] = 1.0
    v_aug = torch.cat([torch.cat([vh, torch.zeros(hq, kv, 1, dtype=q.dtype)], -1), v_extra], 1)
    m = torch.cat([_visible_mask(qo, kv, causal), torch.ones(qo, 1, dtype=torch.bool)], 1)
    ox = F.scaled_dot_product_attention(q_aug, k_aug, v_aug, attn_mask=m, scale=sm_scale)[..., d]
    lse = torch.log1p(-ox) - torch.log(ox)
    rows = _visible_mask(qo, kv, causal).any(1)
    return o.transpose(0, 1), lse.transpose(0, 1), rows


def _check_against_library(b, causal, sm_scale, lib, o=None, lse=None):
    if o is None:
        o, lse = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, b.num_qo_heads,
                                         b.num_kv_heads, causal, sm_scale, lib=lib)
    group = b.num_qo_heads // b.num_kv_heads
    for r in range(b.batch):
        q0, q1 = int(b.q_indptr[r]), int(b.q_indptr[r + 1])
        k0, k1 = int(b.kv_indptr[r]), int(b.kv_indptr[r + 1])
        if q1 == q0:
            continue
        if k1 == k0:
            assert np.all(o[q0:q1] == 0.0) and np.all(lse[q0:q1] == -np.inf)
            continue
        ro, rl, rows = _sdpa_request(_f64(b.q[q0:q1]), _f64(b.k[k0:k1]), _f64(b.v[k0:k1]), causal,
                                     sm_scale, group)
        rows = rows.numpy()
        got_o, got_l = o[q0:q1], lse[q0:q1]
        np.testing.assert_allclose(got_o[rows], ro.numpy()[rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(got_l[rows], rl.numpy()[rows], rtol=0, atol=1e-9)
        # rows that see no key: exact zeros and -inf
        assert np.all(got_o[~rows] == 0.0) and np.all(got_l[~rows] == -np.inf)


def pin_library_noncausal(lib=None):
    b = make_batch([5, 1, 33, 0, 70], [9, 1, 40, 3, 70], 4, 2, 64, seed=101)
    _check_against_library(b, False, SM, lib)


def pin_library_causal_square(lib=None):
    b = make_batch([1, 17, 64, 0, 90], [1, 17, 64, 0, 90], 6, 2, 64, seed=102)
    _check_against_library(b, True, SM, lib)


def pin_library_causal_bottom_right(lib=None):
    # qo < kv (append over a prefix), qo > kv (leading rows fully masked),
    # kv = 0 with qo > 0
    b = make_batch([3, 20, 12, 4, 7], [50, 24, 5, 0, 7], 8, 2, 32, seed=103)
    _check_against_library(b, True, 0.3, lib)


def pin_library_mha_hd128(lib=None):
    b = make_batch([40, 9], [40, 31], 2, 2, 128, seed=104)
    _check_against_library(b, True, float(np.float32(1 / math.sqrt(128))), lib)
    _check_against_library(b, False, float(np.float32(1 / math.sqrt(128))), lib)


def pin_closed_forms(lib=None):
    d = 16
    # one key: O = V[0] exactly; LSE = the single score
    q = np.zeros((3, 1, d), np.float32); q[:, 0, 0] = [1.0, -2.0, 0.5]
    k = np.zeros((1, 1, d), np.float32); k[0, 0, 0] = 2.0
    v = np.random.default_rng(7).standard_normal((1, 1, d)).astype(np.float32)
    qt, kt, vt = _bf16(q), _bf16(k), _bf16(v)
    o, lse = oracle.ragged_attention(qt, kt, vt, [0, 3], [0, 1], 1, 1, False, 0.25, lib=lib)
    for i in range(3):
        assert np.array_equal(o[i, 0], _f64(vt[0, 0]).numpy())
    np.testing.assert_allclose(lse[:, 0], [0.5, -1.0, 0.25], rtol=0, atol=1e-15)

    # identical keys: O row i = mean of the visible V rows, LSE = s + ln(#visible)
    n = 6
    q = np.zeros((n, 1, d), np.float32); q[:, 0, 0] = 3.0
    k = np.zeros((n, 1, d), np.float32); k[:, 0, 0] = 0.5
    v = np.random.default_rng(8).standard_normal((n, 1, d)).astype(np.float32)
    qt, kt, vt = _bf16(q), _bf16(k), _bf16(v)
    vd = _f64(vt).numpy()
    o, lse = oracle.ragged_attention(qt, kt, vt, [0, n], [0, n], 1, 1, True, 0.5, lib=lib)
    for i in range(n):
        np.testing.assert_allclose(o[i, 0], vd[: i + 1, 0].mean(0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[i, 0], 0.75 + math.log(i + 1), rtol=0, atol=1e-14)

    # zero scale: O = mean of visible V, LSE = ln(#visible), bottom-right rows
    b = make_batch([4, 9, 5], [10, 9, 2], 2, 1, d, seed=9)
    o, lse = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 2, 1, True, 0.0,
                                     lib=lib)
    vd = _f64(b.v).numpy()
    for r in range(3):
        q0, k0 = int(b.q_indptr[r]), int(b.kv_indptr[r])
        qo, kv = b.qo_lens[r], b.kv_lens[r]
        for i in range(qo):
            lim = min(max(i + kv - qo + 1, 0), kv)
            for h in range(2):
                if lim == 0:
                    assert np.all(o[q0 + i, h] == 0) and lse[q0 + i, h] == -np.inf
                else:
                    np.testing.assert_allclose(o[q0 + i, h], vd[k0:k0 + lim, 0].mean(0),
                                               rtol=0, atol=1e-14)
                    np.testing.assert_allclose(lse[q0 + i, h], math.log(lim), rtol=0, atol=1e-14)

    # constant values: O = c whatever the scores
    b = make_batch([7], [11], 2, 2, d, seed=10)
    vc = torch.full_like(b.v, 1.5)
    o, _ = oracle.ragged_attention(b.q, b.k, vc, b.q_indptr, b.kv_indptr, 2, 2, True, SM,
                                   lib=lib)
    np.testing.assert_allclose(o, 1.5, rtol=0, atol=1e-14)

    # square causal: row 0 sees only key 0 -> O = V[0] exactly
    b = make_batch([12, 30], [12, 30], 4, 2, d, seed=11)
    o, _ = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2, True, SM,
                                   lib=lib)
    for r in range(2):
        q0, k0 = int(b.q_indptr[r]), int(b.kv_indptr[r])
        for h in range(4):
            assert np.array_equal(o[q0, h], _f64(b.v[k0, h // 2]).numpy())


def pin_invariants(lib=None):
    d = 32
    lens_q, lens_kv = [13, 0, 40, 7, 25], [13, 5, 60, 7, 3]
    b = make_batch(lens_q, lens_kv, 8, 2, d, seed=21)
    o, lse = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 8, 2, True, SM,
                                     lib=lib)
    # batch composition: each request alone and in a permuted batch, bit for bit
    for r in range(len(lens_q)):
        s = make_batch([lens_q[r]], [lens_kv[r]], 8, 2, d, seed=21, request_ids=[r])
        so, sl = oracle.ragged_attention(s.q, s.k, s.v, s.q_indptr, s.kv_indptr, 8, 2, True, SM,
                                         lib=lib)
        q0, q1 = int(b.q_indptr[r]), int(b.q_indptr[r + 1])
        assert np.array_equal(so, o[q0:q1]) and np.array_equal(sl, lse[q0:q1])
    perm = [3, 0, 4, 2, 1]
    p = make_batch([lens_q[i] for i in perm], [lens_kv[i] for i in perm], 8, 2, d, seed=21,
                   request_ids=perm)
    po, pl = oracle.ragged_attention(p.q, p.k, p.v, p.q_indptr, p.kv_indptr, 8, 2, True, SM,
                                     lib=lib)
    for pos, r in enumerate(perm):
        a0, a1 = int(p.q_indptr[pos]), int(p.q_indptr[pos + 1])
        q0, q1 = int(b.q_indptr[r]), int(b.q_indptr[r + 1])
        assert np.array_equal(po[a0:a1], o[q0:q1]) and np.array_equal(pl[a0:a1], lse[q0:q1])

    # GQA equals MHA with each kv head replicated over its group, bit for bit
    kr = b.k.repeat_interleave(4, dim=1).contiguous()
    vr = b.v.repeat_interleave(4, dim=1).contiguous()
    mo, ml = oracle.ragged_attention(b.q, kr, vr, b.q_indptr, b.kv_indptr, 8, 8, True, SM,
                                     lib=lib)
    rows = ~np.isnan(lse[:, 0])
    assert np.array_equal(mo[rows], o[rows]) and np.array_equal(ml[rows], lse[rows])

    # scaling V by 2 scales O by 2 exactly; LSE unchanged
    so, sl = oracle.ragged_attention(b.q, b.k, (b.v.float() * 2).to(torch.bfloat16),
                                     b.q_indptr, b.kv_indptr, 8, 2, True, SM, lib=lib)
    assert np.array_equal(so[rows], 2 * o[rows]) and np.array_equal(sl[rows], lse[rows])

    # score shift: an extra dimension with q = 1, k = c adds sm_scale*c to every
    # score -> O unchanged, LSE + sm_scale*c
    c = 6.0
    q_aug = torch.cat([b.q, torch.ones(b.q.shape[0], 8, 1, dtype=torch.bfloat16)], -1)
    k_aug = torch.cat([b.k, torch.full((b.k.shape[0], 2, 1), c, dtype=torch.bfloat16)], -1)
    v_aug = torch.cat([b.v, torch.zeros(b.v.shape[0], 2, 1, dtype=torch.bfloat16)], -1)
    ao, al = oracle.ragged_attention(q_aug, k_aug, v_aug, b.q_indptr, b.kv_indptr, 8, 2, True,
                                     SM, lib=lib)
    np.testing.assert_allclose(ao[rows][..., :d], o[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(al[rows], lse[rows] + SM * c, rtol=0, atol=1e-12)

    # no mask: permuting the keys (with their values) changes nothing
    nb = make_batch([6, 20], [33, 17], 4, 2, d, seed=22)
    no, nl = oracle.ragged_attention(nb.q, nb.k, nb.v, nb.q_indptr, nb.kv_indptr, 4, 2, False,
                                     SM, lib=lib)
    idx = np.concatenate([np.random.default_rng(3).permutation(33),
                          33 + np.random.default_rng(4).permutation(17)])
    po, pl = oracle.ragged_attention(nb.q, nb.k[idx], nb.v[idx], nb.q_indptr, nb.kv_indptr, 4, 2,
                                     False, SM, lib=lib)
    np.testing.assert_allclose(po, no, rtol=0, atol=1e-12)
    np.testing.assert_allclose(pl, nl, rtol=0, atol=1e-12)

    # rows outside every request (indptr[0] != 0) and zero-length requests are
    # not written
    ob = make_batch([0, 5, 0, 3], [4, 5, 0, 9], 2, 1, d, seed=23, q_base=3, kv_base=2)
    oo, ol = oracle.ragged_attention(ob.q, ob.k, ob.v, ob.q_indptr, ob.kv_indptr, 2, 1, True, SM,
                                     lib=lib)
    assert np.all(np.isnan(oo[:3])) and np.all(np.isnan(ol[:3]))
    assert not np.any(np.isnan(oo[3:])) and not np.any(np.isnan(ol[3:]))


def pin_merge(lib=None):
    d = 32
    b = make_batch([9, 30, 4], [9, 64, 40], 4, 2, d, seed=31)
    for causal in (False, True):
        full_o, full_l = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2,
                                                 causal, SM, lib=lib)
        for split in (1, 5, 17, 33):
            ao, al = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2, causal,
                                             SM, key_window=(0, split), lib=lib)
            bo, bl = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2, causal,
                                             SM, key_window=(split, -1), lib=lib)
            mo, ml = oracle.merge_state(ao, al, bo, bl, lib=lib)
            np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)
    # an empty state is the identity, exactly
    e_o = np.zeros_like(full_o)
    e_l = np.full_like(full_l, -np.inf)
    mo, ml = oracle.merge_state(full_o, full_l, e_o, e_l, lib=lib)
    assert np.array_equal(mo, full_o) and np.array_equal(ml, full_l)
    mo, ml = oracle.merge_state(e_o, e_l, full_o, full_l, lib=lib)
    assert np.array_equal(mo, full_o) and np.array_equal(ml, full_l)
    # two states of equal log-sum-exp average with weight 1/2 each and add ln 2
    x = np.random.default_rng(5).standard_normal((3, d))
    y = np.random.default_rng(6).standard_normal((3, d))
    l0 = np.array([0.0, 2.0, -3.0])
    mo, ml = oracle.merge_state(x, l0, y, l0, lib=lib)
    np.testing.assert_allclose(mo, 0.5 * (x + y), rtol=0, atol=1e-15)
    np.testing.assert_allclose(ml, l0 + math.log(2.0), rtol=0, atol=1e-15)


def pin_merge_states(lib=None):
    """merge_states over k disjoint key windows equals attention over their
    union; closed-form weights; identity, order and empty-state cases."""
    d = 32
    b = make_batch([9, 30, 4], [9, 64, 40], 4, 2, d, seed=37)
    for causal in (False, True):
        full_o, full_l = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2,
                                                 causal, SM, lib=lib)
        for cuts in ((0, 3, 20, -1), (0, 1, 2, 30, 50, -1), (0, 7, 7, -1)):
            parts = [oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2, causal,
                                             SM, key_window=(lo, hi), lib=lib)
                     for lo, hi in zip(cuts[:-1], cuts[1:])]
            o = np.stack([p[0] for p in parts], axis=-2)    # [rows, Hq, k, D]
            l = np.stack([p[1] for p in parts], axis=-1)    # [rows, Hq, k]
            mo, ml = oracle.merge_states(o, l, lib=lib)
            np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)
            # the order of the states does not matter
            perm = np.random.default_rng(len(cuts)).permutation(len(parts))
            po, pl = oracle.merge_states(o[..., perm, :], l[..., perm], lib=lib)
            np.testing.assert_allclose(po, mo, rtol=0, atol=1e-14)
            np.testing.assert_allclose(pl, ml, rtol=0, atol=1e-14)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 3, d))
    # closed form: masses 1 : 2 : 5 give weights 1/8, 2/8, 5/8 and lse log 8 (+ offset)
    for off in (0.0, 40.0, -700.0):
        l = np.full((2, 3), off) + np.log([1.0, 2.0, 5.0])
        mo, ml = oracle.merge_states(x, l, lib=lib)
        np.testing.assert_allclose(mo, (x[:, 0] + 2 * x[:, 1] + 5 * x[:, 2]) / 8, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, off + math.log(8.0), rtol=0, atol=1e-12)
    # one state is returned unchanged; empty states carry no mass; all empty -> (0, -inf)
    mo, ml = oracle.merge_states(x[:, :1], np.array([[0.5], [-2.0]]), lib=lib)
    assert np.array_equal(mo, x[:, 0]) and np.array_equal(ml, [0.5, -2.0])
    l = np.array([[-np.inf, 1.5, -np.inf], [-np.inf, -np.inf, -np.inf]])
    mo, ml = oracle.merge_states(x, l, lib=lib)
    assert np.array_equal(mo[0], x[0, 1]) and ml[0] == 1.5
    assert np.array_equal(mo[1], np.zeros(d)) and ml[1] == -np.inf
    # two states: the same as the pairwise merge
    l2 = np.array([[0.3, -1.2], [4.0, 4.5]])
    mo, ml = oracle.merge_states(x[:, :2], l2, lib=lib)
    po, pl = oracle.merge_state(x[:, 0], l2[:, 0], x[:, 1], l2[:, 1], lib=lib)
    np.testing.assert_allclose(mo, po, rtol=0, atol=1e-15)
    np.testing.assert_allclose(ml, pl, rtol=0, atol=1e-15)


def pin_rows_api(lib=None):
    d = 32
    b = make_batch([9, 30, 0, 4], [12, 64, 3, 40], 4, 2, d, seed=41)
    fo, fl = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2, True, SM,
                                     lib=lib)
    rng = np.random.default_rng(0)
    toks = rng.integers(0, int(b.q_indptr[-1]), 25)
    heads = rng.integers(0, 4, 25)
    ro, rl = oracle.ragged_attention_rows(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2, True, SM,
                                          toks, heads, lib=lib)
    assert np.array_equal(ro, fo[toks, heads]) and np.array_equal(rl, fl[toks, heads])


ALL_PINS = [
    pin_library_noncausal,
    pin_library_causal_square,
    pin_library_causal_bottom_right,
    pin_library_mha_hd128,
    pin_closed_forms,
    pin_invariants,
    pin_merge,
    pin_merge_states,
    pin_rows_api,
]
