"""Pins of the FP8 (E4M3) K/V oracle (CPU).

* the E4M3 decoder against torch's float8_e4m3fn conversion for all 256
  codes, and hand-checked values of the format;
* attention over FP8 K/V with unit scales against the C oracle run on the
  same values as bf16 (every E4M3 value is a bf16 value): two independent
  implementations of the definition;
* the scales: v_scale scales O and leaves the LSE alone; k_scale acts as a
  factor of sm_scale.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_batch, make_fp8_kv


def test_e4m3_decoder_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    hand = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
            0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x80: -0.0}
    for c, x in hand.items():
        assert ours[c] == x and np.signbit(ours[c]) == np.signbit(x)
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


CASES = [
    ([9, 30, 4], [9, 64, 40], 4, 2, 32, True),
    ([9, 30, 4], [9, 64, 40], 4, 2, 32, False),
    ([5, 0, 12], [0, 7, 3], 8, 2, 16, True),       # kv = 0, qo = 0, qo > kv
    ([17], [50], 3, 1, 64, True),                    # g = 3
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_unit_scales_match_c_oracle(case):
    qo, kv, hq, hkv, d, causal = CASES[case]
    b = make_batch(qo, kv, hq, hkv, d, seed=70 + case, q_base=1)
    k8, v8 = make_fp8_kv(b, 1.0, 1.0)
    sm = 1.0 / np.sqrt(d)
    o, l = oracle.fp8_kv_attention(b.q, k8.numpy(), v8.numpy(), 1.0, 1.0, b.q_indptr, b.kv_indptr,
                                   hq, hkv, causal, sm)
    kb = k8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    vb = v8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    ro, rl = oracle.ragged_attention(b.q, kb, vb, b.q_indptr, b.kv_indptr, hq, hkv, causal, sm)
    live = ~np.isnan(ro[..., 0])
    assert np.array_equal(live, ~np.isnan(o[..., 0]))
    np.testing.assert_allclose(o[live], ro[live], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l[live], rl[live], rtol=0, atol=1e-12)


def test_scales():
    b = make_batch([12, 40], [30, 40], 4, 2, 32, seed=80)
    k8, v8 = make_fp8_kv(b, 0.25, 0.5)
    sm = 0.17
    o1, l1 = oracle.fp8_kv_attention(b.q, k8.numpy(), v8.numpy(), 0.25, 0.5, b.q_indptr, b.kv_indptr,
                                     4, 2, True, sm)
    o2, l2 = oracle.fp8_kv_attention(b.q, k8.numpy(), v8.numpy(), 0.25, 1.0, b.q_indptr, b.kv_indptr,
                                     4, 2, True, sm)
    assert np.array_equal(o1, o2 * 0.5) and np.array_equal(l1, l2)
    o3, l3 = oracle.fp8_kv_attention(b.q, k8.numpy(), v8.numpy(), 1.0, 0.5, b.q_indptr, b.kv_indptr,
                                     4, 2, True, sm * 0.25)
    np.testing.assert_allclose(o3, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, l1, rtol=0, atol=1e-12)
