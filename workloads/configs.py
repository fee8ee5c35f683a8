"""The synthetic ragged-prefill workloads, with their request lengths recorded.

The lengths were drawn once with ``numpy.random.default_rng(seed)`` by the
recipe written next to each entry and are stored here verbatim: NumPy does not
promise stable generator streams across versions, so these lists, not the
recipe, are authoritative.

Shapes follow the ragged prefill workloads of the FlashInfer benchmark suite
(page "flashinfer-ai/flashinfer", benchmarks README, attention flags: batch
size, qo/kv lengths, qo/kv head counts, head_dim) and the two head dims of the
Atlas ragged prefill FFI (page "Module flashinfer", functions
``ragged_prefill_bf16_hd128`` / ``ragged_prefill_bf16_hd256``).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    qo_lens: Sequence[int]
    kv_lens: Sequence[int]
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    causal: bool
    seed: int
    description: str = ""
    # extra causal settings the config is also run with (hd256 runs both)
    also_noncausal: bool = False

    @property
    def batch(self) -> int:
        return len(self.qo_lens)

    @property
    def total_q(self) -> int:
        return int(sum(self.qo_lens))

    @property
    def total_kv(self) -> int:
        return int(sum(self.kv_lens))


# recipe: fixed lengths [17, 64]
_TINY = [17, 64]

# recipe: rng = default_rng(2); rng.integers(128, 2049, 8)
_HD128 = [1736, 630, 337, 701, 922, 1692, 994, 304]

# recipe: rng = default_rng(3); rng.integers(512, 4097, 16)
_HD256 = [3421, 819, 1155, 1360, 1162, 3384, 3628, 2599,
          653, 849, 1702, 2064, 2739, 2229, 1461, 1084]

# recipe: rng = default_rng(4);
#   L = clip(rint(exp(ln 256 + 1.0 * rng.standard_normal(64))), 0, 8192)
#   then L[0] = L[17] = L[63] = 0 and L[1] = L[31] = L[62] = 1
# (log-normal with median 256; sigma = 1.0 is a reading, only the median and
#  the clip range are given)
_RAGGED = [0, 1, 1351, 495, 50, 255, 137, 297, 51, 326, 324, 1237, 351, 427, 58, 2435,
           38, 0, 184, 106, 133, 131, 374, 229, 1127, 41, 255, 105, 556, 31, 182, 1,
           58, 686, 306, 701, 668, 96, 115, 209, 541, 600, 126, 139, 115, 143, 202, 224,
           2005, 154, 192, 405, 99, 177, 259, 555, 69, 1009, 180, 303, 597, 496, 1, 0]

# recipe: rng = default_rng(5); kv = rng.integers(4096, 16385, 32);
#         qo = rng.integers(256, 1025, 32)   (drawn after kv, same generator)
_APPEND_KV = [12339, 13988, 4374, 14024, 9857, 10428, 11840, 7608, 16133, 4758, 7511,
              8807, 11115, 9115, 5706, 4652, 4108, 4695, 5924, 16374, 6442, 12112,
              13315, 6977, 7564, 9441, 7330, 16067, 6280, 15127, 13898, 14470]
_APPEND_QO = [344, 557, 738, 635, 768, 776, 765, 302, 993, 683, 950, 464, 534, 932, 399,
              305, 543, 778, 350, 925, 518, 430, 674, 944, 935, 926, 491, 270, 854, 800,
              848, 256]

# recipe: rng = default_rng(6); kv = rng.integers(1024, 16385, 64); qo = 1 each
_DECODE_KV = [7860, 9290, 8977, 6296, 15557, 6693, 11127, 6776, 7935, 16192, 3889, 10743,
              7582, 11382, 12632, 6092, 11350, 11468, 7966, 2912, 10509, 1818, 14632, 14083,
              14023, 1160, 15947, 16058, 10023, 13727, 12814, 13085, 3383, 1762, 5097, 4210,
              9446, 14078, 12514, 7667, 9371, 10662, 12844, 2902, 12979, 3886, 9853, 8662,
              14188, 12690, 3625, 9316, 1760, 2665, 8272, 14329, 4341, 3169, 15585, 7777,
              2848, 10038, 6050, 5926]

# recipe: rng = default_rng(7); kv = rng.integers(16384, 32769, 4); qo = 1 each
_DECODE_FEW_KV = [31866, 26626, 27594, 31084]

# recipe: rng = default_rng(8); p = rng.integers(512, 2049, 4) (prefill, qo = kv = p);
#         d = rng.integers(1024, 8193, 60) (decode, qo = 1, kv = d), drawn after p
_MIXED_PREFILL = [1617, 1014, 872, 2029]
_MIXED_DECODE = [2285, 3308, 5630, 6677, 5610, 7260, 1370, 3827, 5136, 4163, 3810, 3696, 1311,
                 1790, 4914, 4457, 7893, 2754, 7109, 2867, 2049, 2348, 3875, 2413, 7445, 6858,
                 6791, 4056, 1241, 2858, 4218, 5260, 4249, 5356, 3738, 5661, 1220, 7557, 4866,
                 2100, 6869, 3686, 7301, 3064, 7427, 1144, 4127, 2325, 4151, 3853, 8101, 3843,
                 6453, 5445, 3805, 4266, 1578, 5377, 3867, 2623]


CONFIGS: Dict[str, WorkloadConfig] = {
    "tiny": WorkloadConfig(
        name="tiny", qo_lens=_TINY, kv_lens=_TINY, num_qo_heads=4, num_kv_heads=2,
        head_dim=128, causal=True, seed=1,
        description="2 requests qo=kv={17,64}, 4/2 heads, hd128, causal"),
    "hd128_gqa_causal": WorkloadConfig(
        name="hd128_gqa_causal", qo_lens=_HD128, kv_lens=_HD128, num_qo_heads=32,
        num_kv_heads=8, head_dim=128, causal=True, seed=2,
        description="8 requests qo=kv~U[128,2048], 32/8 heads, hd128, causal"),
    "hd256_gqa": WorkloadConfig(
        name="hd256_gqa", qo_lens=_HD256, kv_lens=_HD256, num_qo_heads=16,
        num_kv_heads=4, head_dim=256, causal=True, seed=3, also_noncausal=True,
        description="16 requests qo=kv~U[512,4096], 16/4 heads, hd256, causal and non-causal"),
    "ragged64": WorkloadConfig(
        name="ragged64", qo_lens=_RAGGED, kv_lens=_RAGGED, num_qo_heads=32,
        num_kv_heads=8, head_dim=128, causal=True, seed=4,
        description="64 requests, log-normal lengths (median 256, clip [0,8192]) with 0/1-token "
                    "requests, 32/8 heads, hd128, causal"),
    "append_prefix": WorkloadConfig(
        name="append_prefix", qo_lens=_APPEND_QO, kv_lens=_APPEND_KV, num_qo_heads=64,
        num_kv_heads=8, head_dim=128, causal=True, seed=5,
        description="32 requests kv~U[4096,16384], qo~U[256,1024], causal aligned to the end "
                    "of each KV, 64/8 heads, hd128"),
    "decode64": WorkloadConfig(
        name="decode64", qo_lens=[1] * 64, kv_lens=_DECODE_KV, num_qo_heads=32,
        num_kv_heads=8, head_dim=128, causal=True, seed=6,
        description="64 decode requests (qo=1), kv~U[1024,16384], 32/8 heads, hd128"),
    "decode_few": WorkloadConfig(
        name="decode_few", qo_lens=[1] * 4, kv_lens=_DECODE_FEW_KV, num_qo_heads=32,
        num_kv_heads=8, head_dim=128, causal=True, seed=7,
        description="4 decode requests (qo=1), kv~U[16384,32768], 32/8 heads, hd128 "
                    "(low concurrency: needs split-KV)"),
    "mixed": WorkloadConfig(
        name="mixed", qo_lens=_MIXED_PREFILL + [1] * 60, kv_lens=_MIXED_PREFILL + _MIXED_DECODE,
        num_qo_heads=32, num_kv_heads=8, head_dim=128, causal=True, seed=8,
        description="4 prefill requests qo=kv~U[512,2048] and 60 decode requests (qo=1, "
                    "kv~U[1024,8192]) in one batch, 32/8 heads, hd128"),
}

CONFIG_ORDER: List[str] = ["tiny", "hd128_gqa_causal", "hd256_gqa", "ragged64", "append_prefix",
                           "decode64", "decode_few", "mixed"]


def get_config(name: str) -> WorkloadConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
