"""Seeded synthetic inputs for ragged (varlen) prefill attention.

This package only draws random numbers and packs them; it performs none of the
attention arithmetic.  Both the fp64 oracle tests and the GPU path take their
inputs from here, so that the two sides see exactly the same bf16 values.

Layout (the packed "NHD" layout of the FlashInfer ragged prefill API, page
"flashinfer-ai/flashinfer" docs, attention API section): Q is
``[sum(qo_len), num_qo_heads, head_dim]``, K and V are
``[sum(kv_len), num_kv_heads, head_dim]``; request ``b`` owns rows
``q_indptr[b]:q_indptr[b+1]`` of Q and ``kv_indptr[b]:kv_indptr[b+1]`` of K/V.
"""

from .configs import CONFIGS, WorkloadConfig, get_config
from .gen import (PagedKV, RaggedBatch, make_batch, make_config_batch, make_fp8_kv, make_paged,
                  request_tensors)

__all__ = [
    "CONFIGS",
    "WorkloadConfig",
    "get_config",
    "RaggedBatch",
    "make_batch",
    "make_config_batch",
    "request_tensors",
    "PagedKV",
    "make_paged",
    "make_fp8_kv",
]
