"""Seeded bf16 Q/K/V generation and ragged packing.

Every request ``r`` of a batch drawn with seed ``s`` takes its values from its
own stream ``numpy.random.default_rng([s, r])``: first Q ``[qo_len, Hq, D]``,
then K ``[kv_len, Hkv, D]``, then V ``[kv_len, Hkv, D]``, standard normal in
float32, rounded to bf16 (round-to-nearest-even).  A request therefore holds
the same values whatever batch it sits in, which the batch-composition tests
rely on.  ``request_ids`` lets a caller give a request the stream of another
position (used to rebuild a batch from a subset of requests).

No attention arithmetic happens here.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

from .configs import WorkloadConfig


@dataclass
class RaggedBatch:
    q: torch.Tensor            # bf16 [q_base + sum(qo), Hq, D] (CPU)
    k: torch.Tensor            # bf16 [kv_base + sum(kv), Hkv, D] (CPU)
    v: torch.Tensor            # bf16 [kv_base + sum(kv), Hkv, D] (CPU)
    q_indptr: np.ndarray       # int32 [batch + 1], starts at q_base
    kv_indptr: np.ndarray      # int32 [batch + 1], starts at kv_base
    qo_lens: List[int]
    kv_lens: List[int]
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    seed: int

    @property
    def batch(self) -> int:
        return len(self.qo_lens)


def _bf16(x: np.ndarray) -> torch.Tensor:
    # torch's float32 -> bfloat16 conversion rounds to nearest even
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def request_tensors(seed: int, request_id: int, qo_len: int, kv_len: int,
                    num_qo_heads: int, num_kv_heads: int, head_dim: int):
    """Q, K, V (bf16, CPU) of one request from its own stream."""
    rng = np.random.default_rng([seed, request_id])
    q = rng.standard_normal((qo_len, num_qo_heads, head_dim), dtype=np.float32)
    k = rng.standard_normal((kv_len, num_kv_heads, head_dim), dtype=np.float32)
    v = rng.standard_normal((kv_len, num_kv_heads, head_dim), dtype=np.float32)
    return _bf16(q), _bf16(k), _bf16(v)


def indptr_from_lens(lens: Sequence[int], base: int = 0) -> np.ndarray:
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[0] = base
    if len(lens):
        out[1:] = base + np.cumsum(np.asarray(lens, dtype=np.int64))
    if out[-1] > np.iinfo(np.int32).max:
        raise ValueError("ragged offsets overflow int32")
    return out.astype(np.int32)


def make_batch(qo_lens: Sequence[int], kv_lens: Sequence[int], num_qo_heads: int,
               num_kv_heads: int, head_dim: int, seed: int, *,
               request_ids: Optional[Sequence[int]] = None,
               q_base: int = 0, kv_base: int = 0) -> RaggedBatch:
    """Pack requests into NHD buffers with int32 offsets.

    ``q_base``/``kv_base`` leave leading rows that belong to no request (filled
    from the separate stream ``[seed, -1]``), so that ``indptr[0] != 0`` and
    rows outside every request can be exercised.
    """
    qo_lens = [int(x) for x in qo_lens]
    kv_lens = [int(x) for x in kv_lens]
    if len(qo_lens) != len(kv_lens):
        raise ValueError("qo_lens and kv_lens differ in length")
    if request_ids is None:
        request_ids = list(range(len(qo_lens)))
    qs, ks, vs = [], [], []
    if q_base or kv_base:
        rng = np.random.default_rng([seed, 2**31 - 1])
        qs.append(_bf16(rng.standard_normal((q_base, num_qo_heads, head_dim), dtype=np.float32)))
        ks.append(_bf16(rng.standard_normal((kv_base, num_kv_heads, head_dim), dtype=np.float32)))
        vs.append(_bf16(rng.standard_normal((kv_base, num_kv_heads, head_dim), dtype=np.float32)))
    for rid, nq, nk in zip(request_ids, qo_lens, kv_lens):
        q, k, v = request_tensors(seed, int(rid), nq, nk, num_qo_heads, num_kv_heads, head_dim)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    empty_q = torch.empty((0, num_qo_heads, head_dim), dtype=torch.bfloat16)
    empty_kv = torch.empty((0, num_kv_heads, head_dim), dtype=torch.bfloat16)
    return RaggedBatch(
        q=torch.cat(qs, 0) if qs else empty_q,
        k=torch.cat(ks, 0) if ks else empty_kv,
        v=torch.cat(vs, 0) if vs else empty_kv,
        q_indptr=indptr_from_lens(qo_lens, q_base),
        kv_indptr=indptr_from_lens(kv_lens, kv_base),
        qo_lens=qo_lens, kv_lens=kv_lens,
        num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        seed=seed)


def make_config_batch(cfg: WorkloadConfig) -> RaggedBatch:
    return make_batch(cfg.qo_lens, cfg.kv_lens, cfg.num_qo_heads, cfg.num_kv_heads,
                      cfg.head_dim, cfg.seed)


@dataclass
class PagedKV:
    """A batch's K/V scattered into a page pool (NHD pages)."""
    k_pages: torch.Tensor      # bf16 [num_pages, page_size, Hkv, D] (CPU)
    v_pages: torch.Tensor      # bf16 [num_pages, page_size, Hkv, D] (CPU)
    block_table: np.ndarray    # int32 [batch, max_blocks]
    page_size: int


def make_paged(batch: RaggedBatch, page_size: int, seed: int, spare_pages: int = 3,
               spare_columns: int = 2, k: Optional[torch.Tensor] = None,
               v: Optional[torch.Tensor] = None) -> PagedKV:
    """Scatter each request's keys into pages of ``page_size`` keys at random
    physical positions of a pool.

    Logical page p of request b (keys p*page_size ...) goes to physical page
    ``block_table[b, p]``.  Slots past a request's last key hold NaN, and the
    pool has ``spare_pages`` pages no request uses (NaN as well).  Table
    columns past a request's pages hold padding: -1, 0 or a stale id of
    another page, drawn at random.  None of this padding may change a result.
    ``k``/``v`` replace the batch's K/V (e.g. uint8 FP8 E4M3 codes of the same
    shape); unused slots then hold the E4M3 NaN code 0x7f.
    """
    rng = np.random.default_rng([seed, 7919, page_size])
    kv_lens = np.diff(batch.kv_indptr).astype(np.int64)
    need = (kv_lens + page_size - 1) // page_size
    n_pages = int(need.sum()) + spare_pages
    perm = rng.permutation(n_pages)
    hkv, d = batch.num_kv_heads, batch.head_dim
    src_k = batch.k if k is None else k
    src_v = batch.v if v is None else v
    fill = float("nan") if src_k.dtype == torch.bfloat16 else 0x7F
    kp = torch.full((max(n_pages, 1), page_size, hkv, d), fill, dtype=src_k.dtype)
    vp = torch.full((max(n_pages, 1), page_size, hkv, d), fill, dtype=src_v.dtype)
    max_blocks = int(need.max() if len(need) else 0) + spare_columns
    table = np.zeros((batch.batch, max(max_blocks, 1)), dtype=np.int32)
    nxt = 0
    for b in range(batch.batch):
        base = int(batch.kv_indptr[b])
        for p in range(int(need[b])):
            phys = int(perm[nxt])
            nxt += 1
            table[b, p] = phys
            lo = p * page_size
            hi = min(lo + page_size, int(kv_lens[b]))
            kp[phys, : hi - lo] = src_k[base + lo: base + hi]
            vp[phys, : hi - lo] = src_v[base + lo: base + hi]
        pad = rng.integers(0, 3, table.shape[1] - int(need[b]))
        stale = rng.integers(0, max(n_pages, 1), pad.size)
        table[b, int(need[b]):] = np.where(pad == 0, -1, np.where(pad == 1, 0, stale))
    return PagedKV(k_pages=kp, v_pages=vp, block_table=table, page_size=page_size)


def make_fp8_kv(batch: RaggedBatch, k_scale: float, v_scale: float):
    """FP8 (OCP E4M3) codes of the batch's K and V: K / k_scale and V / v_scale
    rounded to the nearest E4M3 value (torch's float8_e4m3fn conversion),
    returned as uint8 tensors of the same shape (CPU)."""
    k8 = (batch.k.float() / k_scale).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (batch.v.float() / v_scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return k8, v8
