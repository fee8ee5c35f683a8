"""Ragged (varlen) batched prefill attention for MI355X (gfx950).

    O = softmax(sm_scale * Q K^T + causal mask) V   over N ragged requests in one launch,

BF16 with grouped-query heads, head_dim 128 or 256, causal selectable (bottom-right
aligned), with the per-row log-sum-exp.  The computation runs in the HIP library
``librp.so`` behind the C ABI of ``include/ragged_prefill.h``; this module only
marshals torch tensors (device memory and the current stream) into that ABI.

Entry points:
  ragged_prefill(q, k, v, q_indptr, kv_indptr, ...)  one-shot (plans are cached)
  Plan(q_indptr, kv_indptr, ...).run(q, k, v, ...)   plan once, run many
  Plan(...).run_paged(q, k_pages, v_pages, block_table, ...)   K/V in a paged cache
  Plan(...).run_fp8kv / run_paged_fp8kv(...)          FP8 (E4M3) K/V with per-tensor scales
  SharedPrefixPlan(q_indptr, kv_indptr, shared_kv_len, ...).run(q, k_shared, v_shared,
                   k_unique, v_unique, ...)            shared-prefix (cascade) attention
  merge_state / merge_state_in_place / merge_states    merging attention states (v, lse)
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import (RP_SPLIT_ALWAYS, RP_SPLIT_AUTO, RP_SPLIT_NEVER, RaggedPrefillError,
                   RpPlanInfo, RpPlanOpts)

__all__ = [
    "available",
    "ragged_prefill",
    "Plan",
    "SharedPrefixPlan",
    "merge_state",
    "merge_state_in_place",
    "merge_states",
    "RaggedPrefillError",
    "RP_SPLIT_AUTO",
    "RP_SPLIT_NEVER",
    "RP_SPLIT_ALWAYS",
    "ITEM_FIELDS",
]

# field names of one worklist item (int32 x 16), see rp_internal.h
ITEM_FIELDS = ["q_tok0", "n_tok", "t0", "qo_len", "kv_row0", "kv_len", "kv_head", "key_begin",
               "key_end", "slot", "request", "chunk", "cost", "lim_first", "fold_keys",
               "reserved1"]


def available() -> bool:
    """True if the library is built and the current HIP device is a gfx950."""
    return bool(_lib.load().rp_available())


def _host_indptr(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu")  # device offsets are copied to the host (a sync)
            return np.ascontiguousarray(x.numpy().astype(np.int32, copy=False))
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.dtype.kind not in "iu":
        raise TypeError("indptr must hold integers")
    if a.size and (a.min() < np.iinfo(np.int32).min or a.max() > np.iinfo(np.int32).max):
        raise ValueError("indptr does not fit int32")
    return np.ascontiguousarray(a.astype(np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _stream_handle(stream) -> ctypes.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensor(t, name: str, rows_needed: int, heads: int, head_dim: int) -> None:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16")
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != head_dim:
        raise ValueError(f"{name} must have shape [rows, {heads}, {head_dim}], got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (packed NHD)")
    if t.shape[0] < rows_needed:
        raise ValueError(f"{name} has {t.shape[0]} rows but the offsets need {rows_needed}")


def _default_scale(head_dim: int) -> float:
    return float(np.float32(1.0 / math.sqrt(head_dim)))


class Plan:
    """A worklist for one batch shape: plan once, run many times.

    ``kv_chunk`` (keys, multiple of 64; 0 = library default) fixes where long
    KV is cut into partial states; ``split_mode`` only moves work between
    workgroups and never changes results.  ``host_only`` plans can be
    inspected (``items()``, ``info``) without a GPU.
    """

    def __init__(self, q_indptr, kv_indptr, num_qo_heads: int, num_kv_heads: int, head_dim: int,
                 causal: bool = True, kv_chunk: int = 0, split_mode: int = RP_SPLIT_AUTO,
                 host_only: bool = False, num_xcds: int = 0):
        lib = _lib.load()
        self._lib = lib
        self.q_indptr = _host_indptr(q_indptr)
        self.kv_indptr = _host_indptr(kv_indptr)
        if self.q_indptr.shape != self.kv_indptr.shape or self.q_indptr.ndim != 1 or self.q_indptr.size < 1:
            raise ValueError("q_indptr and kv_indptr must be 1-D with the same length >= 1")
        self.batch = int(self.q_indptr.size - 1)
        self.num_qo_heads = int(num_qo_heads)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.causal = bool(causal)
        opts = RpPlanOpts(int(kv_chunk), int(split_mode), 1 if host_only else 0, int(num_xcds))
        handle = ctypes.c_void_p()
        st = lib.rp_plan_create(_ptr(self.q_indptr), _ptr(self.kv_indptr), self.batch,
                                self.num_qo_heads, self.num_kv_heads, self.head_dim,
                                1 if self.causal else 0, ctypes.byref(opts), ctypes.byref(handle))
        _lib.check(st, "rp_plan_create")
        self._handle = handle
        self._workspaces = {}

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._handle is None:
            raise RuntimeError("plan has been closed")
        return self._handle

    @property
    def info(self) -> dict:
        inf = RpPlanInfo()
        _lib.check(self._lib.rp_plan_get_info(self.handle, ctypes.byref(inf)), "rp_plan_get_info")
        return {name: getattr(inf, name) for name, _ in RpPlanInfo._fields_}

    @property
    def workspace_bytes(self) -> int:
        return int(self._lib.rp_plan_workspace_bytes(self.handle))

    def _workspace_for(self, workspace, device, stream):
        """(pointer, bytes) of the workspace for one run: the caller's, or
        one the plan keeps per stream (torch allocates it for that stream), so
        that runs of one plan enqueued on different streams never share
        partial states."""
        import torch
        need = self.workspace_bytes
        if workspace is None and need > 0:
            s = torch.cuda.current_stream(device) if stream is None else stream
            ws = self._workspaces.get(s.cuda_stream)
            if ws is None or ws.numel() < need:
                with torch.cuda.stream(s):
                    ws = torch.empty(need, dtype=torch.uint8, device=device)
                self._workspaces[s.cuda_stream] = ws
            workspace = ws
        if workspace is None:
            return None, 0
        return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()

    def items(self) -> np.ndarray:
        n = self.info["num_items"]
        buf = np.zeros((n, _lib.RP_ITEM_INTS), dtype=np.int32)
        got = self._lib.rp_plan_copy_items(self.handle, _ptr(buf), n)
        if got < 0:
            _lib.check(int(got), "rp_plan_copy_items")
        return buf[:got]

    def run(self, q, k, v, out=None, lse=None, sm_scale: Optional[float] = None,
            return_lse: bool = True, workspace=None, stream=None):
        import torch
        rows_q = int(self.q_indptr[-1])
        rows_kv = int(self.kv_indptr[-1])
        _check_tensor(q, "q", rows_q, self.num_qo_heads, self.head_dim)
        _check_tensor(k, "k", rows_kv, self.num_kv_heads, self.head_dim)
        _check_tensor(v, "v", rows_kv, self.num_kv_heads, self.head_dim)
        if out is None:
            out = torch.empty_like(q)
        else:
            _check_tensor(out, "out", rows_q, self.num_qo_heads, self.head_dim)
        if lse is None and return_lse:
            lse = torch.empty((q.shape[0], self.num_qo_heads), dtype=torch.float32, device=q.device)
        if lse is not None:
            if (lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous()
                    or tuple(lse.shape[1:]) != (self.num_qo_heads,) or lse.shape[0] < rows_q):
                raise ValueError("lse must be a contiguous float32 [rows, num_qo_heads] GPU tensor")
        ws_ptr, ws_bytes = self._workspace_for(workspace, q.device, stream)
        scale = _default_scale(self.head_dim) if sm_scale is None else float(sm_scale)
        st = self._lib.rp_run(self.handle, ctypes.c_void_p(q.data_ptr()),
                              ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                              ctypes.c_void_p(out.data_ptr()),
                              ctypes.c_void_p(lse.data_ptr()) if lse is not None else None,
                              ctypes.c_float(scale), ws_ptr, ws_bytes, _stream_handle(stream))
        _lib.check(st, "rp_run")
        return out, lse

    def run_noalloc(self, q, k, v, out=None, lse=None, sm_scale: Optional[float] = None,
                    return_lse: bool = True, stream=None):
        """run() through rp_run_noalloc: the split-KV partial states live in
        the library's fixed device array (no workspace; out and lse are
        allocated here unless given)."""
        rows_q = int(self.q_indptr[-1])
        rows_kv = int(self.kv_indptr[-1])
        _check_tensor(q, "q", rows_q, self.num_qo_heads, self.head_dim)
        _check_tensor(k, "k", rows_kv, self.num_kv_heads, self.head_dim)
        _check_tensor(v, "v", rows_kv, self.num_kv_heads, self.head_dim)
        out, lse, _, _ = self._outputs(q, out, lse, return_lse, None, stream, need_workspace=False)
        scale = _default_scale(self.head_dim) if sm_scale is None else float(sm_scale)
        st = self._lib.rp_run_noalloc(self.handle, ctypes.c_void_p(q.data_ptr()),
                                      ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                      ctypes.c_void_p(out.data_ptr()),
                                      ctypes.c_void_p(lse.data_ptr()) if lse is not None else None,
                                      ctypes.c_float(scale), _stream_handle(stream))
        _lib.check(st, "rp_run_noalloc")
        return out, lse

    def _outputs(self, q, out, lse, return_lse, workspace, stream, need_workspace=True):
        import torch
        rows_q = int(self.q_indptr[-1])
        if out is None:
            out = torch.empty_like(q)
        else:
            _check_tensor(out, "out", rows_q, self.num_qo_heads, self.head_dim)
        if lse is None and return_lse:
            lse = torch.empty((q.shape[0], self.num_qo_heads), dtype=torch.float32, device=q.device)
        if lse is not None:
            _check_lse(lse, rows_q, self.num_qo_heads, q.device)
        if not need_workspace:
            return out, lse, None, 0
        ws_ptr, ws_bytes = self._workspace_for(workspace, q.device, stream)
        return out, lse, ws_ptr, ws_bytes

    def run_fp8kv(self, q, k_fp8, v_fp8, k_scale: float, v_scale: float, out=None, lse=None,
                  sm_scale: Optional[float] = None, return_lse: bool = True, workspace=None,
                  stream=None):
        """Run with FP8 (OCP E4M3) K/V: k_fp8, v_fp8 uint8 (or float8_e4m3fn)
        [rows_kv, num_kv_heads, head_dim] on the GPU, dequantised as code x
        k_scale / code x v_scale."""
        rows_q = int(self.q_indptr[-1])
        rows_kv = int(self.kv_indptr[-1])
        _check_tensor(q, "q", rows_q, self.num_qo_heads, self.head_dim)
        for name, t in (("k_fp8", k_fp8), ("v_fp8", v_fp8)):
            _check_fp8(t, name, rows_kv, self.num_kv_heads, self.head_dim, 3)
        out, lse, ws_ptr, ws_bytes = self._outputs(q, out, lse, return_lse, workspace, stream)
        scale = _default_scale(self.head_dim) if sm_scale is None else float(sm_scale)
        st = self._lib.rp_run_fp8kv(self.handle, ctypes.c_void_p(q.data_ptr()),
                                    ctypes.c_void_p(k_fp8.data_ptr()), ctypes.c_void_p(v_fp8.data_ptr()),
                                    ctypes.c_float(k_scale), ctypes.c_float(v_scale),
                                    ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(lse.data_ptr()) if lse is not None else None,
                                    ctypes.c_float(scale), ws_ptr, ws_bytes, _stream_handle(stream))
        _lib.check(st, "rp_run_fp8kv")
        return out, lse

    def run_paged_fp8kv(self, q, k_pages, v_pages, block_table, k_scale: float, v_scale: float,
                        out=None, lse=None, sm_scale: Optional[float] = None,
                        return_lse: bool = True, workspace=None, stream=None):
        """run_paged with FP8 (OCP E4M3) page pools [num_pages, page_size,
        num_kv_heads, head_dim] (uint8 or float8_e4m3fn)."""
        import torch
        rows_q = int(self.q_indptr[-1])
        _check_tensor(q, "q", rows_q, self.num_qo_heads, self.head_dim)
        for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
            _check_fp8(t, name, None, self.num_kv_heads, self.head_dim, 4)
        if k_pages.shape != v_pages.shape:
            raise ValueError("k_pages and v_pages must have the same shape")
        if (not isinstance(block_table, torch.Tensor) or block_table.device.type != "cuda"
                or block_table.dtype != torch.int32 or block_table.dim() != 2
                or block_table.shape[0] != self.batch or not block_table.is_contiguous()):
            raise ValueError(f"block_table must be a contiguous int32 [{self.batch}, max_blocks] GPU tensor")
        out, lse, ws_ptr, ws_bytes = self._outputs(q, out, lse, return_lse, workspace, stream)
        scale = _default_scale(self.head_dim) if sm_scale is None else float(sm_scale)
        st = self._lib.rp_run_paged_fp8kv(self.handle, ctypes.c_void_p(q.data_ptr()),
                                          ctypes.c_void_p(k_pages.data_ptr()),
                                          ctypes.c_void_p(v_pages.data_ptr()),
                                          ctypes.c_void_p(block_table.data_ptr()),
                                          int(block_table.shape[1]), int(k_pages.shape[1]),
                                          ctypes.c_float(k_scale), ctypes.c_float(v_scale),
                                          ctypes.c_void_p(out.data_ptr()),
                                          ctypes.c_void_p(lse.data_ptr()) if lse is not None else None,
                                          ctypes.c_float(scale), ws_ptr, ws_bytes, _stream_handle(stream))
        _lib.check(st, "rp_run_paged_fp8kv")
        return out, lse

    def run_paged(self, q, k_pages, v_pages, block_table, out=None, lse=None,
                  sm_scale: Optional[float] = None, return_lse: bool = True, workspace=None,
                  stream=None):
        """Run over paged K/V: k_pages, v_pages bf16 [num_pages, page_size,
        num_kv_heads, head_dim]; block_table int32 [batch, max_blocks] on the
        GPU (key j of request b: page block_table[b, j // page_size], slot
        j % page_size; negative entries read as page 0)."""
        import torch
        rows_q = int(self.q_indptr[-1])
        _check_tensor(q, "q", rows_q, self.num_qo_heads, self.head_dim)
        _check_pages(k_pages, v_pages, block_table, self.batch, self.num_kv_heads, self.head_dim)
        page_size = int(k_pages.shape[1])
        if out is None:
            out = torch.empty_like(q)
        else:
            _check_tensor(out, "out", rows_q, self.num_qo_heads, self.head_dim)
        if lse is None and return_lse:
            lse = torch.empty((q.shape[0], self.num_qo_heads), dtype=torch.float32, device=q.device)
        if lse is not None:
            if (lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous()
                    or tuple(lse.shape[1:]) != (self.num_qo_heads,) or lse.shape[0] < rows_q):
                raise ValueError("lse must be a contiguous float32 [rows, num_qo_heads] GPU tensor")
        ws_ptr, ws_bytes = self._workspace_for(workspace, q.device, stream)
        scale = _default_scale(self.head_dim) if sm_scale is None else float(sm_scale)
        st = self._lib.rp_run_paged(self.handle, ctypes.c_void_p(q.data_ptr()),
                                    ctypes.c_void_p(k_pages.data_ptr()),
                                    ctypes.c_void_p(v_pages.data_ptr()),
                                    ctypes.c_void_p(block_table.data_ptr()),
                                    int(block_table.shape[1]), page_size,
                                    ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(lse.data_ptr()) if lse is not None else None,
                                    ctypes.c_float(scale), ws_ptr, ws_bytes, _stream_handle(stream))
        _lib.check(st, "rp_run_paged")
        return out, lse

    def close(self) -> None:
        if self._handle is not None:
            self._lib.rp_plan_destroy(self._handle)
            self._handle = None
            self._workspaces = {}

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass


class SharedPrefixPlan(Plan):
    """Shared-prefix attention: every request attends to ``shared_kv_len``
    shared keys and then to its own keys ``kv_indptr[b]:kv_indptr[b+1]``
    (two levels plus a state merge, all in the library; see
    rp_plan_create_shared_prefix)."""

    def __init__(self, q_indptr, kv_indptr, shared_kv_len: int, num_qo_heads: int,
                 num_kv_heads: int, head_dim: int, causal: bool = True, kv_chunk: int = 0,
                 split_mode: int = RP_SPLIT_AUTO, host_only: bool = False, num_xcds: int = 0):
        lib = _lib.load()
        self._lib = lib
        self.q_indptr = _host_indptr(q_indptr)
        self.kv_indptr = _host_indptr(kv_indptr)
        if self.q_indptr.shape != self.kv_indptr.shape or self.q_indptr.ndim != 1 or self.q_indptr.size < 1:
            raise ValueError("q_indptr and kv_indptr must be 1-D with the same length >= 1")
        self.batch = int(self.q_indptr.size - 1)
        self.shared_kv_len = int(shared_kv_len)
        self.num_qo_heads = int(num_qo_heads)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.causal = bool(causal)
        opts = RpPlanOpts(int(kv_chunk), int(split_mode), 1 if host_only else 0, int(num_xcds))
        handle = ctypes.c_void_p()
        self._handle = None
        st = lib.rp_plan_create_shared_prefix(_ptr(self.q_indptr), _ptr(self.kv_indptr), self.batch,
                                              self.shared_kv_len, self.num_qo_heads,
                                              self.num_kv_heads, self.head_dim,
                                              1 if self.causal else 0, ctypes.byref(opts),
                                              ctypes.byref(handle))
        _lib.check(st, "rp_plan_create_shared_prefix")
        self._handle = handle
        self._workspaces = {}

    def run(self, q, k_shared, v_shared, k_unique, v_unique, out=None, lse=None,
            sm_scale: Optional[float] = None, return_lse: bool = True, workspace=None,
            stream=None):
        rows_q = int(self.q_indptr[-1])
        _check_tensor(q, "q", rows_q, self.num_qo_heads, self.head_dim)
        _check_tensor(k_shared, "k_shared", self.shared_kv_len, self.num_kv_heads, self.head_dim)
        _check_tensor(v_shared, "v_shared", self.shared_kv_len, self.num_kv_heads, self.head_dim)
        _check_tensor(k_unique, "k_unique", int(self.kv_indptr[-1]), self.num_kv_heads, self.head_dim)
        _check_tensor(v_unique, "v_unique", int(self.kv_indptr[-1]), self.num_kv_heads, self.head_dim)
        out, lse, ws_ptr, ws_bytes, scale = self._shared_outputs(q, out, lse, return_lse, workspace,
                                                                 sm_scale, stream)
        st = self._lib.rp_run_shared_prefix(
            self.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_shared.data_ptr()),
            ctypes.c_void_p(v_shared.data_ptr()), ctypes.c_void_p(k_unique.data_ptr()),
            ctypes.c_void_p(v_unique.data_ptr()), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(lse.data_ptr()) if lse is not None else None, ctypes.c_float(scale),
            ws_ptr, ws_bytes, _stream_handle(stream))
        _lib.check(st, "rp_run_shared_prefix")
        return out, lse

    def run_paged(self, q, k_shared, v_shared, k_pages, v_pages, block_table, out=None, lse=None,
                  sm_scale: Optional[float] = None, return_lse: bool = True, workspace=None,
                  stream=None):
        """run() with each request's own keys in a paged cache: k_pages,
        v_pages bf16 [num_pages, page_size, num_kv_heads, head_dim] and
        block_table int32 [batch, max_blocks] on the GPU, as for Plan.run_paged;
        the shared prefix stays contiguous."""
        rows_q = int(self.q_indptr[-1])
        _check_tensor(q, "q", rows_q, self.num_qo_heads, self.head_dim)
        _check_tensor(k_shared, "k_shared", self.shared_kv_len, self.num_kv_heads, self.head_dim)
        _check_tensor(v_shared, "v_shared", self.shared_kv_len, self.num_kv_heads, self.head_dim)
        _check_pages(k_pages, v_pages, block_table, self.batch, self.num_kv_heads, self.head_dim)
        out, lse, ws_ptr, ws_bytes, scale = self._shared_outputs(q, out, lse, return_lse, workspace,
                                                                 sm_scale, stream)
        st = self._lib.rp_run_shared_prefix_paged(
            self.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_shared.data_ptr()),
            ctypes.c_void_p(v_shared.data_ptr()), ctypes.c_void_p(k_pages.data_ptr()),
            ctypes.c_void_p(v_pages.data_ptr()), ctypes.c_void_p(block_table.data_ptr()),
            int(block_table.shape[1]), int(k_pages.shape[1]), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(lse.data_ptr()) if lse is not None else None, ctypes.c_float(scale),
            ws_ptr, ws_bytes, _stream_handle(stream))
        _lib.check(st, "rp_run_shared_prefix_paged")
        return out, lse

    def _shared_outputs(self, q, out, lse, return_lse, workspace, sm_scale, stream):
        import torch
        rows_q = int(self.q_indptr[-1])
        if out is None:
            out = torch.empty_like(q)
        else:
            _check_tensor(out, "out", rows_q, self.num_qo_heads, self.head_dim)
        if lse is None and return_lse:
            lse = torch.empty((q.shape[0], self.num_qo_heads), dtype=torch.float32, device=q.device)
        if lse is not None:
            _check_lse(lse, rows_q, self.num_qo_heads, q.device)
        ws_ptr, ws_bytes = self._workspace_for(workspace, q.device, stream)
        scale = _default_scale(self.head_dim) if sm_scale is None else float(sm_scale)
        return out, lse, ws_ptr, ws_bytes, scale


def _check_pages(k_pages, v_pages, block_table, batch: int, heads: int, head_dim: int) -> None:
    import torch
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be a bf16 GPU tensor")
        if t.dim() != 4 or t.shape[2] != heads or t.shape[3] != head_dim:
            raise ValueError(f"{name} must be [num_pages, page_size, {heads}, {head_dim}], "
                             f"got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k_pages.shape != v_pages.shape:
        raise ValueError("k_pages and v_pages must have the same shape")
    if (not isinstance(block_table, torch.Tensor) or block_table.device.type != "cuda"
            or block_table.dtype != torch.int32 or block_table.dim() != 2
            or block_table.shape[0] != batch or not block_table.is_contiguous()):
        raise ValueError(f"block_table must be a contiguous int32 [{batch}, max_blocks] GPU tensor")


def _check_fp8(t, name: str, rows_needed, heads: int, head_dim: int, ndim: int) -> None:
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"{name} must hold FP8 E4M3 codes (uint8 or float8_e4m3fn)")
    if t.dim() != ndim or t.shape[-2] != heads or t.shape[-1] != head_dim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [..., {heads}, {head_dim}] tensor of rank {ndim}")
    if rows_needed is not None and t.shape[0] < rows_needed:
        raise ValueError(f"{name} has {t.shape[0]} rows but the offsets need {rows_needed}")


def _check_lse(t, rows: int, heads: int, device, name: str = "lse") -> None:
    import torch
    if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != device
            or not t.is_contiguous() or t.dim() != 2 or t.shape[1] != heads or t.shape[0] < rows):
        raise ValueError(f"{name} must be a contiguous float32 [rows, {heads}] GPU tensor")


def _check_state(v, s, name: str):
    import torch
    if not isinstance(v, torch.Tensor) or v.device.type != "cuda" or v.dtype != torch.bfloat16:
        raise TypeError(f"{name}: v must be a bf16 GPU tensor")
    if v.dim() != 3 or not v.is_contiguous():
        raise ValueError(f"{name}: v must be a contiguous [rows, num_heads, head_dim] tensor")
    _check_lse(s, int(v.shape[0]), int(v.shape[1]), v.device, name=f"{name}: s")
    if s.shape[0] != v.shape[0]:
        raise ValueError(f"{name}: s must have {v.shape[0]} rows")


def merge_state(v_a, s_a, v_b, s_b, v_out=None, s_out=None, stream=None):
    """Merge two attention states over disjoint key sets: v bf16 [rows, H, D],
    s fp32 natural-log LSE [rows, H].  Returns (v, s)."""
    import torch
    lib = _lib.load()
    _check_state(v_a, s_a, "a")
    _check_state(v_b, s_b, "b")
    if v_a.shape != v_b.shape:
        raise ValueError("the two states differ in shape")
    if v_out is None:
        v_out = torch.empty_like(v_a)
    elif v_out.shape != v_a.shape or v_out.dtype != torch.bfloat16 or not v_out.is_contiguous():
        raise ValueError("v_out must be a contiguous bf16 tensor shaped like v_a")
    if s_out is None:
        s_out = torch.empty_like(s_a)
    else:
        _check_lse(s_out, int(v_a.shape[0]), int(v_a.shape[1]), v_a.device, "s_out")
    rows, h, d = (int(x) for x in v_a.shape)
    st = lib.rp_merge_state(ctypes.c_void_p(v_a.data_ptr()), ctypes.c_void_p(s_a.data_ptr()),
                            ctypes.c_void_p(v_b.data_ptr()), ctypes.c_void_p(s_b.data_ptr()),
                            ctypes.c_void_p(v_out.data_ptr()), ctypes.c_void_p(s_out.data_ptr()),
                            rows, h, d, _stream_handle(stream))
    _lib.check(st, "rp_merge_state")
    return v_out, s_out


def merge_state_in_place(v, s, v_other, s_other, stream=None):
    """(v, s) <- merge((v, s), (v_other, s_other))."""
    lib = _lib.load()
    _check_state(v, s, "v")
    _check_state(v_other, s_other, "other")
    if v.shape != v_other.shape:
        raise ValueError("the two states differ in shape")
    rows, h, d = (int(x) for x in v.shape)
    st = lib.rp_merge_state_in_place(ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                                     ctypes.c_void_p(v_other.data_ptr()),
                                     ctypes.c_void_p(s_other.data_ptr()), rows, h, d,
                                     _stream_handle(stream))
    _lib.check(st, "rp_merge_state_in_place")
    return v, s


def merge_states(v, s, v_out=None, s_out=None, stream=None):
    """Merge K states per row: v bf16 [rows, K, H, D], s fp32 [rows, K, H] ->
    (v bf16 [rows, H, D], s fp32 [rows, H])."""
    import torch
    lib = _lib.load()
    if not isinstance(v, torch.Tensor) or v.device.type != "cuda" or v.dtype != torch.bfloat16:
        raise TypeError("v must be a bf16 GPU tensor")
    if v.dim() != 4 or not v.is_contiguous():
        raise ValueError("v must be a contiguous [rows, num_states, num_heads, head_dim] tensor")
    rows, k, h, d = (int(x) for x in v.shape)
    if (not isinstance(s, torch.Tensor) or s.dtype != torch.float32 or s.device != v.device
            or not s.is_contiguous() or tuple(s.shape) != (rows, k, h)):
        raise ValueError("s must be a contiguous float32 [rows, num_states, num_heads] tensor")
    if v_out is None:
        v_out = torch.empty((rows, h, d), dtype=torch.bfloat16, device=v.device)
    elif tuple(v_out.shape) != (rows, h, d) or v_out.dtype != torch.bfloat16 or not v_out.is_contiguous():
        raise ValueError("v_out must be a contiguous bf16 [rows, num_heads, head_dim] tensor")
    if s_out is None:
        s_out = torch.empty((rows, h), dtype=torch.float32, device=v.device)
    else:
        _check_lse(s_out, rows, h, v.device, "s_out")
    st = lib.rp_merge_states(ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                             ctypes.c_void_p(v_out.data_ptr()), ctypes.c_void_p(s_out.data_ptr()),
                             rows, k, h, d, _stream_handle(stream))
    _lib.check(st, "rp_merge_states")
    return v_out, s_out


def ragged_prefill(q, k, v, q_indptr, kv_indptr, causal: bool = True,
                   sm_scale: Optional[float] = None, out=None, lse=None,
                   return_lse: bool = True, stream=None) -> Tuple[object, Optional[object]]:
    """One-shot ragged prefill: returns (O, LSE or None).

    q: bf16 [rows_q, Hq, D]; k, v: bf16 [rows_kv, Hkv, D] (contiguous, on the
    GPU); q_indptr, kv_indptr: int [batch + 1] offsets (host or device; device
    offsets are copied to the host).  sm_scale defaults to 1/sqrt(D).
    """
    import torch
    lib = _lib.load()
    qi = _host_indptr(q_indptr)
    ki = _host_indptr(kv_indptr)
    if qi.shape != ki.shape or qi.ndim != 1 or qi.size < 1:
        raise ValueError("q_indptr and kv_indptr must be 1-D with the same length >= 1")
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be [rows, heads, head_dim]")
    hq, d = int(q.shape[1]), int(q.shape[2])
    hkv = int(k.shape[1])
    batch = int(qi.size - 1)
    _check_tensor(q, "q", int(qi[-1]), hq, d)
    _check_tensor(k, "k", int(ki[-1]), hkv, d)
    _check_tensor(v, "v", int(ki[-1]), hkv, d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", int(qi[-1]), hq, d)
    if lse is None and return_lse:
        lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape[1:]) != (hq,) or lse.shape[0] < int(qi[-1])):
        raise ValueError("lse must be a contiguous float32 [rows, num_qo_heads] GPU tensor")
    scale = _default_scale(d) if sm_scale is None else float(sm_scale)
    st = lib.ragged_prefill_bf16(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                 ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                 ctypes.c_void_p(lse.data_ptr()) if lse is not None else None,
                                 _ptr(qi), _ptr(ki), batch, hq, hkv, d, 1 if causal else 0,
                                 ctypes.c_float(scale), _stream_handle(stream))
    _lib.check(st, "ragged_prefill_bf16")
    return out, lse
