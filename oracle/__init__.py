"""fp64 CPU oracle for ragged prefill attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library: the two share no code.

The arithmetic lives in ``ragged_attention.c`` (plain C, fp64, OpenMP over
independent rows); this module compiles it with gcc and marshals arguments.
See that file's header for the definition it computes and the passages it
follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ragged_attention.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")

_lock = threading.Lock()
_default = None


SOURCE = _SRC


def compile_source(src: str, out: str) -> str:
    """gcc -O2 with OpenMP; no fast-math and no fma contraction."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/_build/liboracle.so."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    return compile_source(_SRC, _LIB_PATH)


def _bind(lib):
    P = ctypes.c_void_p
    lib.oracle_ragged_attention.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_double, ctypes.c_int64, ctypes.c_int64]
    lib.oracle_ragged_attention.restype = ctypes.c_int
    lib.oracle_ragged_attention_rows.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_double, P, P, ctypes.c_int64, P, P]
    lib.oracle_ragged_attention_rows.restype = ctypes.c_int
    lib.oracle_merge_state.argtypes = [P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int]
    lib.oracle_merge_state.restype = None
    lib.oracle_merge_states.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    lib.oracle_merge_states.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    return lib


def _load():
    global _default
    with _lock:
        if _default is not None:
            return _default
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _default = _bind(ctypes.CDLL(_LIB_PATH))
        return _default


def load_library(path: str):
    """Bind another build of the oracle source (the mutation tests build
    deliberately broken copies to show the pins catch them)."""
    return _bind(ctypes.CDLL(path))


def _bits(x) -> np.ndarray:
    """bf16 tensor/array -> contiguous uint16 bit patterns (numpy)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.dtype != torch.bfloat16:
                raise TypeError("oracle inputs must be bfloat16")
            return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy()
                                        .view(np.uint16))
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns as uint16")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def ragged_attention(q, k, v, q_indptr: Sequence[int], kv_indptr: Sequence[int],
                     num_qo_heads: int, num_kv_heads: int, causal: bool, sm_scale: float,
                     key_window: Optional[Tuple[int, int]] = None,
                     fill: float = np.nan, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """O (fp64 [rows, Hq, D]) and LSE (fp64 [rows, Hq]) over the whole batch.

    Rows outside every request keep ``fill``.  ``key_window=(lo, hi)`` gives
    the partial state over request-relative keys ``lo <= j < hi`` (hi < 0: no
    upper bound).
    """
    lib = lib or _load()
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    rows, hq, d = qb.shape
    if hq != num_qo_heads or kb.shape[1] != num_kv_heads or kb.shape[2] != d or vb.shape != kb.shape:
        raise ValueError("shape mismatch")
    qi = np.ascontiguousarray(np.asarray(q_indptr, dtype=np.int32))
    ki = np.ascontiguousarray(np.asarray(kv_indptr, dtype=np.int32))
    batch = len(qi) - 1
    if batch > 0 and (qi[-1] > rows or ki[-1] > kb.shape[0]):
        raise ValueError("indptr exceeds the buffers")
    o = np.full((rows, hq, d), fill, dtype=np.float64)
    lse = np.full((rows, hq), fill, dtype=np.float64)
    lo, hi = key_window if key_window is not None else (0, -1)
    rc = lib.oracle_ragged_attention(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(o), _ptr(lse), _ptr(qi),
                                     _ptr(ki), batch, num_qo_heads, num_kv_heads, d,
                                     1 if causal else 0, float(sm_scale), int(lo), int(hi))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, lse


def paged_kv_gather(k_pages, v_pages, block_table, kv_lens: Sequence[int], page_size: int):
    """Contiguous K, V (bf16 bit patterns, [sum(kv_lens), Hkv, D]) and kv_indptr
    from a paged KV cache, by the definition of the paged layout: key j of
    request b is slot j % page_size of page block_table[b][j // page_size],
    table entries clamped to >= 0 (the block tables and page sizes of page
    "vllm-rlt PR #112", design notes; paged KV cache of page
    "flashinfer-ai/flashinfer", attention API).  Written key by key."""
    kb, vb = _bits(k_pages), _bits(v_pages)
    table = np.asarray(block_table, dtype=np.int64)
    lens = [int(x) for x in kv_lens]
    total = sum(lens)
    k = np.empty((total,) + kb.shape[2:], dtype=np.uint16)
    v = np.empty((total,) + vb.shape[2:], dtype=np.uint16)
    indptr = np.zeros(len(lens) + 1, dtype=np.int32)
    row = 0
    for b, n in enumerate(lens):
        indptr[b] = row
        for j in range(n):
            page = max(int(table[b, j // page_size]), 0)
            k[row] = kb[page, j % page_size]
            v[row] = vb[page, j % page_size]
            row += 1
    indptr[len(lens)] = row
    return k, v, indptr


def e4m3_to_f64(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (uint8), from the format's definition:
    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal (m x 2^-9); exponent 15 with mantissa 7 is NaN (no infinities),
    largest finite 448.  The FP8 K/V dtype of page "flashinfer-ai/flashinfer",
    benchmarks README, attention flags (--kv_dtype fp8_e4m3)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((b >> 7) != 0, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def fp8_kv_attention(q, k_fp8, v_fp8, k_scale: float, v_scale: float, q_indptr, kv_indptr,
                     num_qo_heads: int, num_kv_heads: int, causal: bool, sm_scale: float,
                     fill: float = np.nan) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over FP8 K/V (fp64, numpy): K = code x k_scale and
    V = code x v_scale are dequantised exactly, then for every request and
    qo head S = sm_scale Q K^T, the bottom-right causal mask, P = softmax(S),
    O = P V and LSE = log sum exp(S) over the visible keys (rows that see no
    key: O = 0, LSE = -inf).  Written independently of the C oracle."""
    qb = _bits(q)
    qf = (qb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kf = e4m3_to_f64(np.asarray(k_fp8)) * float(k_scale)
    vf = e4m3_to_f64(np.asarray(v_fp8)) * float(v_scale)
    rows, hq, d = qf.shape
    g = num_qo_heads // num_kv_heads
    o = np.full((rows, hq, d), fill, dtype=np.float64)
    lse = np.full((rows, hq), fill, dtype=np.float64)
    qi = np.asarray(q_indptr, dtype=np.int64)
    ki = np.asarray(kv_indptr, dtype=np.int64)
    for b in range(len(qi) - 1):
        qo, kv = qi[b + 1] - qi[b], ki[b + 1] - ki[b]
        if qo == 0:
            continue
        i = np.arange(qo)[:, None]
        j = np.arange(kv)[None, :]
        visible = (j <= i + kv - qo) if causal else np.ones((qo, kv), dtype=bool)
        for h in range(hq):
            Q = qf[qi[b]:qi[b + 1], h, :]
            K = kf[ki[b]:ki[b + 1], h // g, :]
            V = vf[ki[b]:ki[b + 1], h // g, :]
            S = np.where(visible, sm_scale * (Q @ K.T), -np.inf)
            m = S.max(axis=1, initial=-np.inf)
            none = np.isneginf(m)
            msafe = np.where(none, 0.0, m)
            P = np.exp(S - msafe[:, None])
            lsum = P.sum(axis=1)
            out = (P @ V) / np.where(none, 1.0, lsum)[:, None]
            o[qi[b]:qi[b + 1], h, :] = np.where(none[:, None], 0.0, out)
            lse[qi[b]:qi[b + 1], h] = np.where(none, -np.inf, msafe + np.log(np.where(none, 1.0, lsum)))
    return o, lse


def ragged_attention_rows(q, k, v, q_indptr, kv_indptr, num_qo_heads: int, num_kv_heads: int,
                          causal: bool, sm_scale: float, tokens, heads, lib=None
                          ) -> Tuple[np.ndarray, np.ndarray]:
    """O/LSE of the chosen (token row, qo head) pairs only."""
    lib = lib or _load()
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    d = qb.shape[2]
    qi = np.ascontiguousarray(np.asarray(q_indptr, dtype=np.int32))
    ki = np.ascontiguousarray(np.asarray(kv_indptr, dtype=np.int32))
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    hd = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    if tok.shape != hd.shape:
        raise ValueError("tokens and heads differ in shape")
    n = tok.size
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_ragged_attention_rows(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(qi), _ptr(ki),
                                          len(qi) - 1, num_qo_heads, num_kv_heads, d,
                                          1 if causal else 0, float(sm_scale), _ptr(tok),
                                          _ptr(hd), n, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, lse


def merge_state(o_a, lse_a, o_b, lse_b, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Merge two attention states over disjoint key sets (fp64)."""
    lib = lib or _load()
    o_a = np.ascontiguousarray(o_a, dtype=np.float64)
    o_b = np.ascontiguousarray(o_b, dtype=np.float64)
    lse_a = np.ascontiguousarray(lse_a, dtype=np.float64)
    lse_b = np.ascontiguousarray(lse_b, dtype=np.float64)
    if o_a.shape != o_b.shape or lse_a.shape != lse_b.shape or o_a.shape[:-1] != lse_a.shape:
        raise ValueError("shape mismatch")
    d = o_a.shape[-1]
    n = int(np.prod(lse_a.shape))
    o = np.empty_like(o_a)
    lse = np.empty_like(lse_a)
    lib.oracle_merge_state(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse),
                           n, d)
    return o, lse


def merge_states(o, lse, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Merge k states per row over disjoint key sets (fp64): o [..., k, D],
    lse [..., k] -> o [..., D], lse [...].  Inputs are widened to fp64."""
    lib = lib or _load()
    o = np.ascontiguousarray(o, dtype=np.float64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    if o.shape[:-1] != lse.shape or o.ndim < 2:
        raise ValueError("shape mismatch")
    k, d = o.shape[-2], o.shape[-1]
    n = int(np.prod(lse.shape[:-1]))
    out = np.empty(lse.shape[:-1] + (d,), dtype=np.float64)
    out_lse = np.empty(lse.shape[:-1], dtype=np.float64)
    lib.oracle_merge_states(_ptr(o), _ptr(lse), _ptr(out), _ptr(out_lse), n, k, d)
    return out, out_lse


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))
