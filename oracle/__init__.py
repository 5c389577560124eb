"""Q2_0 CPU oracle (fp64) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (``ternary_bit_quantized_amd``)
never does and shares no code with it.

The arithmetic lives in ``q2_0_oracle.c`` (plain C loops, fp64, OpenMP only
across output rows).  This module builds it with gcc on first use and wraps it
with ctypes; the wrappers only marshal arguments.

Sources: bisque.today "WebGPU: add Q2_0 support" (the block-format and mat-vec
paragraphs) and aisvetem.cz "Llama.cpp umi dvoubitovy Q2_0 i na kartach NVIDIA"
(sections "Osmnact bajtu na ctyriasedesat vah" and "Na bezny model to neni").
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q2_0_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_q2_0.so")

BLOCK_WEIGHTS = 64
BLOCK_BYTES = 18


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no intrinsics)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_double_to_half.argtypes = [ctypes.c_double]
        L.oracle_double_to_half.restype = ctypes.c_uint16
        L.oracle_dequant_row.argtypes = [P, I64, I64, P]
        L.oracle_get_rows.argtypes = [P, I64, I64, P, I64, P, I64]
        L.oracle_mul_mat_rows.argtypes = [P, I64, I64, P, I64, I64, P, I64, P, P, I64]
        L.oracle_quantize_ref.argtypes = [P, I64, I64, P]
        L.oracle_dequant_g128_row.argtypes = [P, I64, I64, P]
        L.oracle_repack_g128.argtypes = [P, I64, I64, P]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        for f in (L.oracle_dequant_row, L.oracle_get_rows, L.oracle_mul_mat_rows,
                  L.oracle_quantize_ref, L.oracle_set_num_threads, L.oracle_dequant_g128_row,
                  L.oracle_repack_g128):
            f.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_w(w: np.ndarray, M: int, K: int) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.uint8)
    assert K % BLOCK_WEIGHTS == 0 and w.size == M * (K // BLOCK_WEIGHTS) * BLOCK_BYTES
    return w


def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(int(bits) & 0xFFFF)


def double_to_half(x: float) -> int:
    return int(lib().oracle_double_to_half(float(x)))


def dequant(w: np.ndarray, M: int, K: int) -> np.ndarray:
    """Dense fp64 (M, K) matrix of (q - 1) * d."""
    w = _check_w(w, M, K)
    out = np.empty((M, K), dtype=np.float64)
    for m in range(M):
        lib().oracle_dequant_row(_p(w), K, m, _p(out[m]))
    return out


def get_rows(w: np.ndarray, M: int, K: int, ids: np.ndarray, ld_out: int | None = None) -> np.ndarray:
    """(n_ids, ld_out) float32; columns >= K are left as written (NaN-free zeros)."""
    w = _check_w(w, M, K)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    ld = K if ld_out is None else ld_out
    out = np.zeros((ids.size, ld), dtype=np.float32)
    if ids.size:
        lib().oracle_get_rows(_p(w), M, K, _p(ids), ids.size, _p(out), ld)
    return out


def mul_mat(w: np.ndarray, M: int, K: int, x: np.ndarray, rows: np.ndarray | None = None):
    """x: (N, K) float32 -> (y, bound), each (N, M) fp64 (or (N, len(rows)) for a row subset).

    y[n, m] = sum_b d * sum_i (q - 1) * x[n, 64b + i];  bound = same with absolute values.
    """
    w = _check_w(w, M, K)
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.ndim == 2 and x.shape[1] == K
    N = x.shape[0]
    if rows is None:
        cnt, rp = M, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < M)
        cnt, rp = rows.size, _p(rows)
    y = np.zeros((N, cnt), dtype=np.float64)
    b = np.zeros((N, cnt), dtype=np.float64)
    if N and cnt:
        lib().oracle_mul_mat_rows(_p(w), M, K, _p(x), K, N, rp, cnt if rows is not None else 0,
                                  _p(y), _p(b), cnt)
    return y, b


def quantize_ref(wf: np.ndarray) -> np.ndarray:
    """f32 weights (M, K) -> packed Q2_0 (M, K/64*18) uint8 by the reference quantizer."""
    wf = np.ascontiguousarray(wf, dtype=np.float32)
    M, K = wf.shape
    assert K % BLOCK_WEIGHTS == 0
    out = np.zeros((M, K // BLOCK_WEIGHTS * BLOCK_BYTES), dtype=np.uint8)
    lib().oracle_quantize_ref(_p(wf), M, K, _p(out))
    return out


def dequant_g128(w128: np.ndarray, M: int, K: int) -> np.ndarray:
    """Legacy group-128 matrix (M rows of K/128 34-byte blocks) -> dense fp64 (M, K)."""
    w128 = np.ascontiguousarray(w128, dtype=np.uint8)
    assert K % 128 == 0 and w128.size == M * (K // 128) * 34
    out = np.zeros((M, K), dtype=np.float64)
    for m in range(M):
        lib().oracle_dequant_g128_row(_p(w128), K, m, _p(out[m]))
    return out


def repack_g128(w128: np.ndarray, M: int, K: int) -> np.ndarray:
    """Legacy group-128 matrix -> Q2_0 group 64 (M, K/64*18) uint8."""
    w128 = np.ascontiguousarray(w128, dtype=np.uint8)
    assert K % 128 == 0 and w128.size == M * (K // 128) * 34
    out = np.zeros((M, K // BLOCK_WEIGHTS * BLOCK_BYTES), dtype=np.uint8)
    lib().oracle_repack_g128(_p(w128), M, K, _p(out))
    return out


def mul_mat_id(w: np.ndarray, n_expert: int, M: int, K: int, x: np.ndarray, ids: np.ndarray):
    """Expert product, by its definition: pair (t, u) is W_{ids[t, u]} times activation
    x[t * x_slots + u % x_slots] (x_slots = x rows / n_tokens, 1 or n_used).  Returns
    (y, bound) of shape (n_tokens * n_used, M), pair order; pairs with an id outside
    [0, n_expert) get NaN in y and 0 in bound."""
    ids = np.asarray(ids)
    n_tokens, n_used = ids.shape
    x = np.asarray(x, dtype=np.float32)
    x_slots = x.shape[0] // n_tokens
    assert x_slots in (1, n_used) and x.shape[0] == n_tokens * x_slots
    eb = M * (K // BLOCK_WEIGHTS) * BLOCK_BYTES
    wall = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    assert wall.size == n_expert * eb
    y = np.full((n_tokens * n_used, M), np.nan)
    bound = np.zeros((n_tokens * n_used, M))
    pairs = np.arange(n_tokens * n_used)
    flat = ids.reshape(-1)
    for e in range(n_expert):
        sel = pairs[flat == e]
        if sel.size == 0:
            continue
        cols = (sel // n_used) if x_slots == 1 else sel
        ye, be = mul_mat(wall[e * eb:(e + 1) * eb], M, K, x[cols])
        y[sel] = ye
        bound[sel] = be
    return y, bound


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def check_products(y: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, rel: float) -> dict:
    """Acceptance rule for products: |y - y_ref| <= rel * bound elementwise; a non-finite y
    fails where y_ref is finite; bound == 0 demands y exactly 0.  Returns a summary."""
    y = np.asarray(y, dtype=np.float64)
    finite_ref = np.isfinite(y_ref)
    err = np.abs(y - y_ref)
    bad_nonfinite = finite_ref & ~np.isfinite(y)
    bad_tol = finite_ref & np.isfinite(y) & (err > rel * bound)
    bad = bad_nonfinite | bad_tol
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1), np.where(err > 0, np.inf, 0))
    return {"ok": not bad.any(), "n_bad": int(bad.sum()), "n": int(y.size),
            "max_err_over_bound": float(np.nanmax(ratio[finite_ref])) if finite_ref.any() else 0.0,
            "first_bad": tuple(int(i) for i in np.argwhere(bad)[0]) if bad.any() else None}
