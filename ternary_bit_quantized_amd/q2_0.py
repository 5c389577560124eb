"""Python binding of libq2_0.so (ctypes).  Argument marshalling only.

Every computation happens in the HIP kernels behind the C ABI declared in
include/q2_0.h.  PyTorch supplies device memory and the current stream; there is
no fallback of any kind: if the library is missing or a call fails, an exception
is raised.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# Q2_0_LIB names another build of the library (the sanitized host-only build of
# ternary_bit_quantized_amd.build --sanitize, for the ABI tests); default: the in-tree one.
LIB_PATH = os.environ.get("Q2_0_LIB") or os.path.join(PKG, "libq2_0.so")

Q2_0_OK = 0
Q2_0_ERR_NULL = 1
Q2_0_ERR_SHAPE = 2
Q2_0_ERR_LAYOUT = 3
Q2_0_ERR_ALIGN = 4
Q2_0_ERR_UNSUPPORTED = 5
Q2_0_ERR_WORKSPACE = 6
Q2_0_ERR_HIP = 7
Q2_0_ERR_TOO_LARGE = 8
Q2_0_PREC_F16_MFMA = 0
Q2_0_PREC_F32 = 1
Q2_0_PREC_F32_MFMA = 2
Q2_0_ACT_F32 = 0
Q2_0_ACT_F16 = 1
Q2_0_ACT_BF16 = 2
BLOCK_WEIGHTS = 64
BLOCK_BYTES = 18
MAT_VEC_MAX_N = 8
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("q2_0_get_rows", "q2_0_mul_mat_vec", "q2_0_mul_mat_vec_group", "q2_0_mul_mat",
           "q2_0_mul_mat_workspace_bytes", "q2_0_mul_mat_group", "q2_0_mul_mat_group_workspace_bytes",
           "q2_0_mul_mat_vec_act", "q2_0_mul_mat_vec_group_act", "q2_0_mul_mat_act", "q2_0_mul_mat_group_act",
           "q2_0_quantize", "q2_0_repack_g128", "q2_0_mul_mat_id", "q2_0_mul_mat_id_workspace_bytes",
           "q2_0_mul_mat_noalloc", "q2_0_mul_mat_vec_batch", "q2_0_status_string", "q2_0_last_hip_error", "q2_0_version")


class MatVecItem(ctypes.Structure):
    """q2_0_mat_vec_item: one matrix of a grouped mat-vec."""
    _fields_ = [("w", ctypes.c_void_p), ("M", ctypes.c_int64), ("y", ctypes.c_void_p),
                ("ldy", ctypes.c_int64)]


class MatVecBatchItem(ctypes.Structure):
    """q2_0_mat_vec_batch_item: one product of a batched mat-vec (its own K and x)."""
    _fields_ = [("w", ctypes.c_void_p), ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("x", ctypes.c_void_p),
                ("ldx", ctypes.c_int64), ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


def make_batch_items(entries):
    """[(w_ptr, M, K, x_ptr, ldx, y_ptr, ldy), ...] -> a ctypes array for mul_mat_vec_batch_raw."""
    arr = (MatVecBatchItem * len(entries))()
    for i, e in enumerate(entries):
        arr[i] = MatVecBatchItem(*e)
    return arr


def make_items(entries):
    """[(w_ptr, M, y_ptr, ldy), ...] -> a ctypes array to pass to mul_mat_vec_group_raw."""
    arr = (MatVecItem * len(entries))()
    for i, (w, M, y, ldy) in enumerate(entries):
        arr[i] = MatVecItem(w, M, y, ldy)
    return arr


class Q2_0Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib().q2_0_status_string(status).decode()
        if status == Q2_0_ERR_HIP:
            msg += " (hipError %d)" % lib().q2_0_last_hip_error()
        super().__init__("%s: %s" % (what, msg))


_lib = None


def lib() -> ctypes.CDLL:
    """Load libq2_0.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libq2_0.so is not built (%s); run `python -m "
                               "ternary_bit_quantized_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.q2_0_get_rows.argtypes = [P, I64, I64, P, I64, P, I64, P]
        L.q2_0_mul_mat_vec.argtypes = [P, I64, I64, P, I64, I64, P, I64, P]
        L.q2_0_mul_mat_vec_group.argtypes = [P, I64, I64, P, I64, I64, P]
        L.q2_0_mul_mat_vec_group.restype = ctypes.c_int
        L.q2_0_mul_mat.argtypes = [P, I64, I64, P, I64, I64, P, I64, ctypes.c_int, P,
                                   ctypes.c_size_t, P]
        L.q2_0_mul_mat_workspace_bytes.argtypes = [I64, I64, I64, ctypes.c_int]
        L.q2_0_mul_mat_workspace_bytes.restype = ctypes.c_size_t
        L.q2_0_mul_mat_group.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, P, ctypes.c_size_t, P]
        L.q2_0_mul_mat_group.restype = ctypes.c_int
        L.q2_0_mul_mat_group_workspace_bytes.argtypes = [P, I64, I64, I64, ctypes.c_int]
        L.q2_0_mul_mat_group_workspace_bytes.restype = ctypes.c_size_t
        C = ctypes.c_int
        L.q2_0_mul_mat_vec_act.argtypes = [P, I64, I64, P, C, I64, I64, P, I64, P]
        L.q2_0_mul_mat_vec_group_act.argtypes = [P, I64, I64, P, C, I64, I64, P]
        L.q2_0_mul_mat_act.argtypes = [P, I64, I64, P, C, I64, I64, P, I64, C, P, ctypes.c_size_t, P]
        L.q2_0_mul_mat_group_act.argtypes = [P, I64, I64, P, C, I64, I64, C, P, ctypes.c_size_t, P]
        L.q2_0_quantize.argtypes = [P, I64, I64, I64, P, P]
        L.q2_0_mul_mat_id.argtypes = [P, I64, I64, I64, P, C, I64, I64, P, I64, I64, P, I64, C, P,
                                      ctypes.c_size_t, P]
        L.q2_0_mul_mat_id_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, C]
        L.q2_0_mul_mat_id_workspace_bytes.restype = ctypes.c_size_t
        L.q2_0_repack_g128.argtypes = [P, I64, I64, P, P]
        L.q2_0_mul_mat_vec_batch.argtypes = [P, I64, ctypes.c_int, I64, P]
        L.q2_0_mul_mat_vec_batch.restype = ctypes.c_int
        L.q2_0_mul_mat_noalloc.argtypes = [P, I64, I64, P, I64, I64, P, I64, ctypes.c_int, P]
        L.q2_0_mul_mat_noalloc.restype = ctypes.c_int
        for f in (L.q2_0_mul_mat_vec_act, L.q2_0_mul_mat_vec_group_act, L.q2_0_mul_mat_act,
                  L.q2_0_mul_mat_group_act, L.q2_0_quantize, L.q2_0_repack_g128, L.q2_0_mul_mat_id):
            f.restype = ctypes.c_int
        L.q2_0_status_string.argtypes = [ctypes.c_int]
        L.q2_0_status_string.restype = ctypes.c_char_p
        L.q2_0_version.restype = ctypes.c_char_p
        for f in (L.q2_0_get_rows, L.q2_0_mul_mat_vec, L.q2_0_mul_mat, L.q2_0_last_hip_error):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != Q2_0_OK:
        raise Q2_0Error(status, what)


# ----------------------------------------------------------------------------- raw (pointers)

def _items_ptr(items):
    return ctypes.cast(items, ctypes.c_void_p) if items is not None else None


def get_rows_raw(w: int, M: int, K: int, ids: int, n_ids: int, out: int, ld_out: int,
                 stream: int = 0) -> int:
    return lib().q2_0_get_rows(w, M, K, ids, n_ids, out, ld_out, stream)


def mul_mat_vec_raw(w: int, M: int, K: int, x: int, ldx: int, N: int, y: int, ldy: int,
                    stream: int = 0) -> int:
    return lib().q2_0_mul_mat_vec(w, M, K, x, ldx, N, y, ldy, stream)


def mul_mat_vec_group_raw(items, n_items: int, K: int, x: int, ldx: int, N: int,
                          stream: int = 0) -> int:
    """items: a ctypes array from make_items (or None with n_items == 0)."""
    return lib().q2_0_mul_mat_vec_group(ctypes.cast(items, ctypes.c_void_p) if items is not None else None,
                                        n_items, K, x, ldx, N, stream)


def mul_mat_vec_batch_raw(items, n_items: int, x_type: int, N: int, stream: int = 0) -> int:
    """items: a ctypes array from make_batch_items (or None with n_items == 0)."""
    return lib().q2_0_mul_mat_vec_batch(_items_ptr(items), n_items, x_type, N, stream)


def mul_mat_raw(w: int, M: int, K: int, x: int, ldx: int, N: int, y: int, ldy: int, precision: int,
                workspace: int, ws_bytes: int, stream: int = 0) -> int:
    return lib().q2_0_mul_mat(w, M, K, x, ldx, N, y, ldy, precision, workspace, ws_bytes, stream)


def mul_mat_noalloc_raw(w: int, M: int, K: int, x: int, ldx: int, N: int, y: int, ldy: int, precision: int,
                        stream: int = 0) -> int:
    return lib().q2_0_mul_mat_noalloc(w, M, K, x, ldx, N, y, ldy, precision, stream)


def mul_mat_workspace_bytes(M: int, K: int, N: int, precision: int) -> int:
    return int(lib().q2_0_mul_mat_workspace_bytes(M, K, N, precision))


def mul_mat_group_raw(items, n_items: int, K: int, x: int, ldx: int, N: int, precision: int,
                      workspace: int, ws_bytes: int, stream: int = 0) -> int:
    """items: a ctypes array from make_items (or None with n_items == 0)."""
    return lib().q2_0_mul_mat_group(_items_ptr(items), n_items, K, x, ldx, N, precision, workspace, ws_bytes,
                                    stream)


def mul_mat_group_workspace_bytes(items, n_items: int, K: int, N: int, precision: int) -> int:
    return int(lib().q2_0_mul_mat_group_workspace_bytes(_items_ptr(items), n_items, K, N, precision))


def mul_mat_vec_act_raw(w: int, M: int, K: int, x: int, x_type: int, ldx: int, N: int, y: int, ldy: int,
                        stream: int = 0) -> int:
    return lib().q2_0_mul_mat_vec_act(w, M, K, x, x_type, ldx, N, y, ldy, stream)


def mul_mat_vec_group_act_raw(items, n_items: int, K: int, x: int, x_type: int, ldx: int, N: int,
                              stream: int = 0) -> int:
    return lib().q2_0_mul_mat_vec_group_act(_items_ptr(items), n_items, K, x, x_type, ldx, N, stream)


def mul_mat_act_raw(w: int, M: int, K: int, x: int, x_type: int, ldx: int, N: int, y: int, ldy: int,
                    precision: int, workspace: int, ws_bytes: int, stream: int = 0) -> int:
    return lib().q2_0_mul_mat_act(w, M, K, x, x_type, ldx, N, y, ldy, precision, workspace, ws_bytes, stream)


def mul_mat_group_act_raw(items, n_items: int, K: int, x: int, x_type: int, ldx: int, N: int, precision: int,
                          workspace: int, ws_bytes: int, stream: int = 0) -> int:
    return lib().q2_0_mul_mat_group_act(_items_ptr(items), n_items, K, x, x_type, ldx, N, precision,
                                        workspace, ws_bytes, stream)


def mul_mat_id_raw(w: int, n_expert: int, M: int, K: int, x: int, x_type: int, ldx: int, x_slots: int,
                   ids: int, n_used: int, n_tokens: int, y: int, ldy: int, precision: int, workspace: int,
                   ws_bytes: int, stream: int = 0) -> int:
    return lib().q2_0_mul_mat_id(w, n_expert, M, K, x, x_type, ldx, x_slots, ids, n_used, n_tokens, y, ldy,
                                 precision, workspace, ws_bytes, stream)


def mul_mat_id_workspace_bytes(n_expert: int, M: int, K: int, n_used: int, n_tokens: int, precision: int) -> int:
    return int(lib().q2_0_mul_mat_id_workspace_bytes(n_expert, M, K, n_used, n_tokens, precision))


def quantize_raw(src: int, M: int, K: int, ld_src: int, w: int, stream: int = 0) -> int:
    return lib().q2_0_quantize(src, M, K, ld_src, w, stream)


def repack_g128_raw(w128: int, M: int, K: int, w: int, stream: int = 0) -> int:
    return lib().q2_0_repack_g128(w128, M, K, w, stream)


def version() -> str:
    return lib().q2_0_version().decode()


# ----------------------------------------------------------------------------- torch tensors

def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _cols(t, K, name):
    """A (N, >=K) float32 device tensor with unit column stride -> (ptr, N, ld)."""
    import torch
    if t.dtype != torch.float32 or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("%s must be a 2-D float32 CUDA tensor with unit inner stride" % name)
    if t.shape[1] < K:
        raise ValueError("%s must have at least %d columns" % (name, K))
    ld = t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])
    return t.data_ptr(), t.shape[0], ld


def _xcols(t, K, name):
    """An activation tensor (N, >=K) of float32, float16 or bfloat16 with unit inner stride
    -> (ptr, N, ld, x_type)."""
    import torch
    types = {torch.float32: Q2_0_ACT_F32, torch.float16: Q2_0_ACT_F16, torch.bfloat16: Q2_0_ACT_BF16}
    if t.dtype not in types or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("%s must be a 2-D float32/float16/bfloat16 CUDA tensor with unit inner stride" % name)
    if t.shape[1] < K:
        raise ValueError("%s must have at least %d columns" % (name, K))
    ld = t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])
    return t.data_ptr(), t.shape[0], ld, types[t.dtype]


def q2_0_mul_mat_id(w, n_expert: int, M: int, K: int, x, ids, precision: int = Q2_0_PREC_F16_MFMA, y=None,
                    workspace=None, stream=None):
    """Expert product: w holds n_expert (M, K) Q2_0 matrices back to back; ids (n_tokens, n_used)
    int32 on the device; x (n_tokens * x_slots, K) with x_slots 1 or n_used.  Returns
    y (n_tokens * n_used, M) float32, row t * n_used + u = W_{ids[t, u]} x[t * x_slots + u % x_slots]."""
    import torch
    if ids.dtype != torch.int32 or not ids.is_contiguous() or ids.dim() != 2:
        raise ValueError("ids must be a contiguous 2-D int32 tensor")
    n_tokens, n_used = ids.shape
    xp, rows, ldx, xt = _xcols(x, K, "x")
    if rows != n_tokens and rows != n_tokens * n_used:
        raise ValueError("x must have n_tokens or n_tokens * n_used rows")
    x_slots = 1 if rows == n_tokens else n_used
    if y is None:
        y = torch.empty((n_tokens * n_used, M), dtype=torch.float32, device=x.device)
    yp, _, ldy = _cols(y, M, "y")
    need = mul_mat_id_workspace_bytes(n_expert, M, K, n_used, n_tokens, precision)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() * workspace.element_size()
    _check(mul_mat_id_raw(w.data_ptr(), n_expert, M, K, xp, xt, ldx, x_slots, ids.data_ptr(), n_used, n_tokens,
                          yp, ldy, precision, workspace.data_ptr(), wsb, _stream(stream)), "q2_0_mul_mat_id")
    return y


def q2_0_quantize(src, w=None, stream=None):
    """Q2_0 (uint8 device tensor (M, K/64*18)) of the float32 weights src (M, K) by the reference quantizer."""
    import torch
    M, K = src.shape
    ptr, _, ld = _cols(src, K, "src")
    if w is None:
        w = torch.empty((M, K // BLOCK_WEIGHTS * BLOCK_BYTES), dtype=torch.uint8, device=src.device)
    _check(quantize_raw(ptr, M, K, ld, w.data_ptr(), _stream(stream)), "q2_0_quantize")
    return w


def q2_0_repack_g128(w128, M: int, K: int, w=None, stream=None):
    """The group-64 Q2_0 tensor of a legacy group-128 tensor w128 (uint8, M rows of K/128*34 bytes)."""
    import torch
    if w is None:
        w = torch.empty((M, K // BLOCK_WEIGHTS * BLOCK_BYTES), dtype=torch.uint8, device=w128.device)
    _check(repack_g128_raw(w128.data_ptr(), M, K, w.data_ptr(), _stream(stream)), "q2_0_repack_g128")
    return w


def q2_0_get_rows(w, M: int, K: int, ids, out=None, stream=None):
    """out[r, :K] = dequantized row ids[r] of the (M, K) Q2_0 matrix w (uint8 device tensor)."""
    import torch
    n = ids.numel()
    if out is None:
        out = torch.empty((n, K), dtype=torch.float32, device=w.device)
    ptr, rows, ld = _cols(out, K, "out")
    if ids.dtype != torch.int32 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 tensor")
    _check(get_rows_raw(w.data_ptr(), M, K, ids.data_ptr(), n, ptr, ld, _stream(stream)),
           "q2_0_get_rows")
    return out


def q2_0_mul_mat_vec(w, M: int, K: int, x, y=None, stream=None):
    """y (N, M) = W x for x (N, K) of float32, float16 or bfloat16, N <= 8; y is float32."""
    import torch
    xp, N, ldx, xt = _xcols(x, K, "x")
    if y is None:
        y = torch.empty((N, M), dtype=torch.float32, device=x.device)
    yp, _, ldy = _cols(y, M, "y")
    _check(mul_mat_vec_act_raw(w.data_ptr(), M, K, xp, xt, ldx, N, yp, ldy, _stream(stream)),
           "q2_0_mul_mat_vec_act")
    return y


def q2_0_mul_mat_vec_group(mats, K: int, x, ys=None, stream=None):
    """mats: [(w, M), ...] sharing K; returns [y_i (N, M_i)] with y_i = W_i x (x float32, float16
    or bfloat16)."""
    import torch
    xp, N, ldx, xt = _xcols(x, K, "x")
    if ys is None:
        ys = [torch.empty((N, M), dtype=torch.float32, device=x.device) for (_, M) in mats]
    entries = []
    for (w, M), y in zip(mats, ys):
        yp, _, ldy = _cols(y, M, "y")
        entries.append((w.data_ptr(), M, yp, ldy))
    items = make_items(entries)
    _check(mul_mat_vec_group_act_raw(items, len(entries), K, xp, xt, ldx, N, _stream(stream)),
           "q2_0_mul_mat_vec_group_act")
    return ys


def q2_0_mul_mat_vec_batch(products, x_type_tensor=None, ys=None, stream=None):
    """products: [(w, M, K, x), ...] with x (N, >=K) device tensors of one dtype (float32,
    float16 or bfloat16) and the same N; returns [y_i (N, M_i) float32] with y_i = W_i x_i."""
    import torch
    entries, out = [], []
    xt0, N0 = None, None
    for i, (w, M, K, x) in enumerate(products):
        xp, N, ldx, xt = _xcols(x, K, "x")
        if xt0 is None:
            xt0, N0 = xt, N
        elif xt != xt0 or N != N0:
            raise ValueError("every x of a batch must have the same dtype and column count")
        y = ys[i] if ys is not None else torch.empty((N, M), dtype=torch.float32, device=x.device)
        yp, _, ldy = _cols(y, M, "y")
        entries.append((w.data_ptr(), M, K, xp, ldx, yp, ldy))
        out.append(y)
    items = make_batch_items(entries)
    _check(mul_mat_vec_batch_raw(items, len(entries), xt0 if xt0 is not None else Q2_0_ACT_F32, N0 or 0,
                                 _stream(stream)), "q2_0_mul_mat_vec_batch")
    return out


def q2_0_mul_mat(w, M: int, K: int, x, precision: int = Q2_0_PREC_F16_MFMA, y=None, workspace=None,
                 stream=None):
    """y (N, M) = W x for x (N, K) of float32, float16 or bfloat16, any N; y is float32."""
    import torch
    xp, N, ldx, xt = _xcols(x, K, "x")
    if y is None:
        y = torch.empty((N, M), dtype=torch.float32, device=x.device)
    yp, _, ldy = _cols(y, M, "y")
    need = mul_mat_workspace_bytes(M, K, N, precision)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsp = workspace.data_ptr() if workspace is not None else 0
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(mul_mat_act_raw(w.data_ptr(), M, K, xp, xt, ldx, N, yp, ldy, precision, wsp, wsb, _stream(stream)),
           "q2_0_mul_mat_act")
    return y


def q2_0_mul_mat_group(mats, K: int, x, precision: int = Q2_0_PREC_F16_MFMA, ys=None, workspace=None,
                       stream=None):
    """mats: [(w, M), ...] sharing K; returns [y_i (N, M_i)] with y_i = W_i x, any N (x float32,
    float16 or bfloat16)."""
    import torch
    xp, N, ldx, xt = _xcols(x, K, "x")
    if ys is None:
        ys = [torch.empty((N, M), dtype=torch.float32, device=x.device) for (_, M) in mats]
    entries = []
    for (w, M), y in zip(mats, ys):
        yp, _, ldy = _cols(y, M, "y")
        entries.append((w.data_ptr(), M, yp, ldy))
    items = make_items(entries)
    need = mul_mat_group_workspace_bytes(items, len(entries), K, N, precision)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsp = workspace.data_ptr() if workspace is not None else 0
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(mul_mat_group_act_raw(items, len(entries), K, xp, xt, ldx, N, precision, wsp, wsb, _stream(stream)),
           "q2_0_mul_mat_group_act")
    return ys
