"""Differential attention forward for MI355X (gfx950): Python binding of libdiffattn.so.

This module only marshals arguments (shapes, device pointers, the current HIP stream) into the C ABI declared in
include/diffattn.h; every step of the computation runs in the library's HIP kernels.  torch supplies device memory
and streams.  If the library has not been built, importing the binding's functions fails loudly: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdiffattn.so")

DIFFATTN_BF16 = 0
DIFFATTN_F32 = 1
STATUS = {0: "DIFFATTN_OK", -1: "DIFFATTN_ERR_NULL", -2: "DIFFATTN_ERR_SHAPE", -3: "DIFFATTN_ERR_UNSUPPORTED",
          -4: "DIFFATTN_ERR_ALIGN", -5: "DIFFATTN_ERR_LAYER", -6: "DIFFATTN_ERR_LAMBDA",
          -7: "DIFFATTN_ERR_WORKSPACE", -8: "DIFFATTN_ERR_ALIAS", -9: "DIFFATTN_ERR_HIP"}
EXPORTS = ["diffattn_fwd", "diffattn_fwd_heads", "diffattn_fwd_strided", "diffattn_fwd_split_workspace_bytes",
           "diffattn_fwd_split", "diffattn_decode", "diffattn_decode_heads",
           "diffattn_decode_workspace_bytes", "diffattn_decode_varlen_workspace_bytes", "diffattn_decode_varlen",
           "diffattn_decode_paged_workspace_bytes", "diffattn_decode_paged", "diffattn_decode_strided",
           "diffattn_train_saved_bytes", "diffattn_fwd_train", "diffattn_fwd_train_strided",
           "diffattn_bwd_workspace_bytes", "diffattn_bwd", "diffattn_bwd_strided", "diffattn_lambda_init",
           "diffattn_decode_noalloc", "diffattn_status_str",
           "diffattn_abi_version"]

_lib = None


class DiffAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_str(status)})")


def lib() -> ctypes.CDLL:
    """Load libdiffattn.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libdiffattn.so is not built ({LIB_PATH}); run differential_attention_fwd_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, c_int, c_float = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.diffattn_fwd.argtypes = [P, P, P, P, P, P, i64, i64, i64, c_int, c_int, c_float, c_int, c_int, P]
    L.diffattn_fwd.restype = c_int
    L.diffattn_decode.argtypes = [P, P, P, P, P, P, i64, i64, i64, c_int, c_int, c_float, c_int, c_int, P,
                                  ctypes.c_size_t, P]
    L.diffattn_decode.restype = c_int
    L.diffattn_decode_noalloc.argtypes = [P, P, P, P, P, P, i64, i64, i64, c_int, c_int, c_float, c_int, c_int, P]
    L.diffattn_decode_noalloc.restype = c_int
    L.diffattn_fwd_heads.argtypes = [P, P, P, P, P, P, i64, i64, i64, c_int, c_int, P, c_int, c_int, P]
    L.diffattn_fwd_heads.restype = c_int
    L.diffattn_decode_heads.argtypes = [P, P, P, P, P, P, i64, i64, i64, c_int, c_int, P, c_int, c_int, P,
                                        ctypes.c_size_t, P]
    L.diffattn_decode_heads.restype = c_int
    L.diffattn_fwd_strided.argtypes = [P, P, P, P, P, P, i64, i64, i64, c_int, c_int, c_float, P, c_int, c_int, P, P]
    L.diffattn_fwd_strided.restype = c_int
    L.diffattn_fwd_split_workspace_bytes.argtypes = [i64, i64, i64, c_int]
    L.diffattn_fwd_split_workspace_bytes.restype = ctypes.c_size_t
    L.diffattn_fwd_split.argtypes = [P, P, P, P, P, P, i64, i64, i64, c_int, c_int, c_float, P, c_int, c_int, P,
                                     ctypes.c_size_t, P]
    L.diffattn_fwd_split.restype = c_int
    L.diffattn_decode_varlen_workspace_bytes.argtypes = [i64, i64, i64, i64, c_int]
    L.diffattn_decode_varlen_workspace_bytes.restype = ctypes.c_size_t
    L.diffattn_decode_varlen.argtypes = [P, P, P, P, P, P, i64, i64, i64, i64, P, c_int, c_int, c_float, P, c_int, P,
                                         ctypes.c_size_t, P]
    L.diffattn_decode_varlen.restype = c_int
    L.diffattn_decode_strided.argtypes = [P, P, P, P, P, P, i64, i64, i64, i64, P, P, c_int, c_int, c_float, P, c_int,
                                          P, ctypes.c_size_t, P]
    L.diffattn_decode_strided.restype = c_int
    L.diffattn_decode_paged_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, c_int]
    L.diffattn_decode_paged_workspace_bytes.restype = ctypes.c_size_t
    L.diffattn_decode_paged.argtypes = [P, P, P, P, P, P, i64, i64, i64, P, i64, i64, i64, P, c_int, c_int, c_float, P,
                                        c_int, P, ctypes.c_size_t, P]
    L.diffattn_decode_paged.restype = c_int
    L.diffattn_train_saved_bytes.argtypes = [i64, i64, i64, c_int]
    L.diffattn_train_saved_bytes.restype = ctypes.c_size_t
    L.diffattn_bwd_workspace_bytes.argtypes = [i64, i64, i64, c_int]
    L.diffattn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.diffattn_fwd_train.argtypes = [P, P, P, P, P, P, i64, i64, i64, c_int, c_int, c_float, P, c_int, c_int, P,
                                     ctypes.c_size_t, P]
    L.diffattn_fwd_train.restype = c_int
    L.diffattn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, i64, i64, i64, c_int, c_int, c_float, P, c_int,
                               c_int, P, ctypes.c_size_t, P]
    L.diffattn_bwd.restype = c_int
    L.diffattn_fwd_train_strided.argtypes = [P, P, P, P, P, P, i64, i64, i64, c_int, c_int, c_float, P, c_int, c_int,
                                             P, P, ctypes.c_size_t, P]
    L.diffattn_fwd_train_strided.restype = c_int
    L.diffattn_bwd_strided.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, i64, i64, i64, c_int, c_int, c_float, P,
                                       c_int, c_int, P, P, ctypes.c_size_t, P]
    L.diffattn_bwd_strided.restype = c_int
    L.diffattn_decode_workspace_bytes.argtypes = [i64, i64, i64, c_int]
    L.diffattn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.diffattn_lambda_init.argtypes = [c_int]
    L.diffattn_lambda_init.restype = ctypes.c_double
    L.diffattn_status_str.argtypes = [c_int]
    L.diffattn_status_str.restype = ctypes.c_char_p
    L.diffattn_abi_version.restype = c_int
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().diffattn_status_str(int(status)).decode()


def diffattn_status_str(status: int) -> str:
    return status_str(status)


def diffattn_lambda_init(layer: int) -> float:
    return float(lib().diffattn_lambda_init(int(layer)))


def diffattn_abi_version() -> int:
    return int(lib().diffattn_abi_version())


def diffattn_decode_workspace_bytes(B: int, H: int, L: int, d: int) -> int:
    return int(lib().diffattn_decode_workspace_bytes(int(B), int(H), int(L), int(d)))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DIFFATTN_BF16
    if t.dtype == torch.float32:
        return DIFFATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream, device) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def _check_tensors(ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _lambda_heads(lam, H, device):
    """A per-head lambda tensor (H fp32 values on the GPU), or None when lam is a number."""
    import torch
    if not isinstance(lam, torch.Tensor):
        return None
    if lam.dtype != torch.float32 or lam.device != device or tuple(lam.shape) != (H,) or not lam.is_contiguous():
        raise ValueError(f"per-head lambda must be a contiguous float32 tensor of shape ({H},) on {device}")
    return lam


def diffattn_fwd_split_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().diffattn_fwd_split_workspace_bytes(int(B), int(H), int(N), int(d)))


def diffattn_fwd_split(q1, k1, q2, k2, v, lam, layer: int, causal: bool, out=None, workspace=None, stream=None):
    """Split-key prefill (bf16, d = 64, dense): diffattn_fwd's result up to rounding, for launches too small to fill
    the GPU.  lam: a number, or a float32 GPU tensor of shape (H,) holding one lambda per head.  `workspace`: a GPU
    tensor of at least diffattn_fwd_split_workspace_bytes(B, H, N, d) bytes (allocated here if None)."""
    import torch
    _check_tensors((q1, k1, q2, k2, v))
    B, H, N, d = q1.shape
    if out is None:
        out = torch.empty((B, H, N, 2 * d), dtype=q1.dtype, device=q1.device)
    _check_tensors((out,))
    for t, shp in ((k1, q1.shape), (q2, q1.shape), (k2, q1.shape), (v, (B, H, N, 2 * d)), (out, (B, H, N, 2 * d))):
        if tuple(t.shape) != tuple(shp) or t.dtype != q1.dtype:
            raise ValueError(f"shape/dtype mismatch: {tuple(t.shape)} {t.dtype}, expected {tuple(shp)} {q1.dtype}")
    need = diffattn_fwd_split_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    _check_tensors((workspace,))
    lam_f, lam_p = _lambda_args(lam, H, q1.device)
    st = lib().diffattn_fwd_split(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(),
                                  out.data_ptr(), B, H, N, d, _dtype_code(q1), lam_f, lam_p, int(layer),
                                  int(bool(causal)), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_fwd_split")
    return out


def diffattn_fwd(q1, k1, q2, k2, v, lam, layer: int, causal: bool, out=None, stream=None):
    """Prefill: q1,k1,q2,k2 [B][H][N][d], v [B][H][N][2d] -> out [B][H][N][2d] (same dtype), on `stream`.

    lam: a number, or a float32 GPU tensor of shape (H,) holding one lambda per head (diffattn_fwd_heads)."""
    import torch
    _check_tensors((q1, k1, q2, k2, v))
    B, H, N, d = q1.shape
    if out is None:
        out = torch.empty((B, H, N, 2 * d), dtype=q1.dtype, device=q1.device)
    _check_tensors((out,))
    for t, shp in ((k1, q1.shape), (q2, q1.shape), (k2, q1.shape), (v, (B, H, N, 2 * d)), (out, (B, H, N, 2 * d))):
        if tuple(t.shape) != tuple(shp) or t.dtype != q1.dtype:
            raise ValueError(f"shape/dtype mismatch: {tuple(t.shape)} {t.dtype}, expected {tuple(shp)} {q1.dtype}")
    lh = _lambda_heads(lam, H, q1.device)
    args = (q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
            _dtype_code(q1))
    tail = (int(layer), int(bool(causal)), _stream_handle(stream, q1.device))
    if lh is None:
        st, name = lib().diffattn_fwd(*args, float(lam), *tail), "diffattn_fwd"
    else:
        st, name = lib().diffattn_fwd_heads(*args, lh.data_ptr(), *tail), "diffattn_fwd_heads"
    if st != 0:
        raise DiffAttnError(st, name)
    return out


def diffattn_decode(q1, k1, q2, k2, v, lam, layer: int, causal: bool = True, out=None, workspace=None,
                    stream=None):
    """Decode: q1,q2 [B][H][d]; k1,k2 [B][H][L][d]; v [B][H][L][2d] -> out [B][H][2d], on `stream`.

    lam: a number, or a float32 GPU tensor of shape (H,) holding one lambda per head (diffattn_decode_heads)."""
    import torch
    _check_tensors((q1, k1, q2, k2, v))
    B, H, d = q1.shape
    L = k1.shape[2]
    if out is None:
        out = torch.empty((B, H, 2 * d), dtype=q1.dtype, device=q1.device)
    for t, shp in ((q2, (B, H, d)), (k1, (B, H, L, d)), (k2, (B, H, L, d)), (v, (B, H, L, 2 * d)),
                   (out, (B, H, 2 * d))):
        if tuple(t.shape) != tuple(shp) or t.dtype != q1.dtype:
            raise ValueError(f"shape/dtype mismatch: {tuple(t.shape)} {t.dtype}, expected {tuple(shp)} {q1.dtype}")
    need = diffattn_decode_workspace_bytes(B, H, L, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lh = _lambda_heads(lam, H, q1.device)
    args = (q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, L, d,
            _dtype_code(q1))
    tail = (int(layer), int(bool(causal)), ws_ptr, ws_bytes, _stream_handle(stream, q1.device))
    if lh is None:
        st, name = lib().diffattn_decode(*args, float(lam), *tail), "diffattn_decode"
    else:
        st, name = lib().diffattn_decode_heads(*args, lh.data_ptr(), *tail), "diffattn_decode_heads"
    if st != 0:
        raise DiffAttnError(st, name)
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20   # DIFFATTN_NOALLOC_SCRATCH_BYTES


def diffattn_decode_noalloc(q1, k1, q2, k2, v, lam: float, layer: int, causal: bool = True, out=None, stream=None):
    """Decode as diffattn_decode, with the split partials in the library's per-GPU scratch array: the call allocates
    nothing (pass `out` to keep the whole call allocation-free).  Calls that may overlap on one GPU race."""
    import torch
    _check_tensors((q1, k1, q2, k2, v))
    B, H, d = q1.shape
    L = k1.shape[2]
    if out is None:
        out = torch.empty((B, H, 2 * d), dtype=q1.dtype, device=q1.device)
    for t, shp in ((q2, (B, H, d)), (k1, (B, H, L, d)), (k2, (B, H, L, d)), (v, (B, H, L, 2 * d)),
                   (out, (B, H, 2 * d))):
        if tuple(t.shape) != tuple(shp) or t.dtype != q1.dtype:
            raise ValueError(f"shape/dtype mismatch: {tuple(t.shape)} {t.dtype}, expected {tuple(shp)} {q1.dtype}")
    st = lib().diffattn_decode_noalloc(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(),
                                       out.data_ptr(), B, H, L, d, _dtype_code(q1), float(lam), int(layer),
                                       int(bool(causal)), _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_decode_noalloc")
    return out


def diffattn_train_saved_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().diffattn_train_saved_bytes(int(B), int(H), int(N), int(d)))


def diffattn_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().diffattn_bwd_workspace_bytes(int(B), int(H), int(N), int(d)))


def _lambda_args(lam, H, device):
    lh = _lambda_heads(lam, H, device)
    return (0.0, lh.data_ptr()) if lh is not None else (float(lam), None)


def diffattn_fwd_train(q1, k1, q2, k2, v, lam, layer: int, causal: bool, out=None, saved=None, stream=None):
    """Training forward (bf16, d = 64): returns (out, saved); `saved` feeds diffattn_bwd."""
    import torch
    _check_tensors((q1, k1, q2, k2, v))
    B, H, N, d = q1.shape
    if out is None:
        out = torch.empty((B, H, N, 2 * d), dtype=q1.dtype, device=q1.device)
    if saved is None:
        saved = torch.empty(max(diffattn_train_saved_bytes(B, H, N, d), 16), dtype=torch.uint8, device=q1.device)
    _check_tensors((out, saved))
    for t, shp in ((k1, q1.shape), (q2, q1.shape), (k2, q1.shape), (v, (B, H, N, 2 * d)), (out, (B, H, N, 2 * d))):
        if tuple(t.shape) != tuple(shp) or t.dtype != q1.dtype:
            raise ValueError(f"shape/dtype mismatch: {tuple(t.shape)} {t.dtype}, expected {tuple(shp)} {q1.dtype}")
    lam_f, lam_p = _lambda_args(lam, H, q1.device)
    st = lib().diffattn_fwd_train(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(),
                                  out.data_ptr(), B, H, N, d, _dtype_code(q1), lam_f, lam_p, int(layer),
                                  int(bool(causal)), saved.data_ptr(), saved.numel() * saved.element_size(),
                                  _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_fwd_train")
    return out, saved


def diffattn_bwd(q1, k1, q2, k2, v, dy, saved, lam, layer: int, causal: bool, grads=None, workspace=None,
                 stream=None):
    """Backward (bf16, d = 64): returns a dict dq1, dk1, dq2, dk2, dv (bf16, shapes of the inputs) and dlambda
    (float32, one per head, summed over the batch)."""
    import torch
    _check_tensors((q1, k1, q2, k2, v, dy, saved))
    B, H, N, d = q1.shape
    if grads is None:
        grads = {k: torch.empty_like(t) for k, t in (("dq1", q1), ("dk1", k1), ("dq2", q2), ("dk2", k2), ("dv", v))}
        grads["dlambda"] = torch.empty(H, dtype=torch.float32, device=q1.device)
    _check_tensors(tuple(grads.values()))
    need = diffattn_bwd_workspace_bytes(B, H, N, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lam_f, lam_p = _lambda_args(lam, H, q1.device)
    g = grads
    st = lib().diffattn_bwd(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(), dy.data_ptr(),
                            saved.data_ptr(), g["dq1"].data_ptr(), g["dk1"].data_ptr(), g["dq2"].data_ptr(),
                            g["dk2"].data_ptr(), g["dv"].data_ptr(), g["dlambda"].data_ptr(), B, H, N, d,
                            _dtype_code(q1), lam_f, lam_p, int(layer), int(bool(causal)), ws_ptr, ws_bytes,
                            _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_bwd")
    return grads


def diffattn_decode_varlen_workspace_bytes(B: int, H: int, T: int, L: int, d: int) -> int:
    return int(lib().diffattn_decode_varlen_workspace_bytes(int(B), int(H), int(T), int(L), int(d)))


def diffattn_decode_varlen(q1, k1, q2, k2, v, lam, layer: int, lens=None, out=None, workspace=None, stream=None):
    """Variable-length / multi-token decode (bf16, d = 64): q1, q2 [B][H][T][d]; caches [B][H][L][d] and
    [B][H][L][2d]; lens: None or an int32 GPU tensor of B cache lengths.  Returns out [B][H][T][2d]."""
    import torch
    _check_tensors((q1, k1, q2, k2, v))
    B, H, T, d = q1.shape
    L = k1.shape[2]
    if out is None:
        out = torch.empty((B, H, T, 2 * d), dtype=q1.dtype, device=q1.device)
    for t, shp in ((q2, (B, H, T, d)), (k1, (B, H, L, d)), (k2, (B, H, L, d)), (v, (B, H, L, 2 * d)),
                   (out, (B, H, T, 2 * d))):
        if tuple(t.shape) != tuple(shp) or t.dtype != q1.dtype:
            raise ValueError(f"shape/dtype mismatch: {tuple(t.shape)} {t.dtype}, expected {tuple(shp)} {q1.dtype}")
    if lens is not None:
        if lens.dtype != torch.int32 or tuple(lens.shape) != (B,) or lens.device != q1.device:
            raise ValueError(f"lens must be an int32 tensor of shape ({B},) on {q1.device}")
        _check_tensors((lens,))
    need = diffattn_decode_varlen_workspace_bytes(B, H, T, L, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lam_f, lam_p = _lambda_args(lam, H, q1.device)
    st = lib().diffattn_decode_varlen(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(),
                                      out.data_ptr(), B, H, T, L, lens.data_ptr() if lens is not None else None, d,
                                      _dtype_code(q1), lam_f, lam_p, int(layer), ws_ptr, ws_bytes,
                                      _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_decode_varlen")
    return out


def diffattn_decode_paged_workspace_bytes(B: int, H: int, T: int, max_pages: int, page_size: int, d: int) -> int:
    return int(lib().diffattn_decode_paged_workspace_bytes(int(B), int(H), int(T), int(max_pages), int(page_size),
                                                           int(d)))


def diffattn_decode_paged(q1, k1_pages, q2, k2_pages, v_pages, block_table, lam, layer: int, lens=None, out=None,
                          workspace=None, stream=None):
    """Paged decode (bf16, d = 64): q1, q2 [B][H][T][d]; page pools k1/k2 [num_pages][H][page_size][d] and
    v [num_pages][H][page_size][2d]; block_table an int32 GPU tensor [B][max_pages] (logical row r of sequence b is
    row r % page_size of page block_table[b][r // page_size]); lens: None or an int32 GPU tensor of B cache lengths.
    Returns out [B][H][T][2d]."""
    import torch
    _check_tensors((q1, k1_pages, q2, k2_pages, v_pages, block_table))
    B, H, T, d = q1.shape
    num_pages, _, page_size, _ = k1_pages.shape
    max_pages = block_table.shape[1] if block_table.dim() == 2 else -1
    if out is None:
        out = torch.empty((B, H, T, 2 * d), dtype=q1.dtype, device=q1.device)
    for t, shp in ((q2, (B, H, T, d)), (k1_pages, (num_pages, H, page_size, d)),
                   (k2_pages, (num_pages, H, page_size, d)), (v_pages, (num_pages, H, page_size, 2 * d)),
                   (out, (B, H, T, 2 * d))):
        if tuple(t.shape) != tuple(shp) or t.dtype != q1.dtype:
            raise ValueError(f"shape/dtype mismatch: {tuple(t.shape)} {t.dtype}, expected {tuple(shp)} {q1.dtype}")
    if block_table.dtype != torch.int32 or tuple(block_table.shape) != (B, max_pages) or block_table.device != q1.device:
        raise ValueError(f"block_table must be an int32 tensor of shape ({B}, max_pages) on {q1.device}")
    if lens is not None:
        if lens.dtype != torch.int32 or tuple(lens.shape) != (B,) or lens.device != q1.device:
            raise ValueError(f"lens must be an int32 tensor of shape ({B},) on {q1.device}")
        _check_tensors((lens,))
    need = diffattn_decode_paged_workspace_bytes(B, H, T, max_pages, page_size, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lam_f, lam_p = _lambda_args(lam, H, q1.device)
    st = lib().diffattn_decode_paged(q1.data_ptr(), k1_pages.data_ptr(), q2.data_ptr(), k2_pages.data_ptr(),
                                     v_pages.data_ptr(), out.data_ptr(), B, H, T, block_table.data_ptr(), max_pages,
                                     page_size, num_pages, lens.data_ptr() if lens is not None else None, d,
                                     _dtype_code(q1), lam_f, lam_p, int(layer), ws_ptr, ws_bytes,
                                     _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_decode_paged")
    return out


def diffattn_decode_strided(q1, k1, q2, k2, v, lam, layer: int, lens=None, out=None, workspace=None, stream=None):
    """Decode (bf16, d = 64) with strided caches: k1, k2 [B][H][L][d] and v [B][H][L][2d] may be any GPU views whose
    last dimension is contiguous (e.g. permuted token-major caches, or slices of one packed buffer); q1, q2
    [B][H][T][d] and out are contiguous.  lens as for diffattn_decode_varlen.  Returns out [B][H][T][2d]."""
    import torch
    _check_tensors((q1, q2))
    B, H, T, d = q1.shape
    L = k1.shape[2]
    if out is None:
        out = torch.empty((B, H, T, 2 * d), dtype=q1.dtype, device=q1.device)
    _check_tensors((out,))
    if tuple(q2.shape) != (B, H, T, d) or q2.dtype != q1.dtype or tuple(out.shape) != (B, H, T, 2 * d):
        raise ValueError("q1, q2 must be [B][H][T][d] and out [B][H][T][2d], contiguous, of one dtype")
    caches = (k1, k2, v)
    for t, w in zip(caches, (d, d, 2 * d)):
        if not t.is_cuda or t.dtype != q1.dtype or tuple(t.shape) != (B, H, L, w) or t.stride(-1) != 1:
            raise ValueError("strided caches must be [B][H][L][w] GPU views of the queries' dtype with a contiguous "
                             "last dimension")
    if lens is not None:
        if lens.dtype != torch.int32 or tuple(lens.shape) != (B,) or lens.device != q1.device:
            raise ValueError(f"lens must be an int32 tensor of shape ({B},) on {q1.device}")
        _check_tensors((lens,))
    strides = (ctypes.c_int64 * 9)(*[int(x) for t in caches for x in t.stride()[:3]])
    need = diffattn_decode_varlen_workspace_bytes(B, H, T, L, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lam_f, lam_p = _lambda_args(lam, H, q1.device)
    st = lib().diffattn_decode_strided(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(),
                                       out.data_ptr(), B, H, T, L, lens.data_ptr() if lens is not None else None,
                                       strides, d, _dtype_code(q1), lam_f, lam_p, int(layer), ws_ptr, ws_bytes,
                                       _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_decode_strided")
    return out


def diffattn_fwd_strided(q1, k1, q2, k2, v, lam, layer: int, causal: bool, out=None, stream=None):
    """Prefill (bf16, d = 64) on strided [B][H][N][.] views, e.g. slices of packed projection outputs; out may be a
    strided view too (default: a new contiguous tensor).  Each tensor's last dimension must be contiguous."""
    import torch
    B, H, N, d = q1.shape
    if out is None:
        out = torch.empty((B, H, N, 2 * d), dtype=q1.dtype, device=q1.device)
    ts = (q1, k1, q2, k2, v, out)
    for t, w in zip(ts, (d, d, d, d, 2 * d, 2 * d)):
        if not t.is_cuda or t.dtype != q1.dtype or tuple(t.shape) != (B, H, N, w) or t.stride(-1) != 1:
            raise ValueError("strided prefill needs [B][H][N][w] GPU views of one dtype with a contiguous last dim")
    strides = (ctypes.c_int64 * 18)(*[int(x) for t in ts for x in t.stride()[:3]])
    lam_f, lam_p = _lambda_args(lam, H, q1.device)
    st = lib().diffattn_fwd_strided(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(),
                                    out.data_ptr(), B, H, N, d, _dtype_code(q1), lam_f, lam_p, int(layer),
                                    int(bool(causal)), strides, _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_fwd_strided")
    return out


def _strided_views(ts, widths, shape4, what):
    B, H, N = shape4
    for t, w in zip(ts, widths):
        if not t.is_cuda or t.dtype != ts[0].dtype or tuple(t.shape) != (B, H, N, w) or t.stride(-1) != 1:
            raise ValueError(f"{what} needs [B][H][N][w] GPU views of one dtype with a contiguous last dimension")
    return (ctypes.c_int64 * (3 * len(ts)))(*[int(x) for t in ts for x in t.stride()[:3]])


def diffattn_fwd_train_strided(q1, k1, q2, k2, v, lam, layer: int, causal: bool, out=None, saved=None, stream=None):
    """Training forward (bf16, d = 64) on strided [B][H][N][.] views (e.g. slices of packed projection outputs);
    out may be a strided view too.  Returns (out, saved) as diffattn_fwd_train."""
    import torch
    B, H, N, d = q1.shape
    if out is None:
        out = torch.empty((B, H, N, 2 * d), dtype=q1.dtype, device=q1.device)
    if saved is None:
        saved = torch.empty(max(diffattn_train_saved_bytes(B, H, N, d), 16), dtype=torch.uint8, device=q1.device)
    _check_tensors((saved,))
    strides = _strided_views((q1, k1, q2, k2, v, out), (d, d, d, d, 2 * d, 2 * d), (B, H, N),
                             "strided training forward")
    lam_f, lam_p = _lambda_args(lam, H, q1.device)
    st = lib().diffattn_fwd_train_strided(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), B, H, N, d, _dtype_code(q1), lam_f, lam_p, int(layer),
                                          int(bool(causal)), strides, saved.data_ptr(),
                                          saved.numel() * saved.element_size(), _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_fwd_train_strided")
    return out, saved


def diffattn_bwd_strided(q1, k1, q2, k2, v, dy, saved, lam, layer: int, causal: bool, grads, workspace=None,
                         stream=None):
    """Backward (bf16, d = 64) on strided views: q1, k1, q2, k2, v, dy and the gradients grads["dq1"], ["dk1"],
    ["dq2"], ["dk2"], ["dv"] are [B][H][N][.] GPU views with a contiguous last dimension (e.g. column slices of one
    packed projection buffer and of its gradient buffer); grads["dlambda"] is a float32 tensor of H values.
    Returns grads."""
    import torch
    B, H, N, d = q1.shape
    g = grads
    _check_tensors((saved, g["dlambda"]))
    strides = _strided_views((q1, k1, q2, k2, v, dy, g["dq1"], g["dk1"], g["dq2"], g["dk2"], g["dv"]),
                             (d, d, d, d, 2 * d, 2 * d, d, d, d, d, 2 * d), (B, H, N), "strided backward")
    need = diffattn_bwd_workspace_bytes(B, H, N, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lam_f, lam_p = _lambda_args(lam, H, q1.device)
    st = lib().diffattn_bwd_strided(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), v.data_ptr(),
                                    dy.data_ptr(), saved.data_ptr(), g["dq1"].data_ptr(), g["dk1"].data_ptr(),
                                    g["dq2"].data_ptr(), g["dk2"].data_ptr(), g["dv"].data_ptr(),
                                    g["dlambda"].data_ptr(), B, H, N, d, _dtype_code(q1), lam_f, lam_p, int(layer),
                                    int(bool(causal)), strides, ws_ptr, ws_bytes, _stream_handle(stream, q1.device))
    if st != 0:
        raise DiffAttnError(st, "diffattn_bwd_strided")
    return grads
