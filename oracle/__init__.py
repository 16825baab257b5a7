"""CPU oracle for the differential attention forward pass (double precision).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg are the only
callers.  The product path never imports this package, and this package imports nothing from the product.

The arithmetic lives in `diffattn_oracle.c` (plain C, OpenMP over query rows); this module only builds that file
with gcc and marshals numpy arrays into it.  Pages cited: Ultralytics glossary entry "Differential Transformer",
section on how differential attention works (worked example and the paragraph after it); jisaku.com glossary
entry "Differential Transformer (Diff Attention)", section "main features / mechanism".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "diffattn_oracle.c")


def lib_path(mutant: int = 0) -> str:
    if mutant:
        return os.path.join(HERE, "_build", f"liboracle_mutant{mutant}.so")
    return os.path.join(HERE, "liboracle.so")


def build(mutant: int = 0) -> str:
    """Compile the oracle with gcc (-O3, no fast-math, OpenMP).  `mutant` plants a numbered mistake (tests)."""
    out = lib_path(mutant)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = ["gcc", "-O3", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall", f"-DORACLE_MUTANT={int(mutant)}",
           SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_libs: dict = {}


def _load(mutant: int = 0):
    if mutant in _libs:
        return _libs[mutant]
    path = lib_path(mutant)
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
        build(mutant)
    lib = ctypes.CDLL(path)
    lib.oracle_lambda_init.argtypes = [ctypes.c_int]
    lib.oracle_lambda_init.restype = ctypes.c_double
    lib.oracle_mutant.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_diffattn.argtypes = [P, P, P, P, P, i64, i64, i64, i64, i64, ctypes.c_double, ctypes.c_int,
                                    ctypes.c_int, P, i64, P, P, ctypes.c_int]
    lib.oracle_diffattn.restype = ctypes.c_int
    lib.oracle_diffattn_bwd.argtypes = [P, P, P, P, P, P, i64, i64, i64, i64, P, ctypes.c_int, ctypes.c_int,
                                        P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_diffattn_bwd.restype = ctypes.c_int
    _libs[mutant] = lib
    return lib


def lambda_init(layer: int, mutant: int = 0) -> float:
    """lambda_init(l) = 0.8 - 0.6 exp(-0.3 (l - 1)), 1-based layer index."""
    return float(_load(mutant).oracle_lambda_init(int(layer)))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x), dtype=np.float32)


def diffattn(q1, k1, q2, k2, v, lam, layer: int, causal: bool, rows=None, want_diff: bool = False,
             threads: int = 0, mutant: int = 0):
    """Evaluate the definition for selected query rows.

    q1, q2: [B][H][Nq][d]; k1, k2: [B][H][Nk][d]; v: [B][H][Nk][2d]  (float32 values; bf16 inputs widened).
    lam: one float, or an array of H floats (one lambda per head).
    rows: None (all B*H*Nq rows, in [B][H][Nq] order) or indices into the flattened query rows.
    Returns out as float64 [nrows][2d] (reshaped to [B][H][Nq][2d] when rows is None), and with want_diff
    also the difference-map rows [nrows][Nk] (masked keys hold 0).
    """
    q1, k1, q2, k2, v = (_f32(t) for t in (q1, k1, q2, k2, v))
    B, H, Nq, d = q1.shape
    Nk = k1.shape[2]
    assert q2.shape == q1.shape and k1.shape == (B, H, Nk, d) and k2.shape == k1.shape
    assert v.shape == (B, H, Nk, 2 * d)
    if np.ndim(lam) == 1:
        # One lambda per head: the same definition, evaluated head by head with that head's lambda.
        lam = np.asarray(lam, dtype=np.float64)
        assert lam.shape == (H,)
        return _per_head(q1, k1, q2, k2, v, lam, layer, causal, rows, want_diff, threads, mutant)
    if rows is None:
        rows_arr = None
        nrows = B * H * Nq
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).ravel())
        nrows = rows_arr.size
    out = np.zeros((nrows, 2 * d), dtype=np.float64)
    diff = np.zeros((nrows, Nk), dtype=np.float64) if want_diff else None
    rc = _load(mutant).oracle_diffattn(
        q1.ctypes.data, k1.ctypes.data, q2.ctypes.data, k2.ctypes.data, v.ctypes.data,
        B, H, Nq, Nk, d, float(lam), int(layer), int(bool(causal)),
        rows_arr.ctypes.data if rows_arr is not None else None, nrows,
        out.ctypes.data, diff.ctypes.data if diff is not None else None, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_diffattn rejected its arguments (rc={rc})")
    if rows is None:
        out = out.reshape(B, H, Nq, 2 * d)
        if diff is not None:
            diff = diff.reshape(B, H, Nq, Nk)
    return (out, diff) if want_diff else out


def _per_head(q1, k1, q2, k2, v, lam, layer, causal, rows, want_diff, threads, mutant):
    B, H, Nq, d = q1.shape
    Nk = k1.shape[2]
    flat = np.arange(B * H * Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64).ravel()
    out = np.zeros((flat.size, 2 * d), dtype=np.float64)
    diff = np.zeros((flat.size, Nk), dtype=np.float64) if want_diff else None
    b, h, i = flat // (H * Nq), (flat // Nq) % H, flat % Nq
    for hh in range(H):
        sel = np.nonzero(h == hh)[0]
        if sel.size == 0:
            continue
        sl = (slice(None), slice(hh, hh + 1))
        res = diffattn(q1[sl], k1[sl], q2[sl], k2[sl], v[sl], float(lam[hh]), layer, causal,
                       rows=b[sel] * Nq + i[sel], want_diff=want_diff, threads=threads, mutant=mutant)
        if want_diff:
            out[sel], diff[sel] = res
        else:
            out[sel] = res
    if rows is None:
        out = out.reshape(B, H, Nq, 2 * d)
        if diff is not None:
            diff = diff.reshape(B, H, Nq, Nk)
    return (out, diff) if want_diff else out


def diffattn_bwd(q1, k1, q2, k2, v, dy, lam, layer: int, causal: bool, threads: int = 0, mutant: int = 0):
    """Gradients of a loss with respect to the inputs of the square (Nq = Nk) forward, given dy = dLoss/dout.

    q1, k1, q2, k2: [B][H][N][d]; v, dy: [B][H][N][2d] (float32 values).  lam: one float or H floats.
    Returns a dict of float64 arrays: dq1, dk1, dq2, dk2 [B][H][N][d], dv [B][H][N][2d], dlambda [H] (summed over
    the batch; for a scalar lambda shared by all heads its gradient is dlambda.sum()).
    """
    q1, k1, q2, k2, v, dy = (_f32(t) for t in (q1, k1, q2, k2, v, dy))
    B, H, N, d = q1.shape
    assert k1.shape == q1.shape and q2.shape == q1.shape and k2.shape == q1.shape
    assert v.shape == (B, H, N, 2 * d) and dy.shape == v.shape
    lh = np.ascontiguousarray(np.broadcast_to(np.asarray(lam, dtype=np.float64), (H,)))
    g = {k: np.zeros((B, H, N, d), dtype=np.float64) for k in ("dq1", "dk1", "dq2", "dk2")}
    g["dv"] = np.zeros((B, H, N, 2 * d), dtype=np.float64)
    g["dlambda"] = np.zeros(H, dtype=np.float64)
    rc = _load(mutant).oracle_diffattn_bwd(
        q1.ctypes.data, k1.ctypes.data, q2.ctypes.data, k2.ctypes.data, v.ctypes.data, dy.ctypes.data,
        B, H, N, d, lh.ctypes.data, int(layer), int(bool(causal)),
        g["dq1"].ctypes.data, g["dk1"].ctypes.data, g["dq2"].ctypes.data, g["dk2"].ctypes.data, g["dv"].ctypes.data,
        g["dlambda"].ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_diffattn_bwd rejected its arguments (rc={rc})")
    return g


def decode(q1, k1, q2, k2, v, lam, layer: int, rows=None, threads: int = 0, mutant: int = 0):
    """Single-token decode: q1, q2 [B][H][d] against caches k [B][H][L][d], v [B][H][L][2d]; out [B][H][2d]."""
    q1 = _f32(q1)
    q2 = _f32(q2)
    B, H, d = q1.shape
    out = diffattn(q1[:, :, None, :], k1, q2[:, :, None, :], k2, v, lam, layer, True, rows=rows,
                   threads=threads, mutant=mutant)
    return out.reshape(B, H, 2 * d) if rows is None else out
