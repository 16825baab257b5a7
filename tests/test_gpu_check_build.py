"""Race check of the LDS load rings: the check build of the library (libdiffattn_check.so, compiled with
-DDIFFATTN_CHECK) fills every LDS piece with NaN just before the direct load that refills it is issued, in the
prefill, dQ and dK/dV kernels.  A read of a ring slot that races ahead of its load (a missing or short wait, or a
slot refilled before every wave has passed the barrier after reading it) then returns NaN instead of stale but
plausible data from four tiles earlier.  The fills change no arithmetic, so every output of the check build must be
finite and bit-identical to the ordinary build's on the same inputs.
"""
import contextlib
import os

import numpy as np
import pytest

import diffattn_inputs as di
import differential_attention_fwd_amd as da
from differential_attention_fwd_amd import build as dbuild

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("gpu")]


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def say(msg):
    print(msg, flush=True)


@contextlib.contextmanager
def check_library():
    """The binding's calls go to libdiffattn_check.so inside the block."""
    if not os.path.exists(dbuild.CHECK_LIB):
        raise FileNotFoundError(f"{dbuild.CHECK_LIB} is not built (differential_attention_fwd_amd/build.py)")
    da.lib()   # the ordinary library stays loaded for after the block
    saved = (da._lib, da.LIB_PATH)
    da._lib, da.LIB_PATH = None, dbuild.CHECK_LIB
    try:
        da.lib()
        yield
    finally:
        da._lib, da.LIB_PATH = saved


def dev_bf16(bits):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def same_bits(a, b, what):
    torch = torch_mod()
    assert torch.isfinite(b.float()).all(), f"{what}: the check build produced non-finite values"
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"{what}: bits differ"


@pytest.mark.parametrize("B,H,N,causal,layer,outliers", [
    (4, 12, 4096, True, 12, True),    # the benchmarked prefill
    (1, 2, 1, True, 1, False), (2, 2, 33, True, 0, False), (1, 3, 129, False, 2, False),
    (2, 1, 1000, True, 1, False), (1, 2, 4097, False, 3, False),
])
def test_prefill_check_build(B, H, N, causal, layer, outliers):
    torch = torch_mod()
    say(f"case: prefill check build B{B} H{H} N{N} causal={causal} layer={layer}")
    inp = {k: dev_bf16(v) for k, v in di.prefill_bf16(B, H, N, 64, seed=900 + N, outliers=outliers).items()}
    lam = float(np.float32(da.diffattn_lambda_init(max(layer, 1))))
    args = (inp["q1"], inp["k1"], inp["q2"], inp["k2"], inp["v"], lam, layer, causal)
    ref = da.diffattn_fwd(*args)
    torch.cuda.synchronize()
    with check_library():
        got = da.diffattn_fwd(*args)
        torch.cuda.synchronize()
    same_bits(ref, got, f"prefill N{N}")


@pytest.mark.parametrize("N,causal,layer", [(64, True, 0), (300, True, 3), (1000, False, 1), (4096, True, 12)])
def test_training_check_build(N, causal, layer):
    torch = torch_mod()
    B, H = (1, 2) if N < 4096 else (1, 4)
    say(f"case: training check build B{B} H{H} N{N} causal={causal} layer={layer}")
    inp = {k: dev_bf16(v) for k, v in di.prefill_bf16(B, H, N, 64, seed=950 + N).items()}
    dy = dev_bf16(di.prefill_bf16(B, H, N, 128, seed=960 + N)["q1"])   # N(0,1), [B][H][N][128]
    lam = float(np.float32(da.diffattn_lambda_init(max(layer, 1))))
    x = (inp["q1"], inp["k1"], inp["q2"], inp["k2"], inp["v"])

    def run():
        out, saved = da.diffattn_fwd_train(*x, lam, layer, causal)
        g = da.diffattn_bwd(*x, dy, saved, lam, layer, causal)
        torch.cuda.synchronize()
        return out, saved, g

    ref = run()
    with check_library():
        got = run()
    same_bits(ref[0], got[0], f"training forward N{N}")
    same_bits(ref[1], got[1], f"saved statistics N{N}")
    for k in ref[2]:
        same_bits(ref[2][k], got[2][k], f"{k} N{N}")
