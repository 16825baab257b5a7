"""The allocation-free decode (diffattn_decode_noalloc) against diffattn_decode: same kernels and split plan, so the
outputs must be identical bit for bit.  Two calls in a row, the second on a smaller problem, so the second call
reuses the per-GPU scratch array the first one filled with larger partials; then a call whose partials would not fit
is rejected before any HIP call."""
import numpy as np
import pytest

import diffattn_inputs as di
import differential_attention_fwd_amd as da

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("gpu")]


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


@pytest.mark.parametrize("cases", [[(8, 16, 4100, 1, 0.8), (2, 3, 777, 3, 0.6)]])
def test_decode_noalloc_equals_decode(cases):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    for (B, H, L, layer, lam) in cases:
        print(f"case: decode noalloc B{B} H{H} L{L} layer {layer}", flush=True)
        assert da.diffattn_decode_workspace_bytes(B, H, L, 64) <= da.NOALLOC_SCRATCH_BYTES
        inp = di.decode_bf16(B, H, L, 64, seed=900 + L)
        dev = {k: _dev(v) for k, v in inp.items()}
        lam = float(np.float32(lam))
        ref = da.diffattn_decode(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, layer)
        got = da.diffattn_decode_noalloc(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, layer)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # Partials past the scratch size (B64 H16 L65536: 16 splits of 4096 keys per head, 17.0 MB) are rejected with
    # DIFFATTN_ERR_WORKSPACE before anything runs, so the call reads none of the (small) buffers it is handed.
    B, H, L = 64, 16, 65536
    assert da.diffattn_decode_workspace_bytes(B, H, L, 64) > da.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(1, 1, 64, dtype=torch.bfloat16, device="cuda:0")
    o = torch.zeros(1, 1, 128, dtype=torch.bfloat16, device="cuda:0")
    st = da.lib().diffattn_decode_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                          o.data_ptr(), B, H, L, 64, 0, 0.8, 1, 1, None)
    assert st == -7
