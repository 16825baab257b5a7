"""CPU check that the multi-token decode rescale test's inputs force rescales of accumulators that hold data (see
ramp_cases.py); the GPU test then compares the kernel with the oracle on exactly these inputs."""
import pytest

import diffattn_inputs as di
import ramp_cases


@pytest.mark.parametrize("T", [2, 16])
def test_ramp_inputs_force_rescales(T):
    B, H, P, max_pages, lens = ramp_cases.CASE
    inp = ramp_cases.ramp_inputs(B, H, T, P * max_pages, seed=780 + T)
    f = {k: di.bf16_bits_to_f32(v) for k, v in inp.items()}
    ramp_cases.assert_ramp_forces_rescales(f, T, lens)
