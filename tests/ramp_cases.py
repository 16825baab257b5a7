"""Decode inputs that force the multi-token kernel's online softmax to rescale accumulators holding data, and the
CPU check that they do (used by the GPU parity test and, on the CPU alone, by test_ramp_cases.py).

The threshold checked is the multi-token decode kernel's rescale rule: a tile moves the running offset when its
largest exponent argument exceeds the offset by more than 8 (log2 units).
"""
import numpy as np

import diffattn_inputs as di

# B, H, page rows, pages per sequence, cache lengths: the case the GPU test runs (L = 64 * 47 = 3008 rows).
CASE = (2, 2, 64, 47, [3008, 1337])

RAMP_PERIOD = 256


def ramp_inputs(B, H, T, L, seed):
    """Decode inputs whose map-1 scores grow by half a nat per key inside every RAMP_PERIOD-key block of the cache:
    q1 . k1_j / sqrt(d) = (j mod RAMP_PERIOD) / 2 + N(0, 1) noise for every new token (feature 0 of q1 is 64 and of k1_j
    is (j mod RAMP_PERIOD) / 16, both exact in bf16).  Map 2, the other features and V stay seeded N(0, 1)."""
    kv = di.decode_bf16(B, H, L, 64, seed=seed)
    q = di.prefill_bf16(B, H, T, 64, seed=seed + 1)
    inp = {"q1": q["q1"], "q2": q["q2"], "k1": kv["k1"], "k2": kv["k2"], "v": kv["v"]}
    q1 = di.bf16_bits_to_f32(inp["q1"]).copy()
    k1 = di.bf16_bits_to_f32(inp["k1"]).copy()
    q1[..., 0] = 64.0
    k1[..., 0] = (np.arange(L) % RAMP_PERIOD).astype(np.float32) / 16.0
    inp["q1"] = di.f32_to_bf16_bits(q1)
    inp["k1"] = di.f32_to_bf16_bits(k1)
    return inp


def assert_ramp_forces_rescales(f, T, lens):
    """On the CPU, from the inputs alone: for every new token and every placement of two consecutive 32-key tiles
    inside one ramp block (whatever a split's first key), the second tile's largest map-1 exponent argument
    (log2 units, q1 . k1 log2(e) / sqrt(d)) exceeds the first tile's by more than 8, the multi-token kernel's rescale
    threshold, while the first tile's probabilities (and with N(0,1) values its output sums) are non-zero.  So every
    split that holds two such tiles rescales accumulators that already hold data."""
    B, H, L = f["k1"].shape[:3]
    c = np.log2(np.e) / 8.0
    checked = 0
    for b in range(B):
        Lb = min(max(int(lens[b]), T), L)
        for h in range(H):
            x = (f["q1"][b, h].astype(np.float64) @ f["k1"][b, h, :Lb].astype(np.float64).T) * c   # [T][Lb]
            win = np.lib.stride_tricks.sliding_window_view(x, 32, axis=1).max(axis=-1)   # [T][Lb - 31]
            for t in range(T):
                vis = Lb - T + t + 1
                j0 = np.arange(0, max(vis - 63, 0))
                j0 = j0[j0 // RAMP_PERIOD == (j0 + 63) // RAMP_PERIOD]
                gap = win[t, j0 + 32] - win[t, j0]
                assert (gap > 8.0).all(), (b, h, t, gap.min())
                checked += j0.size
    assert checked > 0


