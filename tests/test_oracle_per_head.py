"""Oracle with one lambda per head (no GPU).

Per-head lambda adds no arithmetic: the oracle evaluates the pinned scalar definition head by head.  These checks
tie the per-head path to values fixed independently of it: a head with lambda = 0 is plain softmax attention over
map 1 (the textbook definition, written out here with numpy), and lambda enters the raw output linearly, so two
heads with lambdas l and 2l differ from the lambda = 0 output by exact multiples of one vector.
"""
import numpy as np

import diffattn_inputs as di
import oracle


def softmax_attention(q, k, v, causal):
    d = q.shape[-1]
    s = q.astype(np.float64) @ k.astype(np.float64).T / np.sqrt(d)
    if causal:
        s = np.where(np.tril(np.ones_like(s, dtype=bool)), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p @ v.astype(np.float64)


def test_per_head_lambda_zero_is_softmax_attention():
    f = di.prefill_f32(1, 3, 23, 8, seed=31)
    out = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], np.array([0.0, 0.4, 0.0]), 0, True)
    for h in (0, 2):
        ref = softmax_attention(f["q1"][0, h], f["k1"][0, h], f["v"][0, h], True)
        assert np.abs(out[0, h] - ref).max() < 1e-12


def test_per_head_lambda_is_linear_in_raw_output():
    f = di.prefill_f32(2, 3, 19, 8, seed=32)
    # The same head data in all three heads, lambdas 0, l and 2l.
    g = {k: np.repeat(f[k][:, :1], 3, axis=1) for k in f}
    lam = 0.35
    out = oracle.diffattn(g["q1"], g["k1"], g["q2"], g["k2"], g["v"], np.array([0.0, lam, 2 * lam]), 0, False)
    step = out[:, 1] - out[:, 0]
    assert np.abs(out[:, 2] - out[:, 0] - 2 * step).max() < 1e-12
    assert np.abs(step).max() > 1e-3


def test_per_head_rows_subset_matches_full():
    f = di.prefill_f32(2, 3, 11, 8, seed=33)
    lam = np.array([0.2, 0.6, 0.9])
    full = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, 3, True).reshape(-1, 16)
    rows = np.array([0, 5, 11, 30, 45, 65])
    sub = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, 3, True, rows=rows)
    assert np.array_equal(sub, full[rows])
