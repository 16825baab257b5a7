"""Pins of the backward oracle (no GPU).

The backward oracle is the chain rule written out.  It is pinned to the forward oracle (itself pinned to the pages'
worked example and closed forms) by central finite differences: for a loss L = sum(out * dy), dL/dx from the
backward must match (L(x + h) - L(x - h)) / 2h evaluated with the forward, for every input element and for lambda.
Inputs live on a grid of 2^-14 and h = 2^-10, so x +- h is exact in float32 and the only error is the difference
quotient's own O(h^2) term.  Each planted mistake in the backward (mutants 11..15) must fail this pin.
"""
import numpy as np
import pytest

import oracle

H_STEP = 2.0 ** -10
BWD_MUTANTS = {11: "softmax row term dropped", 12: "map-2 gradient without -lambda",
               13: "normalisation backward without its projection term", 14: "sign of d(lambda)",
               15: "dk1 built from q2"}


def grid_inputs(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    def g(*shape, scale=1.0):
        return (np.round(rng.standard_normal(shape) * scale * 2 ** 14) / 2 ** 14).astype(np.float32)
    return {"q1": g(B, H, N, d), "k1": g(B, H, N, d), "q2": g(B, H, N, d), "k2": g(B, H, N, d),
            "v": g(B, H, N, 2 * d), "dy": g(B, H, N, 2 * d)}


def loss(x, lam, layer, causal):
    out = oracle.diffattn(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, layer, causal)
    return float(np.sum(out * x["dy"].astype(np.float64)))


def fd_check(x, lam, layer, causal, mutant=0):
    """Max relative deviation between the backward oracle and central differences of the forward."""
    g = oracle.diffattn_bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["dy"], lam, layer, causal, mutant=mutant)
    worst = 0.0
    for name in ("q1", "k1", "q2", "k2", "v"):
        ana = g["d" + name]
        flat = x[name].reshape(-1)
        for idx in range(flat.size):
            old = flat[idx]
            flat[idx] = old + np.float32(H_STEP)
            lp = loss(x, lam, layer, causal)
            flat[idx] = old - np.float32(H_STEP)
            lm = loss(x, lam, layer, causal)
            flat[idx] = old
            fd = (lp - lm) / (2 * H_STEP)
            a = ana.reshape(-1)[idx]
            worst = max(worst, abs(fd - a) / (1.0 + abs(a)))
    lam_arr = np.broadcast_to(np.asarray(lam, dtype=np.float64), (x["q1"].shape[1],)).copy()
    for h in range(lam_arr.size):
        lp_arr, lm_arr = lam_arr.copy(), lam_arr.copy()
        lp_arr[h] += H_STEP
        lm_arr[h] -= H_STEP
        fd = (loss(x, lp_arr, layer, causal) - loss(x, lm_arr, layer, causal)) / (2 * H_STEP)
        worst = max(worst, abs(fd - g["dlambda"][h]) / (1.0 + abs(g["dlambda"][h])))
    return worst


CASES = [(0, True), (0, False), (3, True), (5, False)]


@pytest.mark.parametrize("layer,causal", CASES)
def test_backward_matches_finite_differences(layer, causal):
    x = grid_inputs(2, 2, 5, 4, seed=50 + layer)
    worst = fd_check(x, np.array([0.3, 0.75]), layer, causal)
    assert worst < 2e-5, worst


def test_backward_rejects_bad_arguments():
    x = grid_inputs(1, 1, 3, 4, seed=1)
    with pytest.raises(ValueError):
        oracle.diffattn_bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["dy"], 0.5, -1, True)


def test_backward_gradients_of_v_sum_rows():
    """With dy = 1 on channel c only and layer 0, dv[:, c] sums (a - lambda b) over query rows: its total over keys
    is the row count times (1 - lambda), since each row of each map sums to one."""
    x = grid_inputs(1, 1, 6, 4, seed=3)
    x["dy"][:] = 0
    x["dy"][..., 2] = 1
    lam = 0.4
    g = oracle.diffattn_bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], x["dy"], lam, 0, True)
    assert abs(g["dv"][..., 2].sum() - 6 * (1 - lam)) < 1e-12
    assert np.abs(np.delete(g["dv"], 2, axis=-1)).max() == 0.0


@pytest.mark.parametrize("mutant", sorted(BWD_MUTANTS), ids=lambda k: f"mutant{k}")
def test_backward_planted_mistake_is_caught(mutant):
    oracle.build(mutant)
    x = grid_inputs(1, 2, 4, 4, seed=70)
    worst = max(fd_check({k: v.copy() for k, v in x.items()}, np.array([0.3, 0.75]), layer, causal, mutant=mutant)
                for layer, causal in ((0, True), (3, False)))
    assert worst > 1e-3, f"mutant {mutant} ({BWD_MUTANTS[mutant]}) passes the finite-difference pin"
