"""Pins for the CPU oracle: facts fixed by the pages or by mathematics, independent of the oracle's own code.

Each pin takes a `mutant` number (0 = the real oracle) and returns a list of failure strings (empty = pass), so
the same pins both certify the oracle and show that planted mistakes are caught.

Pages: [U] Ultralytics glossary entry "Differential Transformer", section on how differential attention works
(worked example and the paragraph after it).  Library routines used as independent references: torch.softmax,
torch.nn.functional.scaled_dot_product_attention and torch.nn.functional.rms_norm, all in float64 on the CPU.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import diffattn_inputs as di
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _t64(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64))


def pin_worked_example_printed(mutant=0):
    """[U] worked example: row 0 prints as 0.20, 13 of the 36 weights are negative; the prose says every row
    sums to 1 - lambda."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    ex = di.worked_example()
    out, diff = oracle.diffattn(ex["q1"], ex["k1"], ex["q2"], ex["k2"], ex["v"], g["lambda"], 0, g["causal"],
                                want_diff=True, mutant=mutant)
    w = diff[0, 0]
    fails = []
    if f"{w.sum(axis=-1)[0]:.2f}" != g["printed_row0_sum_2dp"]:
        fails.append(f"row-0 sum prints {w.sum(axis=-1)[0]:.2f}")
    if int((w < 0).sum()) != g["printed_negative_count"] or w.size != g["printed_weight_count"]:
        fails.append(f"{int((w < 0).sum())} of {w.size} negative")
    if np.abs(w.sum(axis=-1) - (1 - g["lambda"])).max() > 1e-12:
        fails.append("some row does not sum to 1 - lambda")
    return fails


def pin_worked_example_library(mutant=0):
    """[U] worked example, map and output, from library routines in float64: both maps come from one batched
    torch.softmax over the stacked [2][n][n] score tensor (scores scaled by 1/sqrt(d), d the query/key width), which
    an explicit exp-and-normalise must reproduce; then w = map1 - lambda map2 and o = w V."""
    ex = di.worked_example()
    q = np.stack([ex["q1"][0, 0], ex["q2"][0, 0]]).astype(np.float64)   # [map][n][d]
    k = np.stack([ex["k1"][0, 0], ex["k2"][0, 0]]).astype(np.float64)
    v = ex["v"][0, 0].astype(np.float64)
    lam = float(ex["lambda"])
    scores = np.einsum("mid,mjd->mij", q, k) / math.sqrt(ex["d"])
    maps = torch.softmax(torch.from_numpy(scores), dim=-1).numpy()
    e = np.exp(scores - scores.max(axis=-1, keepdims=True))
    fails = []
    if np.abs(maps - e / e.sum(axis=-1, keepdims=True)).max() > 1e-15:
        fails.append("library softmax disagrees with exp-and-normalise")
    ref_w = maps[0] - lam * maps[1]
    ref_o = ref_w @ v
    out, diff = oracle.diffattn(ex["q1"], ex["k1"], ex["q2"], ex["k2"], ex["v"], ex["lambda"], 0, False,
                                want_diff=True, mutant=mutant)
    if np.abs(diff[0, 0] - ref_w).max() > 1e-12:
        fails.append(f"map differs by {np.abs(diff[0, 0] - ref_w).max():.3g}")
    if np.abs(out[0, 0] - ref_o).max() > 1e-12:
        fails.append(f"output differs by {np.abs(out[0, 0] - ref_o).max():.3g}")
    return fails


def _sdpa(q, k, v, causal):
    return F.scaled_dot_product_attention(_t64(q), _t64(k), _t64(v), is_causal=causal).numpy()


def pin_lambda_zero_is_attention(mutant=0):
    """lambda = 0 leaves map1 . V: ordinary scaled softmax attention (library routine, scale 1/sqrt(d))."""
    fails = []
    for (B, H, N, d, causal, seed) in [(1, 2, 1, 4, True, 1), (2, 3, 17, 8, True, 2), (1, 2, 33, 16, False, 3),
                                       (2, 1, 40, 64, True, 4)]:
        q1, k1, q2, k2 = (_rand(seed * 10 + t, B, H, N, d) for t in range(4))
        v = _rand(seed * 10 + 4, B, H, N, 2 * d)
        got = oracle.diffattn(q1, k1, q2, k2, v, 0.0, 0, causal, mutant=mutant)
        ref = _sdpa(q1, k1, v, causal)
        err = np.abs(got - ref).max()
        if err > 1e-11:
            fails.append(f"B{B} H{H} N{N} d{d} causal={causal}: {err:.3g}")
    return fails


def pin_normalised_epilogue(mutant=0):
    """Layer 1: lambda_init(1) = 0.8 - 0.6 = 0.2, so the output is rms_norm(attention, eps=1e-5) * 0.8
    (lambda = 0 makes the attention part a library routine too)."""
    fails = []
    for (B, H, N, d, causal, seed, vscale) in [(1, 2, 9, 8, True, 5, 1.0), (2, 2, 21, 16, False, 6, 1.0),
                                                (1, 1, 12, 4, True, 7, 1e-3)]:
        q1, k1, q2, k2 = (_rand(seed * 10 + t, B, H, N, d) for t in range(4))
        v = _rand(seed * 10 + 4, B, H, N, 2 * d) * np.float32(vscale)
        got = oracle.diffattn(q1, k1, q2, k2, v, 0.0, 1, causal, mutant=mutant)
        att = torch.from_numpy(_sdpa(q1, k1, v, causal))
        ref = (F.rms_norm(att, (2 * d,), eps=1e-5) * 0.8).numpy()
        err = np.abs(got - ref).max()
        if err > 1e-11:
            fails.append(f"N{N} d{d} causal={causal} vscale={vscale}: {err:.3g}")
    return fails


def pin_row_sums(mutant=0):
    """[U]: each map sums to 1, so each row of the difference map sums to 1 - lambda.  With V all ones every output
    channel equals that row sum."""
    fails = []
    for (N, d, causal, lam, seed) in [(1, 4, True, 0.3, 1), (13, 8, True, 0.8, 2), (13, 8, False, 0.55, 3),
                                      (64, 16, True, 0.999, 4)]:
        q1, k1, q2, k2 = (_rand(seed * 7 + t, 1, 2, N, d) * 3 for t in range(4))
        v = np.ones((1, 2, N, 2 * d), dtype=np.float32)
        got = oracle.diffattn(q1, k1, q2, k2, v, lam, 0, causal, mutant=mutant)
        err = np.abs(got - (1 - lam)).max()
        if err > 1e-12:
            fails.append(f"N{N} causal={causal} lam={lam}: {err:.3g}")
    return fails


def pin_prefix_means(mutant=0):
    """Zero queries make both maps uniform over the visible keys: with the causal mask, row i of the raw output
    is (1 - lambda) times the mean of v_0..v_i."""
    fails = []
    for (N, d, lam, seed) in [(1, 4, 0.8, 1), (19, 8, 0.2, 2), (50, 16, 0.7, 3)]:
        z = np.zeros((1, 1, N, d), dtype=np.float32)
        k1, k2 = _rand(seed, 1, 1, N, d), _rand(seed + 1, 1, 1, N, d)
        v = _rand(seed + 2, 1, 1, N, 2 * d)
        got = oracle.diffattn(z, k1, z, k2, v, lam, 0, True, mutant=mutant)[0, 0]
        vv = v[0, 0].astype(np.float64)
        ref = (1 - lam) * np.cumsum(vv, axis=0) / np.arange(1, N + 1)[:, None]
        err = np.abs(got - ref).max()
        if err > 1e-12:
            fails.append(f"N{N} lam={lam}: {err:.3g}")
    return fails


def pin_causal_row0(mutant=0):
    """Causal row 0 sees only key 0: o_0 = (1 - lambda) v_0, so at layer 1 (scale 0.8)
    y_0 = v_0 / sqrt(mean(v_0^2) + 1e-5 / (1 - lambda)^2) * 0.8."""
    fails = []
    for (N, d, lam, seed, vs) in [(5, 8, 0.8, 11, 1.0), (3, 64, 0.3, 12, 0.01)]:
        q1, k1, q2, k2 = (_rand(seed * 5 + t, 1, 1, N, d) for t in range(4))
        v = _rand(seed * 5 + 4, 1, 1, N, 2 * d) * np.float32(vs)
        got = oracle.diffattn(q1, k1, q2, k2, v, lam, 1, True, mutant=mutant)[0, 0, 0]
        v0 = v[0, 0, 0].astype(np.float64)
        ref = v0 / math.sqrt(np.mean(v0 * v0) + 1e-5 / (1 - lam) ** 2) * 0.8
        err = np.abs(got - ref).max()
        if err > 1e-12:
            fails.append(f"d{d} lam={lam}: {err:.3g}")
    return fails


def pin_identical_halves(mutant=0):
    """Q2 = Q1 and K2 = K1 make the maps equal: the raw output is (1 - lambda) times ordinary attention."""
    fails = []
    for (N, d, causal, lam, seed) in [(23, 8, True, 0.8, 1), (16, 16, False, 0.35, 2)]:
        q, k = _rand(seed, 2, 2, N, d), _rand(seed + 1, 2, 2, N, d)
        v = _rand(seed + 2, 2, 2, N, 2 * d)
        got = oracle.diffattn(q, k, q, k, v, lam, 0, causal, mutant=mutant)
        ref = (1 - lam) * _sdpa(q, k, v, causal)
        err = np.abs(got - ref).max()
        if err > 1e-11:
            fails.append(f"N{N} causal={causal}: {err:.3g}")
    return fails


def pin_swapped_halves(mutant=0):
    """Exchanging (Q1,K1) with (Q2,K2) and lambda = 1 negates the raw output (map1 - map2 = -(map2 - map1))."""
    fails = []
    N, d = 15, 8
    q1, k1, q2, k2 = (_rand(40 + t, 1, 2, N, d) for t in range(4))
    v = _rand(45, 1, 2, N, 2 * d)
    a = oracle.diffattn(q1, k1, q2, k2, v, 1.0, 0, True, mutant=mutant)
    b = oracle.diffattn(q2, k2, q1, k1, v, 1.0, 0, True, mutant=mutant)
    if np.abs(a + b).max() > 1e-12:
        fails.append(f"{np.abs(a + b).max():.3g}")
    return fails


def pin_lambda_init_schedule(mutant=0):
    """[U]: lambda_init(l) = 0.8 - 0.6 exp(-0.3 (l - 1)).  Fixed facts: the first layer starts at 0.2, deeper
    layers start closer to 0.8 (increasing, bounded by 0.8), and the gap to 0.8 shrinks by the factor e^-0.3 per
    layer."""
    fails = []
    vals = [oracle.lambda_init(l, mutant=mutant) for l in range(1, 40)]
    if abs(vals[0] - 0.2) > 1e-15:
        fails.append(f"lambda_init(1) = {vals[0]!r}")
    if not all(b > a for a, b in zip(vals, vals[1:])) or not all(x < 0.8 for x in vals):
        fails.append("not increasing towards 0.8")
    ratios = [(0.8 - b) / (0.8 - a) for a, b in zip(vals, vals[1:])]
    if max(abs(r - math.exp(-0.3)) for r in ratios) > 1e-9:
        fails.append("gap ratio is not exp(-0.3)")
    if abs(oracle.lambda_init(400, mutant=mutant) - 0.8) > 1e-15:
        fails.append("does not tend to 0.8")
    return fails


def pin_decode_is_attention(mutant=0):
    """A single decode query sees every cached key: with lambda = 0 it is ordinary attention of one query."""
    B, H, L, d = 2, 3, 37, 16
    q1, q2 = _rand(1, B, H, d), _rand(2, B, H, d)
    k1, k2 = _rand(3, B, H, L, d), _rand(4, B, H, L, d)
    v = _rand(5, B, H, L, 2 * d)
    got = oracle.decode(q1, k1, q2, k2, v, 0.0, 0, mutant=mutant)
    ref = _sdpa(q1[:, :, None], k1, v, False)[:, :, 0]
    err = np.abs(got - ref).max()
    return [] if err <= 1e-11 else [f"{err:.3g}"]


def pin_identity_values_extract_map(mutant=0):
    """V = [I | 0] copies the difference map into the first output channels: out[i, j] = w[i, j]."""
    N, d = 12, 8
    q1, k1, q2, k2 = (_rand(60 + t, 1, 1, N, d) for t in range(4))
    v = np.zeros((1, 1, N, 2 * d), dtype=np.float32)
    v[0, 0, :, :N] = np.eye(N, dtype=np.float32)
    out, diff = oracle.diffattn(q1, k1, q2, k2, v, 0.8, 0, True, want_diff=True, mutant=mutant)
    err = np.abs(out[0, 0, :, :N] - diff[0, 0]).max()
    return [] if err <= 1e-15 else [f"{err:.3g}"]


ALL_PINS = [pin_worked_example_printed, pin_worked_example_library, pin_lambda_zero_is_attention,
            pin_normalised_epilogue, pin_row_sums, pin_prefix_means, pin_causal_row0, pin_identical_halves,
            pin_swapped_halves, pin_lambda_init_schedule, pin_decode_is_attention, pin_identity_values_extract_map]
