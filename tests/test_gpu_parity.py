"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Tolerances: fp32 path max-abs <= 1e-5; bf16 path (outputs after normalisation, whose RMS is 1 - lambda_init <= 0.8)
max-abs <= 2e-2 and mean-abs <= 2e-3.  Raw (layer 0) bf16 outputs have no fixed scale (a row's weights sum to
1 - lambda, so they are often far below 1); each row is held to the bounds its layer-1 normalisation would have to
meet: max and mean of |got - ref| / rms(ref row) <= 2e-2 / 0.8 and 2e-3 / 0.8.
"""
import numpy as np
import pytest

import diffattn_inputs as di
import differential_attention_fwd_amd as da
import oracle
import ramp_cases

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("gpu")]

F32_TOL = 1e-5
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
RAW_MAX, RAW_MEAN = BF16_MAX / 0.8, BF16_MEAN / 0.8   # raw outputs, relative to each row's RMS (see check_bf16)
BOUNDS = (BF16_MAX, BF16_MEAN, RAW_MAX, RAW_MEAN)


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def say(msg):
    print(msg, flush=True)


def dev_bf16(bits):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def dev_f32(x):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")


def host_bf16(t):
    torch = torch_mod()
    return di.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def widen(inp):
    return {k: di.bf16_bits_to_f32(v) for k, v in inp.items()}


def lam_of(spec):
    if isinstance(spec, tuple):
        return float(np.float32(oracle.lambda_init(spec[1])))
    return float(np.float32(spec))


def check_bf16(got, ref, what, raw=False, scale=1.0):
    """bf16 bounds.  Normalised outputs: absolute.  Raw (layer 0) outputs: every row against its own RMS, as the
    layer-1 normalisation (RMS norm, then the scale 1 - lambda_init(1) = 0.8) would see it, so the normalised bounds
    become 2e-2 / 0.8 and 2e-3 / 0.8 relative to the row's RMS (rows whose RMS is below 1e-3 of the tensor's are
    measured against that floor).  `scale` multiplies every bound: 2 when two results that each meet the bounds
    against the exact values are compared with one another."""
    BF16_MAX, BF16_MEAN, RAW_MAX, RAW_MEAN = (scale * b for b in BOUNDS)
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), what
    if not raw:
        say(f"{what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
        assert err.max() <= BF16_MAX, f"{what}: max-abs {err.max():.3e}"
        assert err.mean() <= BF16_MEAN, f"{what}: mean-abs {err.mean():.3e}"
        return
    rms = np.sqrt(np.mean(np.square(ref), axis=-1, keepdims=True))
    rms = np.maximum(rms, 1e-3 * float(np.sqrt(np.mean(np.square(ref)))))
    rel = err / rms
    say(f"{what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}; relative to row RMS: max {rel.max():.2e} "
        f"mean {rel.mean():.2e} (bounds {RAW_MAX:.1e}, {RAW_MEAN:.1e})")
    assert rel.max() <= RAW_MAX, f"{what}: max relative to row RMS {rel.max():.3e}"
    assert rel.mean() <= RAW_MEAN, f"{what}: mean relative to row RMS {rel.mean():.3e}"


def run_prefill_bf16(inp, lam, layer, causal):
    torch = torch_mod()
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    out = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, layer, causal)
    torch.cuda.synchronize()
    return host_bf16(out)


# ---------------------------------------------------------------------------------------------------------------
# The pages' worked example (fp32): n=6, d=8, lambda 0.8, non-causal, raw output and the difference map.
# ---------------------------------------------------------------------------------------------------------------

def test_worked_example_f32():
    torch = torch_mod()
    ex = di.worked_example()
    say("case: worked example fp32 n6 d8")
    dev = {k: dev_f32(ex[k]) for k in ("q1", "k1", "q2", "k2", "v")}
    out = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.8, 0, False)
    # V = [I | 0] copies the difference map into the first n output channels.
    eye = np.zeros((1, 1, 6, 16), dtype=np.float32)
    eye[0, 0, :, :6] = np.eye(6, dtype=np.float32)
    wmap = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev_f32(eye), 0.8, 0, False)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    got_w = wmap.cpu().numpy()[0, 0, :, :6].astype(np.float64)
    ref, ref_w = oracle.diffattn(ex["q1"], ex["k1"], ex["q2"], ex["k2"], ex["v"], float(np.float32(0.8)), 0, False,
                                 want_diff=True)
    assert np.abs(got - ref).max() <= F32_TOL
    assert np.abs(got_w - ref_w[0, 0]).max() <= F32_TOL
    assert np.abs(got_w.sum(axis=1) - 0.2).max() <= F32_TOL        # every row sums to 1 - lambda
    assert int((got_w < 0).sum()) == 13                              # the pages' printed count


@pytest.mark.parametrize("N,d,causal,layer", [(1, 8, True, 0), (37, 8, True, 2), (100, 64, False, 1),
                                              (129, 64, True, 0)])
def test_f32_path_vs_oracle(N, d, causal, layer):
    torch = torch_mod()
    inp = di.prefill_f32(2, 2, N, d, seed=20 + N)
    say(f"case: fp32 prefill B2 H2 N{N} d{d} causal={causal} layer={layer}")
    dev = {k: dev_f32(v) for k, v in inp.items()}
    out = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.6, layer, causal)
    torch.cuda.synchronize()
    ref = oracle.diffattn(inp["q1"], inp["k1"], inp["q2"], inp["k2"], inp["v"], float(np.float32(0.6)), layer, causal)
    assert np.abs(out.cpu().numpy() - ref).max() <= F32_TOL


def test_f32_decode_vs_oracle():
    torch = torch_mod()
    B, H, L, d = 2, 3, 300, 8
    q1, q2 = di.normal_f32(30, "q1", (B, H, d)), di.normal_f32(30, "q2", (B, H, d))
    k1, k2 = di.normal_f32(30, "k1", (B, H, L, d)), di.normal_f32(30, "k2", (B, H, L, d))
    v = di.normal_f32(30, "v", (B, H, L, 2 * d))
    say("case: fp32 decode B2 H3 L300 d8")
    out = da.diffattn_decode(dev_f32(q1), dev_f32(k1), dev_f32(q2), dev_f32(k2), dev_f32(v), 0.8, 1)
    torch.cuda.synchronize()
    ref = oracle.decode(q1, k1, q2, k2, v, float(np.float32(0.8)), 1)
    assert np.abs(out.cpu().numpy() - ref).max() <= F32_TOL


# ---------------------------------------------------------------------------------------------------------------
# bf16 prefill: the workloads, ragged and edge shapes, invariants.
# ---------------------------------------------------------------------------------------------------------------

def test_prefill_n1024_full():
    c = di.CONFIGS["prefill_n1024"]
    inp = di.prefill_bf16(c["B"], c["H"], c["N"], c["d"], c["seed"])
    lam = lam_of(c["lam"])
    say("case: prefill B1 H8 N1024 causal layer 1 (full oracle)")
    got = run_prefill_bf16(inp, lam, c["layer"], c["causal"])
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, c["layer"], c["causal"])
    check_bf16(got, ref, "prefill N1024")


def test_prefill_n4096_full():
    c = di.CONFIGS["prefill_n4096"]
    inp = di.prefill_bf16(c["B"], c["H"], c["N"], c["d"], c["seed"], outliers=True)
    lam = lam_of(c["lam"])
    say("case: prefill B4 H12 N4096 causal layer 12 outliers (full oracle)")
    got = run_prefill_bf16(inp, lam, c["layer"], c["causal"])
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, c["layer"], c["causal"])
    check_bf16(got, ref, "prefill N4096")


def test_prefill_n65536_sampled():
    c = di.CONFIGS["prefill_n65536"]
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    inp = di.prefill_bf16(B, H, N, d, c["seed"])
    lam = lam_of(c["lam"])
    say("case: prefill B1 H16 N65536 causal layer 24 (256 sampled rows)")
    got = run_prefill_bf16(inp, lam, c["layer"], c["causal"])
    fixed = [(h, i) for h in (0, H - 1) for i in (0, 1, 63, 64, 127, 128, 4095, 4096, N - 1)]
    rng = np.random.default_rng(4)
    rand = [(int(rng.integers(H)), int(rng.integers(N))) for _ in range(256 - len(fixed))]
    pairs = fixed + rand
    rows = np.array([h * N + i for h, i in pairs], dtype=np.int64)
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, c["layer"], True, rows=rows)
    sub = got.reshape(B * H * N, 2 * d)[rows]
    check_bf16(sub, ref, "prefill N65536 sampled")


@pytest.mark.parametrize("B,H,N,causal,layer", [
    (2, 8, 1000, True, 1),   # 16 heads: each XCD takes its two heads one at a time
    (3, 8, 700, False, 0),   # 24 heads, not causal
    (4, 8, 2048, True, 2),   # 32 heads
])
def test_prefill_xcd_head_groups(B, H, N, causal, layer):
    """Grids whose head count is a multiple of 8 take each XCD's heads a group at a time (a different order of the
    same items): every row against the oracle."""
    inp = di.prefill_bf16(B, H, N, 64, seed=1300 + N)
    say(f"case: prefill head groups B{B} H{H} N{N} causal={causal} layer={layer}")
    lam = float(np.float32(0.8 if layer == 0 else oracle.lambda_init(layer)))
    got = run_prefill_bf16(inp, lam, layer, causal)
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, layer, causal)
    check_bf16(got, ref, f"prefill head groups N{N}", raw=layer == 0)


@pytest.mark.parametrize("B,H,N,causal,layer", [
    (1, 8, 1024, True, 1),     # the small benchmarked prefill: 4 key splits per row tile
    (1, 2, 1000, True, 0),     # 8 splits of 128 keys, ragged tail
    (2, 1, 1000, False, 2),    # not causal: every row tile has all 8 splits
    (1, 3, 4097, True, 1),     # 5 splits of 832 keys: split boundaries inside row tiles, a one-row tail
    (1, 1, 1500, False, 3),
    (1, 4, 777, True, 2),      # 7 splits of 128 keys
    (1, 1, 2049, True, 0),     # 11 splits of 192 keys
    (1, 1, 8192, True, 2),     # one head: 9 splits
])
def test_prefill_split_vs_oracle(B, H, N, causal, layer):
    """Split-key prefill (diffattn_fwd_split): row tiles whose keys are split across workgroups, including causal
    rows that see no key of a split inside their row tile, merged by log-sum-exp; against the oracle, and against
    diffattn_fwd (the parts are summed in another order)."""
    torch = torch_mod()
    assert da.diffattn_fwd_split_workspace_bytes(B, H, N, 64) > 0   # the case really splits
    inp = di.prefill_bf16(B, H, N, 64, seed=1100 + N)
    say(f"case: prefill split B{B} H{H} N{N} causal={causal} layer={layer}")
    lam = float(np.float32(0.8 if layer == 0 else oracle.lambda_init(layer)))
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    got = da.diffattn_fwd_split(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, layer, causal)
    full = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, layer, causal)
    torch.cuda.synchronize()
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, layer, causal)
    check_bf16(host_bf16(got), ref, f"prefill split N{N}", raw=layer == 0)
    # Both meet the bounds against the exact values, so they are within twice the bounds of each other.
    check_bf16(host_bf16(got), host_bf16(full), f"prefill split N{N} vs diffattn_fwd", raw=layer == 0, scale=2.0)


def test_prefill_split_without_split_is_fwd():
    """When the query tiles fill the GPU the split entry point runs diffattn_fwd's kernel: identical bits."""
    torch = torch_mod()
    B, H, N = 4, 12, 4096
    assert da.diffattn_fwd_split_workspace_bytes(B, H, N, 64) == 0
    inp = {k: dev_bf16(v) for k, v in di.prefill_bf16(B, H, N, 64, seed=1200).items()}
    lam = float(np.float32(oracle.lambda_init(12)))
    a = da.diffattn_fwd_split(inp["q1"], inp["k1"], inp["q2"], inp["k2"], inp["v"], lam, 12, True)
    b = da.diffattn_fwd(inp["q1"], inp["k1"], inp["q2"], inp["k2"], inp["v"], lam, 12, True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("B,H,N,causal,layer", [
    (1, 1, 1, True, 1), (1, 2, 5, True, 0), (2, 1, 31, True, 2), (1, 2, 33, False, 1), (1, 1, 127, True, 0),
    (2, 2, 129, True, 5), (1, 3, 200, False, 0), (1, 1, 257, True, 1), (3, 1, 1000, True, 3),
    (1, 2, 1000, False, 7),
])
def test_prefill_ragged(B, H, N, causal, layer):
    inp = di.prefill_bf16(B, H, N, 64, seed=100 + N)
    lam = 0.8 if layer == 0 else lam_of(("lambda_init", layer))
    say(f"case: prefill ragged B{B} H{H} N{N} causal={causal} layer={layer}")
    got = run_prefill_bf16(inp, lam, layer, causal)
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, layer, causal)
    check_bf16(got, ref, f"prefill N{N}", raw=layer == 0)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_row_sums_with_unit_values(causal):
    """V all ones and raw output: every channel equals the row sum of the difference map, 1 - lambda.

    The kernel multiplies V by bf16-rounded probabilities (relative error <= u = 2^-8 each: bf16 keeps 8 significant
    bits) and divides by the fp32 sum of the unrounded ones, so each map's row comes out as sum(round(p)) / sum(p) =
    1 + e with |e| <= u; the output 1 - lambda then carries at most (1 + lambda) u plus half a bf16 ulp of 0.2 (2^-11):
    7.5e-3 for lambda 0.8."""
    B, H, N = 1, 2, 300
    inp = di.prefill_bf16(B, H, N, 64, seed=7)
    inp["v"] = di.f32_to_bf16_bits(np.ones((B, H, N, 128), dtype=np.float32))
    say(f"case: prefill unit values N{N} causal={causal}")
    lam = float(np.float32(0.8))
    got = run_prefill_bf16(inp, lam, 0, causal)
    err = np.abs(got - (1.0 - lam))
    bound = (1.0 + lam) * 2.0 ** -8 + 2.0 ** -11
    say(f"row sums: max-abs {err.max():.3e} mean-abs {err.mean():.3e} (bound {bound:.3e})")
    assert err.max() <= bound


def test_prefill_identity_values_extract_map():
    """V = [I | 0] (N <= 128): the raw output's first N channels are the difference map w = a - lambda b; its signs
    match.  Each output is then one weight: the kernel forms round(p1_c) / sum(p1) - lambda round(p2_c) / sum(p2)
    (bf16 probabilities, unit roundoff u = 2^-8, over fp32 sums of the unrounded ones) and rounds it to bf16, so
    |got - w| <= u (a + lambda b) + u |w| per weight, with a and b the two maps (the oracle at lambda = 0)."""
    B, H, N = 1, 1, 96
    inp = di.prefill_bf16(B, H, N, 64, seed=8)
    eye = np.zeros((B, H, N, 128), dtype=np.float32)
    eye[0, 0, :, :N] = np.eye(N, dtype=np.float32)
    inp["v"] = di.f32_to_bf16_bits(eye)
    say("case: prefill identity values N96")
    lam = float(np.float32(0.8))
    got = run_prefill_bf16(inp, lam, 0, True)[0, 0, :, :N]
    f = widen(inp)
    _, ref_w = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, 0, True, want_diff=True)
    _, a = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], 0.0, 0, True, want_diff=True)
    _, b = oracle.diffattn(f["q2"], f["k2"], f["q1"], f["k1"], f["v"], 0.0, 0, True, want_diff=True)
    ref_w, a, b = ref_w[0, 0], a[0, 0], b[0, 0]
    u = 2.0 ** -8
    bound = u * (a + lam * b) + u * np.abs(ref_w) + 1e-6
    err = np.abs(got - ref_w)
    say(f"difference map: max-abs {err.max():.3e}, max err / bound {(err / bound).max():.3f}")
    assert (err <= bound).all()
    clear = np.abs(ref_w) > 1e-2  # signs of weights well away from zero must agree
    assert np.array_equal(np.sign(got[clear]), np.sign(ref_w[clear]))


def test_prefill_lambda_zero_and_layer_ratio():
    """lambda = 0 is plain attention (oracle); outputs at two layers differ by the ratio of their scales."""
    inp = di.prefill_bf16(1, 2, 333, 64, seed=9)
    f = widen(inp)
    say("case: prefill lambda 0 N333")
    got0 = run_prefill_bf16(inp, 0.0, 1, True)
    check_bf16(got0, oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], 0.0, 1, True), "lambda 0")
    got_a = run_prefill_bf16(inp, 0.5, 2, True)
    got_b = run_prefill_bf16(inp, 0.5, 30, True)
    ratio = (1 - oracle.lambda_init(30)) / (1 - oracle.lambda_init(2))
    big = np.abs(got_a) > 0.05
    rel = np.abs(got_b[big] / got_a[big] - ratio) / ratio
    assert np.median(rel) < 1e-2 and rel.max() < 5e-2


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_identical_halves(causal):
    """Q2 = Q1 and K2 = K1: both maps are the same softmax a, the raw output is (1 - lambda) a V, and after the RMS
    norm it is softmax attention normalised on its own, whatever lambda < 1 (the factor 1 - lambda only moves eps:
    y = aV / sqrt(mean((aV)^2) + 1e-5 / (1 - lambda)^2) (1 - lambda_init)).  Reference: that closed form in float64
    from numpy, independent of the oracle."""
    B, H, N, layer = 1, 3, 333, 5
    inp = di.prefill_bf16(B, H, N, 64, seed=23)
    inp["q2"] = inp["q1"].copy()
    inp["k2"] = inp["k1"].copy()
    lam = float(np.float32(0.55))
    say(f"case: prefill identical halves N{N} causal={causal} layer {layer}")
    got = run_prefill_bf16(inp, lam, layer, causal)
    f = widen(inp)
    q, k, v = (f[x].astype(np.float64) for x in ("q1", "k1", "v"))
    s_ = np.einsum("bhid,bhjd->bhij", q, k) / 8.0
    if causal:
        s_ = np.where(np.tril(np.ones((N, N), dtype=bool)), s_, -np.inf)
    a = np.exp(s_ - s_.max(axis=-1, keepdims=True))
    a /= a.sum(axis=-1, keepdims=True)
    o = a @ v
    ref = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + 1e-5 / (1.0 - lam) ** 2) * (1.0 - oracle.lambda_init(layer))
    check_bf16(got, ref, "identical halves")


def test_prefill_odd_length_4097():
    """N = 4097: one key past a whole number of tiles and one row past a whole number of row tiles (causal, the
    4K-context workload's layer and outlier rows), against the full oracle."""
    B, H, N, layer = 1, 2, 4097, 12
    inp = di.prefill_bf16(B, H, N, 64, seed=41, outliers=True)
    lam = lam_of(("lambda_init", layer))
    say(f"case: prefill B{B} H{H} N{N} causal layer {layer} outliers (full oracle)")
    got = run_prefill_bf16(inp, lam, layer, True)
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, layer, True)
    check_bf16(got, ref, "prefill N4097")


@pytest.mark.parametrize("causal,layer", [(True, 1), (False, 0)])
def test_prefill_growing_scores(causal, layer):
    """Map-1 scores that grow by half a nat per key (about 216 in log2 units over 300 keys) in head 0: the
    probabilities at the first tile's offset would overflow, so the rows are recomputed at their final offsets.
    Head 1 and map 2 keep ordinary N(0,1) scores."""
    B, H, N = 1, 2, 300
    inp = di.prefill_bf16(B, H, N, 64, seed=11)
    q1 = di.bf16_bits_to_f32(inp["q1"]).copy()
    k1 = di.bf16_bits_to_f32(inp["k1"]).copy()
    q1[0, 0, :, 0] = 64.0                                   # s_ij = q1_i . k1_j / 8 = j / 2 + noise
    k1[0, 0, :, 0] = np.arange(N, dtype=np.float32) / 16.0
    inp["q1"] = di.f32_to_bf16_bits(q1)
    inp["k1"] = di.f32_to_bf16_bits(k1)
    lam = 0.8 if layer == 0 else lam_of(("lambda_init", layer))
    say(f"case: prefill growing scores N{N} causal={causal} layer={layer}")
    got = run_prefill_bf16(inp, lam, layer, causal)
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, layer, causal)
    check_bf16(got, ref, "growing scores", raw=layer == 0)


def test_prefill_deterministic():
    torch = torch_mod()
    inp = di.prefill_bf16(2, 3, 700, 64, seed=10)
    say("case: prefill determinism N700")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    a = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.7, 4, True)
    b = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.7, 4, True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------------------------------------------
# bf16 decode
# ---------------------------------------------------------------------------------------------------------------

def run_decode_bf16(inp, lam, layer):
    torch = torch_mod()
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    out = da.diffattn_decode(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, layer)
    torch.cuda.synchronize()
    return host_bf16(out)


@pytest.mark.parametrize("B,H,L,layer", [(1, 1, 1, 1), (2, 3, 7, 0), (1, 2, 64, 1), (2, 2, 1000, 2),
                                         (1, 4, 1025, 1), (3, 1, 4097, 0), (1, 1, 20000, 1)])
def test_decode_ragged(B, H, L, layer):
    inp = di.decode_bf16(B, H, L, 64, seed=200 + L)
    say(f"case: decode B{B} H{H} L{L} layer={layer}")
    got = run_decode_bf16(inp, 0.8, layer)
    f = widen(inp)
    ref = oracle.decode(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], float(np.float32(0.8)), layer)
    check_bf16(got, ref, f"decode L{L}", raw=layer == 0)


def test_decode_l8192_full():
    c = di.CONFIGS["decode_l8192"]
    B, H, L, d = c["B"], c["H"], c["L"], c["d"]
    inp = di.decode_bf16(B, H, L, d, c["seed"])
    say("case: decode B64 H16 L8192 layer 1 (full oracle)")
    got = run_decode_bf16(inp, lam_of(c["lam"]), c["layer"])
    errs = []
    for b0 in range(0, B, 8):   # widen and check 8 sequences at a time to bound host memory
        f = {k: di.bf16_bits_to_f32(v[b0:b0 + 8]) for k, v in inp.items()}
        ref = oracle.decode(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam_of(c["lam"]), c["layer"])
        errs.append(np.abs(got[b0:b0 + 8] - ref))
    err = np.concatenate(errs)
    say(f"decode L8192: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN


def test_decode_matches_prefill_last_row():
    """The decode of token L-1 equals the causal prefill's last row (same inputs, both on the GPU)."""
    B, H, L = 1, 2, 513
    inp = di.prefill_bf16(B, H, L, 64, seed=13)
    say("case: decode vs prefill last row L513")
    pre = run_prefill_bf16(inp, 0.8, 1, True)[:, :, -1]
    dinp = {"q1": inp["q1"][:, :, -1], "q2": inp["q2"][:, :, -1], "k1": inp["k1"], "k2": inp["k2"], "v": inp["v"]}
    dec = run_decode_bf16(dinp, 0.8, 1)
    assert np.abs(pre - dec).max() <= 2e-2


# ---------------------------------------------------------------------------------------------------------------
# One lambda per head (diffattn_fwd_heads / diffattn_decode_heads)
# ---------------------------------------------------------------------------------------------------------------

LAM_HEADS = np.array([0.05, 0.5, 0.95], dtype=np.float32)


def dev_lam(lam):
    return dev_f32(np.asarray(lam, dtype=np.float32))


@pytest.mark.parametrize("N,causal,layer", [(300, True, 2), (129, False, 0)])
def test_prefill_bf16_lambda_per_head(N, causal, layer):
    torch = torch_mod()
    inp = di.prefill_bf16(2, 3, N, 64, seed=400 + N)
    say(f"case: prefill bf16 per-head lambda B2 H3 N{N} causal={causal} layer={layer}")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    out = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dev_lam(LAM_HEADS), layer, causal)
    torch.cuda.synchronize()
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], LAM_HEADS.astype(np.float64), layer, causal)
    check_bf16(host_bf16(out), ref, f"prefill per-head N{N}", raw=layer == 0)


@pytest.mark.parametrize("N,causal,layer", [(1000, True, 2), (777, False, 0)])
def test_prefill_split_lambda_per_head(N, causal, layer):
    """diffattn_fwd_split with one lambda per head (B1 H3: 8 or 5 key splits), against the oracle."""
    torch = torch_mod()
    inp = di.prefill_bf16(1, 3, N, 64, seed=420 + N)
    assert da.diffattn_fwd_split_workspace_bytes(1, 3, N, 64) > 0
    say(f"case: prefill split per-head lambda B1 H3 N{N} causal={causal} layer={layer}")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    out = da.diffattn_fwd_split(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dev_lam(LAM_HEADS), layer,
                                causal)
    torch.cuda.synchronize()
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], LAM_HEADS.astype(np.float64), layer, causal)
    check_bf16(host_bf16(out), ref, f"prefill split per-head N{N}", raw=layer == 0)


def test_f32_lambda_per_head():
    torch = torch_mod()
    inp = di.prefill_f32(2, 3, 37, 8, seed=410)
    say("case: fp32 per-head lambda B2 H3 N37 d8")
    dev = {k: dev_f32(v) for k, v in inp.items()}
    out = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dev_lam(LAM_HEADS), 1, True)
    torch.cuda.synchronize()
    ref = oracle.diffattn(inp["q1"], inp["k1"], inp["q2"], inp["k2"], inp["v"], LAM_HEADS.astype(np.float64), 1, True)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref).max()
    say(f"fp32 per-head: max-abs {err:.3e}")
    assert err <= F32_TOL


def test_decode_bf16_lambda_per_head():
    torch = torch_mod()
    inp = di.decode_bf16(2, 3, 1500, 64, seed=420)
    say("case: decode bf16 per-head lambda B2 H3 L1500")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    out = da.diffattn_decode(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dev_lam(LAM_HEADS), 1)
    torch.cuda.synchronize()
    f = widen(inp)
    ref = oracle.decode(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], LAM_HEADS.astype(np.float64), 1)
    check_bf16(host_bf16(out), ref, "decode per-head L1500")


def test_uniform_lambda_heads_equal_scalar_lambda():
    """A per-head array holding one value gives bit-identical output to the scalar entry point."""
    torch = torch_mod()
    inp = di.prefill_bf16(1, 3, 200, 64, seed=430)
    say("case: uniform per-head lambda == scalar lambda (prefill N200, decode L200)")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    lam = float(np.float32(0.625))
    a = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, 3, True)
    b = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dev_lam([lam] * 3), 3, True)
    q1, q2 = dev["q1"][:, :, -1].contiguous(), dev["q2"][:, :, -1].contiguous()
    c = da.diffattn_decode(q1, dev["k1"], q2, dev["k2"], dev["v"], lam, 3)
    e = da.diffattn_decode(q1, dev["k1"], q2, dev["k2"], dev["v"], dev_lam([lam] * 3), 3)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), e.view(torch.int16))


# ---------------------------------------------------------------------------------------------------------------
# Variable-length and multi-token decode (diffattn_decode_varlen)
# ---------------------------------------------------------------------------------------------------------------

def varlen_reference(f, T, L, lens, lam, layer):
    """Oracle: sequence b's cache cut to its clamped length, its T new tokens as the last T query rows (end-aligned
    causal mask)."""
    B, H = f["k1"].shape[:2]
    out = np.zeros((B, H, T, 128))
    for b in range(B):
        Lb = L if lens is None else min(max(int(lens[b]), T), L)
        sl = (slice(b, b + 1), slice(None), slice(0, Lb))
        out[b] = oracle.diffattn(f["q1"][b:b + 1], f["k1"][sl], f["q2"][b:b + 1], f["k2"][sl], f["v"][sl], lam,
                                 layer, True)[0]
    return out


def varlen_inputs(B, H, T, L, seed):
    kv = di.decode_bf16(B, H, L, 64, seed=seed)
    q = di.prefill_bf16(B, H, T, 64, seed=seed + 1)
    return {"q1": q["q1"], "q2": q["q2"], "k1": kv["k1"], "k2": kv["k2"], "v": kv["v"]}


@pytest.mark.parametrize("B,H,T,L,lens,layer", [
    (3, 2, 1, 2000, [1, 777, 2000], 1),
    (2, 2, 4, 300, None, 0),
    (3, 2, 16, 1000, [16, 501, 1000], 2),
    (2, 1, 5, 5, None, 1),
    (2, 3, 7, 4500, [4500, 9], 3),
    (1, 2, 2, 20000, [19999], 1),
    (2, 1, 1, 20000, [20000, 5], 1),   # 313 splits, merged in two levels; the short sequence's later groups are empty
])
def test_decode_varlen_vs_oracle(B, H, T, L, lens, layer):
    torch = torch_mod()
    inp = varlen_inputs(B, H, T, L, seed=600 + T + L)
    say(f"case: decode varlen B{B} H{H} T{T} L{L} lens={lens} layer={layer}")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    ldev = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    out = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.8, layer, lens=ldev)
    torch.cuda.synchronize()
    ref = varlen_reference(widen(inp), T, L, lens, float(np.float32(0.8)), layer)
    check_bf16(host_bf16(out), ref, f"decode varlen T{T} L{L}", raw=layer == 0)


def ragged_lens(rng, B, T, L, lo):
    """Seeded ragged lengths in [lo, L]: a mix of the shortest, the longest and uniform draws, plus (lo = T only)
    values outside [T, L], which the device clamps."""
    lens = rng.integers(lo, L + 1, size=B)
    pick = rng.random(B)
    lens[pick < 0.15] = lo
    lens[(pick >= 0.15) & (pick < 0.3)] = L
    lens[(pick >= 0.3) & (pick < 0.35)] = L + 7
    if lo == T:
        lens[(pick >= 0.35) & (pick < 0.4)] = -3
    return lens.astype(np.int32)


@pytest.mark.parametrize("B,H,T,L,lo,layer", [
    (8, 16, 4, 1000, 4, 1),      # 128 items: the balanced cut, several waves per sequence
    (128, 1, 1, 700, 1, 0),      # short sequences: waves spanning many items
    (16, 8, 16, 2048, 16, 2),
    (130, 1, 3, 65, 11, 1),      # lengths scanned in three rounds of 64 lanes
    (512, 1, 1, 40, 1, 1),       # the most sequences the balanced cut takes
    (513, 1, 2, 40, 2, 1),       # one more: the fixed plan
])
def test_decode_ragged_balanced_vs_oracle(B, H, T, L, lo, layer):
    """Ragged caches with at least 128 (sequence, head) items take the balanced plan: the keys of all items cut into
    equal ranges, one per wave, merged per item.  Against the oracle, every item.

    The B130 case draws lengths of at least 11, so that every query sees 9 keys or more: with T = 3 and lengths of 3,
    a query that sees two keys under nearly equal maps (a = 0.42 / 0.58, b = 0.44 / 0.56 at this seed) has a raw
    output of RMS 0.13, and the normalisation magnifies the bf16 rounding of its probabilities to 2.13e-2, above the
    2e-2 bound, on the fixed plan as on the balanced one; a CPU model of the kernel's rounding (bf16 probabilities,
    fp32 sums, bf16 output) gives the same 2.13e-2."""
    torch = torch_mod()
    rng = np.random.default_rng(640 + B + T)
    lens = ragged_lens(rng, B, T, L, lo)
    inp = varlen_inputs(B, H, T, L, seed=650 + B + T)
    say(f"case: decode ragged balanced B{B} H{H} T{T} L{L} lens {lens.min()}..{lens.max()} layer={layer}")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    ldev = torch.from_numpy(lens).to("cuda:0")
    out = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.8, layer, lens=ldev)
    torch.cuda.synchronize()
    ref = varlen_reference(widen(inp), T, L, lens, float(np.float32(0.8)), layer)
    check_bf16(host_bf16(out), ref, f"decode ragged balanced B{B} T{T} L{L}", raw=layer == 0)


def test_decode_varlen_per_head_lambda():
    torch = torch_mod()
    inp = varlen_inputs(2, 3, 3, 640, seed=650)
    say("case: decode varlen per-head lambda B2 H3 T3 L640 lens [640, 100]")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    ldev = torch.tensor([640, 100], dtype=torch.int32, device="cuda:0")
    out = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dev_lam(LAM_HEADS), 1,
                                    lens=ldev)
    torch.cuda.synchronize()
    ref = varlen_reference(widen(inp), 3, 640, [640, 100], LAM_HEADS.astype(np.float64), 1)
    check_bf16(host_bf16(out), ref, "decode varlen per-head")


def test_decode_ragged_balanced_per_head_lambda():
    """Per-head lambda on the balanced plan (B4 H32: 128 items), one value per head from 0 to 0.95, against the oracle;
    and the scalar entry point's bits when every head holds the same value."""
    torch = torch_mod()
    B, H, T, L = 4, 32, 2, 900
    inp = varlen_inputs(B, H, T, L, seed=660)
    lens = np.array([900, 37, 512, 899], dtype=np.int32)
    lam_h = np.linspace(0.0, 0.95, H).astype(np.float32)
    say(f"case: decode ragged balanced per-head lambda B{B} H{H} T{T} L{L} lens {lens.tolist()}")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    ldev = torch.from_numpy(lens).to("cuda:0")
    out = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dev_lam(lam_h), 2,
                                    lens=ldev)
    one = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"],
                                    dev_lam(np.full(H, 0.6, dtype=np.float32)), 2, lens=ldev)
    scalar = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.6, 2, lens=ldev)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), scalar.view(torch.int16))
    ref = varlen_reference(widen(inp), T, L, lens, lam_h.astype(np.float64), 2)
    check_bf16(host_bf16(out), ref, "decode ragged balanced per-head")


def strided_caches(dev, layout):
    """Views of the same cache rows in another memory layout: 'token' = each cache token-major ([B][L][H][w]);
    'packed' = K1, K2 and V of a row side by side in one [B][L][H][d + d + 2d] buffer."""
    torch = torch_mod()
    k1, k2, v = dev["k1"], dev["k2"], dev["v"]
    if layout == "token":
        return tuple(t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (k1, k2, v))
    B, H, L, d = k1.shape
    buf = torch.empty(B, L, H, 4 * d, dtype=k1.dtype, device=k1.device)
    buf[..., :d] = k1.permute(0, 2, 1, 3)
    buf[..., d:2 * d] = k2.permute(0, 2, 1, 3)
    buf[..., 2 * d:] = v.permute(0, 2, 1, 3)
    return tuple(x.permute(0, 2, 1, 3) for x in (buf[..., :d], buf[..., d:2 * d], buf[..., 2 * d:]))


@pytest.mark.parametrize("layout,B,H,T,L,lens", [
    ("token", 2, 3, 1, 2000, [2000, 777]),
    ("token", 2, 2, 4, 1500, None),
    ("packed", 3, 2, 1, 1100, None),
    ("packed", 2, 2, 5, 4100, [4100, 31]),
    ("token", 8, 16, 2, 600, [600, 2, 599, 300, 45, 600, 128, 1]),   # 128 heads: the balanced plan
])
def test_decode_strided_equals_contiguous(layout, B, H, T, L, lens):
    """Strided caches read in place give the contiguous call's bits (same kernels, same split plan)."""
    torch = torch_mod()
    inp = varlen_inputs(B, H, T, L, seed=900 + T + L)
    say(f"case: decode strided {layout} B{B} H{H} T{T} L{L} lens={lens}")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    ldev = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    k1s, k2s, vs = strided_caches(dev, layout)
    assert not k1s.is_contiguous()
    a = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.8, 1, lens=ldev)
    b = da.diffattn_decode_strided(dev["q1"], k1s, dev["q2"], k2s, vs, 0.8, 1, lens=ldev)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_strided_vs_oracle():
    torch = torch_mod()
    B, H, T, L, lens = 2, 2, 3, 900, [900, 77]
    inp = varlen_inputs(B, H, T, L, seed=950)
    say(f"case: decode strided packed vs oracle B{B} H{H} T{T} L{L} lens={lens}, per-head lambda")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    ldev = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    k1s, k2s, vs = strided_caches(dev, "packed")
    lam = LAM_HEADS[:H]
    out = da.diffattn_decode_strided(dev["q1"], k1s, dev["q2"], k2s, vs, dev_lam(lam), 2, lens=ldev)
    torch.cuda.synchronize()
    ref = varlen_reference(widen(inp), T, L, lens, lam.astype(np.float64), 2)
    check_bf16(host_bf16(out), ref, "decode strided packed")


def test_decode_varlen_single_token_equals_decode():
    """T = 1 without lengths runs the decode kernels: bit-identical to diffattn_decode."""
    torch = torch_mod()
    inp = di.decode_bf16(2, 2, 3000, 64, seed=660)
    say("case: decode varlen T1 == decode, B2 H2 L3000")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    a = da.diffattn_decode(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.8, 1)
    b = da.diffattn_decode_varlen(dev["q1"][:, :, None], dev["k1"], dev["q2"][:, :, None], dev["k2"], dev["v"], 0.8,
                                  1)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b[:, :, 0].contiguous().view(torch.int16))


def test_decode_varlen_matches_prefill_rows():
    """T new tokens at the end of a full cache equal the causal prefill's last T rows."""
    torch = torch_mod()
    B, H, N, T = 1, 2, 700, 9
    inp = di.prefill_bf16(B, H, N, 64, seed=670)
    say("case: decode varlen T9 == prefill last 9 rows, N700")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    pre = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.8, 1, True)
    dec = da.diffattn_decode_varlen(dev["q1"][:, :, N - T:].contiguous(), dev["k1"],
                                    dev["q2"][:, :, N - T:].contiguous(), dev["k2"], dev["v"], 0.8, 1)
    torch.cuda.synchronize()
    assert np.abs(host_bf16(pre)[:, :, N - T:] - host_bf16(dec)).max() <= 2e-2


# ---------------------------------------------------------------------------------------------------------------
# Strided prefill (diffattn_fwd_strided): operands read out of packed projection outputs
# ---------------------------------------------------------------------------------------------------------------

def test_prefill_strided_packed_projection():
    """q1, k1, q2, k2, v as views of one [B][N][H][6][64] projection output, out into a [B][N][H][128] buffer:
    bit-identical to the contiguous call, and within tolerance of the oracle."""
    torch = torch_mod()
    B, H, N = 2, 3, 333
    inp = di.prefill_bf16(B, H, N, 64, seed=700)
    say("case: strided prefill from a packed projection, B2 H3 N333 causal layer 2")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    proj = torch.empty((B, N, H, 6, 64), dtype=torch.bfloat16, device="cuda:0")
    for i, k in enumerate(("q1", "k1", "q2", "k2")):
        proj[:, :, :, i] = dev[k].permute(0, 2, 1, 3)
    proj[:, :, :, 4:6] = dev["v"].permute(0, 2, 1, 3).reshape(B, N, H, 2, 64)
    views = [proj[:, :, :, i].permute(0, 2, 1, 3) for i in range(4)]
    vview = proj[:, :, :, 4:6].reshape(B, N, H, 128).permute(0, 2, 1, 3)
    obuf = torch.zeros((B, N, H, 128), dtype=torch.bfloat16, device="cuda:0")
    oview = obuf.permute(0, 2, 1, 3)
    da.diffattn_fwd_strided(views[0], views[1], views[2], views[3], vview, 0.7, 2, True, out=oview)
    ref_dev = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.7, 2, True)
    torch.cuda.synchronize()
    assert torch.equal(oview.contiguous().view(torch.int16), ref_dev.view(torch.int16))
    f = widen(inp)
    ref = oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], float(np.float32(0.7)), 2, True)
    check_bf16(host_bf16(oview.contiguous()), ref, "strided prefill")


def test_prefill_strided_at_offset_limit():
    """K1 | K2 | V packed in rows of 8192 elements (16 KiB).  N = 261887 is the largest N whose per-head buffer
    range for the direct loads, (N + 256) rows of that stride plus one row of V, fits 32-bit offsets: bit-identical
    to the contiguous call, sampled rows (the last ones read the highest offsets) within tolerance of the oracle,
    and N + 1 rejected as a shape error before any launch."""
    torch = torch_mod()
    N, RS, layer = 261887, 8192, 3
    assert (N + 256) * RS * 2 + 256 <= 2**32 - 1 < (N + 257) * RS * 2 + 256
    say(f"case: strided prefill at the 32-bit offset limit, N{N} row stride {RS} causal layer {layer}")
    g = torch.Generator(device="cuda:0").manual_seed(900)
    buf = torch.empty((N + 1, RS), dtype=torch.bfloat16, device="cuda:0")
    buf[:, :256] = torch.randn((N + 1, 256), generator=g, device="cuda:0").to(torch.bfloat16)
    q = torch.randn((2, 1, 1, N, 64), generator=g, device="cuda:0").to(torch.bfloat16)
    lam = lam_of(("lambda_init", layer))

    def views(n):
        part = lambda lo, w: buf[:n, lo:lo + w].unsqueeze(0).unsqueeze(0)   # [1][1][n][w], row stride RS
        return part(0, 64), part(64, 64), part(128, 128)

    k1v, k2v, vv = views(N)
    got = da.diffattn_fwd_strided(q[0], k1v, q[1], k2v, vv, lam, layer, True)
    ref_dev = da.diffattn_fwd(q[0], k1v.contiguous(), q[1], k2v.contiguous(), vv.contiguous(), lam, layer, True)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref_dev.view(torch.int16))
    rows = np.array([0, 1, 127, 128, 4096, N // 2, N - 257, N - 256, N - 33, N - 32, N - 1]
                    + [int(x) for x in np.random.default_rng(900).integers(0, N, 21)], dtype=np.int64)
    host = lambda t: t.float().cpu().numpy()
    ref = oracle.diffattn(host(q[0]), host(k1v), host(q[1]), host(k2v), host(vv), lam, layer, True, rows=rows)
    check_bf16(host_bf16(got).reshape(N, 128)[rows], ref, "strided prefill at the offset limit")
    q_big = torch.zeros((1, 1, N + 1, 64), dtype=torch.bfloat16, device="cuda:0")
    k1b, k2b, vb = views(N + 1)
    with pytest.raises(da.DiffAttnError) as e:
        da.diffattn_fwd_strided(q_big, k1b, q_big, k2b, vb, lam, layer, True)
    assert e.value.status == -2


def test_prefill_strided_interleaved_heads():
    """Q and K with the two halves interleaved per head ([B][N][2H][64], half 1 at even, half 2 at odd heads),
    non-causal, per-head lambda: bit-identical to the contiguous call."""
    torch = torch_mod()
    B, H, N = 1, 4, 200
    inp = di.prefill_bf16(B, H, N, 64, seed=710)
    say("case: strided prefill, interleaved query/key halves, B1 H4 N200 non-causal per-head lambda")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    q = torch.empty((B, N, 2 * H, 64), dtype=torch.bfloat16, device="cuda:0")
    k = torch.empty_like(q)
    q[:, :, 0::2] = dev["q1"].permute(0, 2, 1, 3)
    q[:, :, 1::2] = dev["q2"].permute(0, 2, 1, 3)
    k[:, :, 0::2] = dev["k1"].permute(0, 2, 1, 3)
    k[:, :, 1::2] = dev["k2"].permute(0, 2, 1, 3)
    lam = dev_lam([0.2, 0.4, 0.6, 0.8])
    got = da.diffattn_fwd_strided(q[:, :, 0::2].permute(0, 2, 1, 3), k[:, :, 0::2].permute(0, 2, 1, 3),
                                  q[:, :, 1::2].permute(0, 2, 1, 3), k[:, :, 1::2].permute(0, 2, 1, 3), dev["v"],
                                  lam, 0, False)
    want = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, 0, False)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


# ---------------------------------------------------------------------------------------------------------------
# Paged decode (diffattn_decode_paged): caches in fixed-size pages of a shared pool, found through a block table.
# The paging is layout only, so the reference is the varlen decode (and the oracle) on the cache gathered page by
# page through the same table.
# ---------------------------------------------------------------------------------------------------------------

def paged_case(B, H, T, P, max_pages, lens, seed, bad_entries=False):
    """Pools [num_pages][H][P][.] holding each sequence's pages in a random order (unused pages and table tails hold
    junk), the int32 block table, and the contiguous [B][H][L][.] caches gathered through the clamped table."""
    rng = np.random.default_rng(seed)
    L = P * max_pages
    inp = varlen_inputs(B, H, T, L, seed)
    need = [max_pages if lens is None else -(-min(max(int(lens[b]), T), L) // P) for b in range(B)]
    num_pages = sum(need) + 3
    perm = rng.permutation(num_pages)
    junk = di.decode_bf16(1, num_pages * H, P, 64, seed=seed + 7)
    pools = {"k1": junk["k1"].reshape(num_pages, H, P, 64).copy(), "k2": junk["k2"].reshape(num_pages, H, P, 64).copy(),
             "v": junk["v"].reshape(num_pages, H, P, 128).copy()}
    table = rng.integers(-1000, 1000, size=(B, max_pages)).astype(np.int32)   # tails: never read
    i = 0
    for b in range(B):
        for j in range(need[b]):
            pg = int(perm[i])
            i += 1
            table[b, j] = pg
            for k in pools:
                pools[k][pg] = inp[k][b, :, j * P:(j + 1) * P]
    if bad_entries:   # in-use entries outside the pool: clamped on the device to [0, num_pages)
        table[0, 0] = -7
        table[B - 1, need[B - 1] - 1] = num_pages + 5
    gathered = {k: np.zeros_like(inp[k]) for k in ("k1", "k2", "v")}
    for b in range(B):
        for j in range(need[b]):
            pg = min(max(int(table[b, j]), 0), num_pages - 1)
            for k in gathered:
                gathered[k][b, :, j * P:(j + 1) * P] = pools[k][pg]
    cont = {"q1": inp["q1"], "q2": inp["q2"], **gathered}
    return cont, pools, table, L


@pytest.mark.parametrize("B,H,T,P,max_pages,lens,layer,bad", [
    (3, 2, 1, 16, 40, [1, 300, 640], 1, False),
    (2, 3, 4, 64, 20, None, 0, False),
    (2, 2, 16, 128, 9, [1100, 17], 2, False),
    (4, 2, 3, 256, 33, [8448, 5000, 3, 100], 1, False),
    (2, 2, 2, 32, 10, [320, 200], 1, True),
    (8, 16, 4, 16, 20, [320, 4, 100, 17, 319, 64, 250, 200], 1, False),   # 128 heads: the balanced plan
])
def test_decode_paged(B, H, T, P, max_pages, lens, layer, bad):
    torch = torch_mod()
    say(f"case: decode paged B{B} H{H} T{T} page {P} x {max_pages} lens={lens} layer={layer} bad={bad}")
    cont, pools, table, L = paged_case(B, H, T, P, max_pages, lens, seed=700 + T + P, bad_entries=bad)
    dev = {k: dev_bf16(v) for k, v in cont.items()}
    pdev = {k: dev_bf16(v) for k, v in pools.items()}
    tdev = torch.from_numpy(table).to("cuda:0")
    ldev = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    assert (da.diffattn_decode_paged_workspace_bytes(B, H, T, max_pages, P, 64) ==
            da.diffattn_decode_varlen_workspace_bytes(B, H, T, L, 64))
    out = da.diffattn_decode_paged(dev["q1"], pdev["k1"], dev["q2"], pdev["k2"], pdev["v"], tdev, 0.8, layer,
                                   lens=ldev)
    ref_dev = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.8, layer, lens=ldev)
    torch.cuda.synchronize()
    # Same kernels and split plan on the same rows: identical bits.
    assert torch.equal(out.view(torch.int16), ref_dev.view(torch.int16))
    ref = varlen_reference(widen(cont), T, L, lens, float(np.float32(0.8)), layer)
    check_bf16(host_bf16(out), ref, f"decode paged T{T} page {P}", raw=layer == 0)


def test_decode_multi_token_long_splits():
    """Multi-token decode at the benchmarked size (B64 H16 T4, caches padded to 8192 rows with seeded ragged lengths
    in [4096, 8192]), where the balanced plan cuts the keys of all 1024 heads into 2048 equal ranges of about 3100
    keys (up to 32 states per head in the workspace): padded and paged (16-row pages of a shuffled pool) give
    identical bits, and sampled sequences match the oracle."""
    torch = torch_mod()
    B, H, T, L, P = 64, 16, 4, 8192, 16
    inp = varlen_inputs(B, H, T, L, seed=880)
    lens = np.random.default_rng(881).integers(L // 2, L + 1, size=B).astype(np.int32)
    say(f"case: decode multi-token long splits B{B} H{H} T{T} L{L} lens {lens.min()}..{lens.max()} page {P}")
    assert da.diffattn_decode_varlen_workspace_bytes(B, H, T, L, 64) == B * H * T * 32 * 1040
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    ldev = torch.from_numpy(lens).to("cuda:0")
    out = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.8, 1, lens=ldev)
    torch.cuda.synchronize()
    for k in ("k1", "k2", "v"):
        del dev[k]
    max_pages = L // P
    perm = np.random.default_rng(882).permutation(B * max_pages)
    pools = {}
    for k in ("k1", "k2", "v"):
        w = inp[k].shape[-1]
        pg = inp[k].reshape(B, H, max_pages, P, w).transpose(0, 2, 1, 3, 4).reshape(B * max_pages, H, P, w)
        pool = np.empty_like(pg)
        pool[perm] = pg
        pools[k] = dev_bf16(pool)
        del pg, pool
    table = torch.from_numpy(perm.reshape(B, max_pages).astype(np.int32)).to("cuda:0")
    outp = da.diffattn_decode_paged(dev["q1"], pools["k1"], dev["q2"], pools["k2"], pools["v"], table, 0.8, 1,
                                    lens=ldev)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), outp.view(torch.int16))
    got = host_bf16(out)
    for b in (0, 31, 63):
        f = widen({k: v[b:b + 1] for k, v in inp.items()})
        ref = varlen_reference(f, T, L, lens[b:b + 1], float(np.float32(0.8)), 1)
        check_bf16(got[b:b + 1], ref, f"decode multi-token long splits b{b} len {lens[b]}")


@pytest.mark.parametrize("T,paged,layer", [(2, False, 0), (16, False, 1), (2, True, 1), (16, True, 0)])
def test_decode_multi_token_rescale(T, paged, layer):
    """Multi-token decode with map-1 scores that grow inside every split (half a nat per key), so the online softmax
    moves its offset and rescales O and l on tiles after the first one, with N(0,1) values already accumulated;
    padded and paged caches against the oracle."""
    torch = torch_mod()
    B, H, P, max_pages, lens = ramp_cases.CASE
    L = P * max_pages
    inp = ramp_cases.ramp_inputs(B, H, T, L, seed=780 + T)
    f = widen(inp)
    ramp_cases.assert_ramp_forces_rescales(f, T, lens)
    say(f"case: decode multi-token rescale B{B} H{H} T{T} L{L} lens={lens} paged={paged} layer={layer}")
    lam = 0.8 if layer == 0 else lam_of(("lambda_init", layer))
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    ldev = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    if paged:
        rng = np.random.default_rng(790 + T)
        perm = rng.permutation(B * max_pages)
        pools = {}
        for k in ("k1", "k2", "v"):
            w = inp[k].shape[-1]
            pg = inp[k].reshape(B, H, max_pages, P, w).transpose(0, 2, 1, 3, 4).reshape(B * max_pages, H, P, w)
            pool = np.empty_like(pg)
            pool[perm] = pg
            pools[k] = dev_bf16(pool)
        table = torch.from_numpy(perm.reshape(B, max_pages).astype(np.int32)).to("cuda:0")
        out = da.diffattn_decode_paged(dev["q1"], pools["k1"], dev["q2"], pools["k2"], pools["v"], table, lam, layer,
                                       lens=ldev)
    else:
        out = da.diffattn_decode_varlen(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, layer, lens=ldev)
    torch.cuda.synchronize()
    ref = varlen_reference(f, T, L, lens, lam, layer)
    check_bf16(host_bf16(out), ref, f"decode multi-token rescale T{T} paged={paged}", raw=layer == 0)


def test_decode_paged_per_head_lambda():
    torch = torch_mod()
    B, H, T, P, max_pages, lens = 2, 3, 3, 64, 12, [700, 64]
    say(f"case: decode paged per-head lambda B{B} H{H} T{T} page {P} x {max_pages}")
    cont, pools, table, L = paged_case(B, H, T, P, max_pages, lens, seed=760)
    dev = {k: dev_bf16(v) for k, v in cont.items()}
    pdev = {k: dev_bf16(v) for k, v in pools.items()}
    tdev = torch.from_numpy(table).to("cuda:0")
    ldev = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    out = da.diffattn_decode_paged(dev["q1"], pdev["k1"], dev["q2"], pdev["k2"], pdev["v"], tdev, dev_lam(LAM_HEADS),
                                   1, lens=ldev)
    torch.cuda.synchronize()
    ref = varlen_reference(widen(cont), T, L, lens, LAM_HEADS.astype(np.float64), 1)
    check_bf16(host_bf16(out), ref, "decode paged per-head")


# ---------------------------------------------------------------------------------------------------------------
# Maximum cache length (DIFFATTN_MAX_LEN = 2^23 rows): a closed-form case of the definition
# ---------------------------------------------------------------------------------------------------------------

MAX_L = 1 << 23


def needle_caches(H, T, needles, seed):
    """Caches of MAX_L rows on the GPU: K1 = K2 = 0 except row j* of head h, which is a bf16 copy of alpha * q (per
    map) with the score q.k / sqrt(d) = 40 for every query of the head (its queries are equal), and V = 0 except rows
    j* - 1, j*, j* + 1 (seeded N(0,1)).  Every other key scores 0, so both maps give row j* the weight
    1 / (1 + (L - 1) e^-40) = 1 - 3.6e-11 and the output is (1 - lambda) V[j*] to within that (then normalised for
    layer >= 1)."""
    torch = torch_mod()
    qd = di.decode_bf16(1, H, 4, 64, seed=seed)
    q1 = dev_bf16(qd["q1"]).view(1, H, 1, 64).expand(1, H, T, 64).contiguous()
    q2 = dev_bf16(qd["q2"]).view(1, H, 1, 64).expand(1, H, T, 64).contiguous()
    rows = dev_bf16(qd["v"][0, :, :3])                  # [H][3][128]: the V rows around each needle
    k1 = torch.zeros(1, H, MAX_L, 64, dtype=torch.bfloat16, device="cuda:0")
    k2 = torch.zeros_like(k1)
    v = torch.zeros(1, H, MAX_L, 128, dtype=torch.bfloat16, device="cuda:0")
    for h, j in enumerate(needles):
        for kk, qq in ((k1, q1), (k2, q2)):
            qf = qq[0, h, 0].float()
            kk[0, h, j] = (qf * (320.0 / float((qf * qf).sum()))).to(torch.bfloat16)
        v[0, h, j - 1:j + 2] = rows[h]
    torch.cuda.synchronize()
    return q1, k1, q2, k2, v


def needle_reference(v, needles, T, lam, layer):
    out = np.zeros((1, len(needles), T, 128))
    for h, j in enumerate(needles):
        o = (1.0 - lam) * host_bf16(v[0, h, j])
        if layer >= 1:
            o = o / np.sqrt((o * o).mean() + 1e-5) * (1.0 - oracle.lambda_init(layer))
        out[0, h, :] = o
    return out


@pytest.mark.parametrize("layer", [0, 1])
def test_decode_max_length_needle(layer):
    """Decode and paged decode at the largest supported cache length: one head's V is 2 GiB, the edge of the 32-bit
    buffer offsets; the paged pools (64-row pages in a shuffled order, V pool 6 GiB) need 64-bit addresses."""
    torch = torch_mod()
    H, lam = 3, 0.5
    needles = [100, (1 << 22) + 7, MAX_L - 2]   # every needle is visible to both queries when T = 2
    say(f"case: decode max length L=2^23 needles {needles} layer {layer}")
    q1, k1, q2, k2, v = needle_caches(H, 2, needles, seed=880)
    out = da.diffattn_decode(q1[:, :, 0].contiguous(), k1, q2[:, :, 0].contiguous(), k2, v, lam, layer)
    torch.cuda.synchronize()
    ref1 = needle_reference(v, needles, 1, lam, layer)
    check_bf16(host_bf16(out)[:, :, None], ref1, f"decode L=2^23 layer {layer}", raw=layer == 0)
    # The same caches in shuffled 64-row pages.
    P, max_pages = 64, MAX_L // 64
    perm = torch.randperm(max_pages, generator=torch.Generator().manual_seed(881)).to("cuda:0")

    def pool(x):
        pages = x.view(1, H, max_pages, P, x.shape[-1]).permute(0, 2, 1, 3, 4).reshape(max_pages, H, P, x.shape[-1])
        dst = torch.empty(pages.shape, dtype=pages.dtype, device=pages.device)   # contiguous
        dst[perm] = pages
        return dst

    k1p, k2p = pool(k1), pool(k2)
    del k1, k2
    vp = pool(v)
    table = perm.to(torch.int32).view(1, max_pages)
    torch.cuda.synchronize()
    for T in (1, 2):
        outp = da.diffattn_decode_paged(q1[:, :, :T].contiguous(), k1p, q2[:, :, :T].contiguous(), k2p, vp, table,
                                        lam, layer)
        torch.cuda.synchronize()
        check_bf16(host_bf16(outp), needle_reference(v, needles, T, lam, layer), f"paged decode L=2^23 T{T}",
                   raw=layer == 0)
