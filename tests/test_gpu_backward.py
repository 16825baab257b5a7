"""GPU parity of the training forward and the backward pass against the CPU oracles.

The backward oracle is the chain rule of the forward definition in double precision, pinned by finite differences
of the forward oracle (tests/test_oracle_bwd.py).  The GPU path computes in bf16 with fp32 accumulation: probabilities
and ds are rounded to bf16 before the matrix products (unit roundoff 2^-8 each), dO is rounded to bf16, and the
gradients are stored as bf16 (2^-8).  Over the key or query sums these errors partly cancel, so each gradient tensor
is checked block by block against its own scale, S = max |ref| over 64 rows of one (batch, head), floored at 1e-2
(with a single key per row the exact dq is zero and the GPU returns rounding residue): |got - ref| <= 1.5e-2 S for
every element and the block's mean |got - ref| <= 2e-3 S.  dlambda is within 1.5e-2 of the largest head's |dlambda|:
it is a sum over rows of terms of both signs, each carrying the forward's bf16-probability error (2^-8 relative) in
o2, and the cancellation enlarges the relative error of the total.  Observed over these cases: element 1.17e-2 S
(dk1 of the full-size workload), block mean 1.58e-3 S (dq1 of a head with lambda 0.9), dlambda 8.7e-3; the bounds
leave a margin of about 1.3x on each.
"""
import numpy as np
import pytest

import diffattn_inputs as di
import differential_attention_fwd_amd as da
import oracle

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("gpu")]

REL_MAX, REL_MEAN, REL_DLAMBDA = 1.5e-2, 2e-3, 1.5e-2
ROW_BLOCK = 64       # rows per scale block
SCALE_FLOOR = 1e-2   # absolute floor of a block's scale (one key per row makes dq exactly zero)


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


def host(t):
    torch = torch_mod()
    return di.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def run_case(B, H, N, causal, layer, lam, seed):
    torch = torch_mod()
    inp = di.prefill_bf16(B, H, N, 64, seed=seed)
    dy_bits = di.output_grad_bf16(B, H, N, 64, seed=seed)
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    dy = dev_bf16(dy_bits)
    lam_dev = torch.tensor(np.asarray(lam, dtype=np.float32), device="cuda:0") if np.ndim(lam) else lam
    out, saved = da.diffattn_fwd_train(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam_dev, layer, causal)
    g = da.diffattn_bwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dy, saved, lam_dev, layer, causal)
    torch.cuda.synchronize()
    f = {k: di.bf16_bits_to_f32(v) for k, v in inp.items()}
    ref = oracle.diffattn_bwd(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], di.bf16_bits_to_f32(dy_bits),
                              np.asarray(lam, dtype=np.float32).astype(np.float64), layer, causal)
    return out, g, ref, dev


def block_scale(r, rows=ROW_BLOCK):
    """Per (batch, head, block of `rows` rows) scale of a [B][H][N][w] gradient: max |ref| over the block, floored."""
    B, H, N, w = r.shape
    nb = -(-N // rows)
    pad = np.zeros((B, H, nb * rows, w))
    pad[:, :, :N] = np.abs(r)
    s = pad.reshape(B, H, nb, rows * w).max(axis=-1)
    return np.maximum(s, SCALE_FLOOR)


def check_grads(g, ref, what):
    for k in ("dq1", "dk1", "dq2", "dk2", "dv"):
        got = host(g[k])
        r = ref[k]
        B, H, N, w = r.shape
        sc = block_scale(r)                                      # [B][H][blocks]
        err = np.abs(got - r)
        rel = err / np.repeat(sc, ROW_BLOCK, axis=2)[:, :, :N, None]
        nb = sc.shape[2]
        pad = np.zeros((B, H, nb * ROW_BLOCK, w))
        pad[:, :, :N] = rel
        # mean over each block's real rows only
        cnt = np.minimum(ROW_BLOCK, N - ROW_BLOCK * np.arange(nb)) * w
        rel_mean = pad.reshape(B, H, nb, ROW_BLOCK * w).sum(axis=-1) / cnt
        say(f"{what} {k}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}; per {ROW_BLOCK}-row block relative "
            f"max {rel.max():.2e} (bound {REL_MAX:.1e}), worst block mean {rel_mean.max():.2e} (bound {REL_MEAN:.1e})")
        assert np.isfinite(got).all(), k
        assert rel.max() <= REL_MAX, f"{what} {k}: relative max {rel.max():.3e}"
        assert rel_mean.max() <= REL_MEAN, f"{what} {k}: relative block mean {rel_mean.max():.3e}"
    dl = g["dlambda"].cpu().numpy().astype(np.float64)
    rel = np.abs(dl - ref["dlambda"]).max() / max(np.abs(ref["dlambda"]).max(), 1e-30)
    say(f"{what} dlambda: got {dl} ref {ref['dlambda']} rel {rel:.2e} (bound {REL_DLAMBDA:.1e})")
    assert rel <= REL_DLAMBDA


def test_training_forward_matches_inference_forward():
    torch = torch_mod()
    inp = di.prefill_bf16(2, 2, 300, 64, seed=500)
    say("case: training forward == forward, B2 H2 N300 causal layer 2")
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    a = da.diffattn_fwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.7, 2, True)
    b, _ = da.diffattn_fwd_train(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], 0.7, 2, True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("B,H,N,causal,layer,lam", [
    (1, 2, 64, True, 0, 0.8),
    (2, 2, 200, True, 3, 0.5),
    (1, 3, 129, False, 1, [0.1, 0.6, 0.9]),
    (1, 1, 33, True, 2, 0.3),
    (1, 2, 1, True, 1, 0.8),
    (1, 1, 1000, True, 12, 0.7778701),
    (1, 2, 300, False, 0, 0.25),
    (2, 8, 600, True, 1, 0.6),      # 16 heads: the dQ and dK/dV grids take each XCD's two heads one at a time
    (4, 8, 256, False, 2, 0.4),     # 32 heads, not causal
])
def test_backward_vs_oracle(B, H, N, causal, layer, lam):
    say(f"case: backward B{B} H{H} N{N} causal={causal} layer={layer} lambda={lam}")
    _, g, ref, _ = run_case(B, H, N, causal, layer, lam, seed=510 + N)
    check_grads(g, ref, f"bwd N{N}")


def test_backward_deterministic():
    torch = torch_mod()
    say("case: backward determinism B1 H2 N257")
    _, g1, _, dev = run_case(1, 2, 257, True, 2, 0.6, seed=530)
    _, g2, _, _ = run_case(1, 2, 257, True, 2, 0.6, seed=530)
    for k in ("dq1", "dk1", "dq2", "dk2", "dv", "dlambda"):
        assert torch.equal(g1[k], g2[k]), k


def test_backward_full_size_sampled_heads():
    """The backward workload bench.py times (B4 H12 N4096, causal, layer 12, lambda = lambda_init(12), outlier query
    rows, synthetic N(0,1) output gradient) run on the GPU in full, in bench.py's launch configuration; heads 0 and
    H - 1 (every batch entry) checked against the oracle.  Heads are independent under a scalar lambda, so the oracle
    runs on those heads' slices, and dlambda of a head sums over its batch entries only."""
    torch = torch_mod()
    B, H, N, layer, seed = 4, 12, 4096, 12, 3
    lam = float(np.float32(da.diffattn_lambda_init(layer)))
    say(f"case: backward full size B{B} H{H} N{N} causal layer {layer}, heads 0 and {H - 1} vs oracle")
    inp = di.prefill_bf16(B, H, N, 64, seed=seed, outliers=True)
    dy_bits = di.output_grad_bf16(B, H, N, 64, seed=seed)
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    dy = dev_bf16(dy_bits)
    out, saved = da.diffattn_fwd_train(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, layer, True)
    g = da.diffattn_bwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dy, saved, lam, layer, True)
    torch.cuda.synchronize()
    heads = [0, H - 1]
    f = {k: di.bf16_bits_to_f32(v[:, heads]) for k, v in inp.items()}
    ref = oracle.diffattn_bwd(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], di.bf16_bits_to_f32(dy_bits[:, heads]),
                              lam, layer, True)
    sub = {k: g[k][:, heads].contiguous() for k in ("dq1", "dk1", "dq2", "dk2", "dv")}
    sub["dlambda"] = g["dlambda"][heads].contiguous()
    check_grads(sub, ref, "backward B4 H12 N4096 heads 0, 11")


@pytest.mark.parametrize("causal,per_head", [(True, False), (False, True)])
def test_strided_training_packed_projection(causal, per_head):
    """q1 | k1 | q2 | k2 | v read as column slices of one packed projection [B][N][H][6][64], dy a token-major view,
    out into a [B][N][H][128] buffer and the five gradients into the packed gradient buffer: out, saved, every
    gradient and dlambda bit-identical to the dense entry points on contiguous copies."""
    torch = torch_mod()
    B, H, N, layer = 2, 3, 333, 2
    say(f"case: strided training from a packed projection, B{B} H{H} N{N} causal={causal} per-head={per_head}")
    inp = di.prefill_bf16(B, H, N, 64, seed=800)
    dev = {k: dev_bf16(v) for k, v in inp.items()}
    dy = dev_bf16(di.output_grad_bf16(B, H, N, 64, seed=800))
    lam = torch.tensor([0.3, 0.55, 0.7], device="cuda:0") if per_head else 0.6
    proj = torch.empty((B, N, H, 6, 64), dtype=torch.bfloat16, device="cuda:0")
    for i, k in enumerate(("q1", "k1", "q2", "k2")):
        proj[:, :, :, i] = dev[k].permute(0, 2, 1, 3)
    proj[:, :, :, 4:6] = dev["v"].permute(0, 2, 1, 3).reshape(B, N, H, 2, 64)
    views = [proj[:, :, :, i].permute(0, 2, 1, 3) for i in range(4)]
    vview = proj[:, :, :, 4:6].reshape(B, N, H, 128).permute(0, 2, 1, 3)
    dy_tok = dy.permute(0, 2, 1, 3).contiguous()                       # [B][N][H][128]
    dyview = dy_tok.permute(0, 2, 1, 3)
    obuf = torch.zeros((B, N, H, 128), dtype=torch.bfloat16, device="cuda:0")
    out, saved = da.diffattn_fwd_train_strided(views[0], views[1], views[2], views[3], vview, lam, layer, causal,
                                               out=obuf.permute(0, 2, 1, 3))
    gbuf = torch.zeros((B, N, H, 6, 64), dtype=torch.bfloat16, device="cuda:0")
    grads = {k: gbuf[:, :, :, i].permute(0, 2, 1, 3) for i, k in enumerate(("dq1", "dk1", "dq2", "dk2"))}
    grads["dv"] = gbuf[:, :, :, 4:6].reshape(B, N, H, 128).permute(0, 2, 1, 3)
    grads["dlambda"] = torch.empty(H, dtype=torch.float32, device="cuda:0")
    da.diffattn_bwd_strided(views[0], views[1], views[2], views[3], vview, dyview, saved, lam, layer, causal, grads)
    ref_out, ref_saved = da.diffattn_fwd_train(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], lam, layer,
                                               causal)
    ref = da.diffattn_bwd(dev["q1"], dev["k1"], dev["q2"], dev["k2"], dev["v"], dy, ref_saved, lam, layer, causal)
    torch.cuda.synchronize()
    assert torch.equal(out.contiguous().view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(saved, ref_saved)
    for k in ("dq1", "dk1", "dq2", "dk2", "dv"):
        assert torch.equal(grads[k].contiguous().view(torch.int16), ref[k].view(torch.int16)), k
    assert torch.equal(grads["dlambda"], ref["dlambda"])
