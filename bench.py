"""Benchmark: differential attention causal prefill (B4 H12 N4096) and decode (B64 H16 L8192) on one MI355X.

One step = one pass of the whole hot path on resident synthetic inputs: the fused prefill kernel at
B=4, H=12, N=4096, d=64, 2d=128 (causal, layer 12, lambda = lambda_init(12), outlier query rows) followed by the
split-K decode (split + merge kernels) at B=64, H=16, L=8192 (lambda 0.8, layer 1).  Each kernel is timed with HIP
events recorded on the stream it is launched on.  Prints ONE JSON line.

  value     prefill TFLOP/s, counting 12*d FLOP per unmasked (query, key) pair (two Q.K^T products of width d and
            two P.V products of width 2d), i.e. B*H*N*(N+1)/2 pairs
  roofline  the prefill kernel against the bf16 dense MFMA peak; decode carries its own against HBM bandwidth
  cpu_baseline  the double-precision CPU oracle on the same prefill workload (all rows by default; on one thread,
            every 16th row), and on the whole decode workload (all threads and one)
  decode_multi  (not part of the step) multi-token decode, 4 new tokens per sequence against ragged caches of
            4096..8192 rows at B64 H16: GB/s of the valid cache rows read
  decode_paged  (not part of the step) the decode workload read from 64-row pages of a shuffled page pool through
            a block table: GB/s of the same bytes as decode
  backward  (not part of the step) the training forward and the backward pass on the prefill workload with a
            synthetic output gradient, timed separately.  Its roofline counts 1280 FLOP per unmasked pair: the two
            score maps and dP once (768) and dV, dQ1, dQ2, dK1, dK2 (512), the least an exact streaming backward
            does; tflops_exec counts the 1792 the kernels execute (the dQ kernel recomputes both score maps and dP and
            forms dQ1, dQ2: 768; the dK/dV kernel recomputes them and forms dV, dK1, dK2: 1024)
  prefill_n1024  (not part of the step) the small causal prefill B1 H8 N1024 (layer 1), reported, not gated (64 row
            tiles for 256 CUs), through diffattn_fwd and (split) through diffattn_fwd_split, and the oracle's time on
            the whole problem, all host threads and one
  prefill_n65536  (not part of the step) the causal prefill at B1 H16 N65536 (layer 24): TFLOP/s with its roofline, and
            the oracle's time on 256 sampled rows with the full-problem time extrapolated from them (labelled so)
  clock     the GPU clock and socket power the box reports (amdsmi GPU metrics) while the prefill runs back to back
            for about two seconds, and the prefill rate over that window
  context   the same box's bf16 GEMM rate (torch.matmul 8192^3, random data), torch's streaming read (a sum over a
            4 GiB tensor), and the best streaming read of a plain probe kernel (16-byte nontemporal loads, as the decode
            kernel reads its V rows; libstreamprobe.so): what this machine reaches, next to the nominal peaks
Each timed kernel reports the median over its repetitions (the headline value uses the median), with the mean and
the minimum beside it.
Every roofline's "traffic" is the HBM bytes per call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
(profiles/hbm_traffic.txt), used only while the kernel source still matches the hash recorded there, else null.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "diff-attn causal fwd TFLOP/s @N=4096 (% MFMA peak); decode GB/s (% HBM)"
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12   # 2516.6: 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0

PREFILL = dict(B=4, H=12, N=4096, d=64, layer=12, seed=3)
DECODE = dict(B=64, H=16, L=8192, d=64, layer=1, lam=0.8, seed=5)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def prefill_pairs(B, H, N):
    return B * H * N * (N + 1) // 2


def decode_bytes(B, H, L, d):
    """Algorithmic HBM bytes of one decode: K1, K2, V read once, Q1, Q2 read, out written (bf16)."""
    return 2 * (2 * B * H * L * d + B * H * L * 2 * d + 2 * B * H * d + B * H * 2 * d)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def read_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches the current kernel source."""
    import hashlib
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    rec = {}
    for line in open(PROFILE_TRAFFIC):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    src = rec.get(f"{kernel}.source")
    if not src:
        return None
    path = os.path.join(ROOT, src)
    if not os.path.exists(path):
        return None
    digest = hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]
    if digest != rec.get(f"{kernel}.source_sha256_16"):
        return None  # kernel changed since the counters were taken
    try:
        return float(rec[f"{kernel}.hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp_bits, lam, layer, N, target_rows, threads=None):
    """Time the oracle on every k-th query row of the prefill workload (uniform over the causal row costs)."""
    import numpy as np

    import diffattn_inputs as di
    import oracle

    f = {k: di.bf16_bits_to_f32(v) for k, v in inp_bits.items()}
    B, H = f["q1"].shape[:2]
    total = B * H * N
    stride = max(1, total // target_rows)
    rows = np.arange(0, total, stride, dtype=np.int64)
    pairs = int(((rows % N) + 1).sum())
    threads = threads or oracle.max_threads()
    oracle.diffattn(f["q1"][:1, :1, :8], f["k1"][:1, :1, :8], f["q2"][:1, :1, :8], f["k2"][:1, :1, :8],
                    f["v"][:1, :1, :8], lam, layer, True)  # load the library outside the timed region
    t0 = time.perf_counter()
    oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, layer, True, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(pairs * 12 * 64 / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"all {total} query rows" if stride == 1 else
                       f"{rows.size} of {total} query rows (every {stride}th row)") +
                      f" ({pairs} unmasked pairs) of the B4 H12 N4096 causal prefill, double precision, {dt:.2f} s on "
                      f"{threads} threads of '{cpu_model()}'",
            "seconds": round(dt, 3)}


def bench_decode_multi(da, stream, k1, k2, v, Dc, steps, T=4):
    """Multi-token decode against the decode workload's caches with seeded ragged lengths in [L/2, L]."""
    import numpy as np
    import torch
    dev = k1.device
    B, H, L, d = Dc["B"], Dc["H"], Dc["L"], Dc["d"]
    rng = np.random.default_rng(Dc["seed"])
    lens_np = rng.integers(L // 2, L + 1, size=B).astype(np.int32)
    lens = torch.from_numpy(lens_np).to(dev)
    g = torch.Generator(device=dev).manual_seed(Dc["seed"])
    q1 = torch.randn(B, H, T, d, device=dev, generator=g).to(torch.bfloat16)
    q2 = torch.randn(B, H, T, d, device=dev, generator=g).to(torch.bfloat16)
    out = torch.empty(B, H, T, 2 * d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(da.diffattn_decode_varlen_workspace_bytes(B, H, T, L, d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()   # inputs are made on torch's current stream; the kernels run on `stream`

    def run():
        da.diffattn_decode_varlen(q1, k1, q2, k2, v, Dc["lam"], Dc["layer"], lens=lens, out=out, workspace=ws,
                                  stream=stream)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    st = med_stats(time_on_stream(run, stream, steps))
    ms = st["ms"]
    nbytes = int(lens_np.sum()) * H * (2 * d * 2 + 2 * d * 2) + 2 * (2 * B * H * T * d + B * H * T * 2 * d)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"decode B{B} H{H} T{T} new tokens, cache lengths {int(lens_np.min())}..{int(lens_np.max())} "
                        f"(seeded uniform in [{L // 2}, {L}]), d64 dv128", "steps": steps, **st,
            "bytes": nbytes, "value": round(gbs, 1), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": read_traffic("decode_multi")}}


def bench_decode_paged(da, stream, q1, k1, q2, k2, v, Dc, steps, ref_out, nbytes, P=64):
    """Single-token decode on the decode workload with its caches split into P-row pages, stored in a seeded
    shuffled order in page pools and found through a block table."""
    import torch
    dev = k1.device
    B, H, L, d = Dc["B"], Dc["H"], Dc["L"], Dc["d"]
    max_pages = L // P
    g = torch.Generator(device="cpu").manual_seed(Dc["seed"] + 1)
    perm = torch.randperm(B * max_pages, generator=g).to(dev)

    def pool(x):
        w = x.shape[-1]
        pages = x.view(B, H, max_pages, P, w).permute(0, 2, 1, 3, 4).reshape(B * max_pages, H, P, w)
        out = torch.empty(pages.shape, dtype=pages.dtype, device=pages.device)   # contiguous
        out[perm] = pages
        return out

    k1p, k2p, vp = pool(k1), pool(k2), pool(v)
    table = perm.to(torch.int32).view(B, max_pages).contiguous()
    out = torch.empty(B, H, 1, 2 * d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(da.diffattn_decode_paged_workspace_bytes(B, H, 1, max_pages, P, d), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()   # the pools are built on torch's current stream; the kernels run on `stream`

    def run():
        da.diffattn_decode_paged(q1[:, :, None], k1p, q2[:, :, None], k2p, vp, table, Dc["lam"], Dc["layer"],
                                 out=out, workspace=ws, stream=stream)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    if not torch.equal(out[:, :, 0].view(torch.int16), ref_out.view(torch.int16)):
        raise RuntimeError("paged decode differs from the contiguous decode on the same rows")
    st = med_stats(time_on_stream(run, stream, steps))
    ms = st["ms"]
    gbs = nbytes / (ms * 1e-3) / 1e9
    del k1p, k2p, vp
    return {"workload": f"decode B{B} H{H} L{L} d64 dv128 in {P}-row pages (shuffled pool, block table)",
            "steps": steps, **st, "bytes": nbytes, "value": round(gbs, 1), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": read_traffic("decode_paged")}}


def bench_backward(da, di, stream, p_bits, q1, k1, q2, k2, v, lam, steps):
    """Training forward + backward on the prefill workload; HIP events on the launch stream."""
    import numpy as np
    import torch
    P = PREFILL
    dev = q1.device
    dy = torch.from_numpy(di.output_grad_bf16(P["B"], P["H"], P["N"], P["d"], P["seed"]).view(np.int16)).view(
        torch.bfloat16).to(dev)
    out = torch.empty_like(v)
    saved = torch.empty(da.diffattn_train_saved_bytes(P["B"], P["H"], P["N"], P["d"]), dtype=torch.uint8, device=dev)
    grads = {k: torch.empty_like(t) for k, t in (("dq1", q1), ("dk1", k1), ("dq2", q2), ("dk2", k2), ("dv", v))}
    grads["dlambda"] = torch.empty(P["H"], dtype=torch.float32, device=dev)
    ws = torch.empty(da.diffattn_bwd_workspace_bytes(P["B"], P["H"], P["N"], P["d"]), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()   # inputs are made on torch's current stream; the kernels run on `stream`

    def fwd():
        da.diffattn_fwd_train(q1, k1, q2, k2, v, lam, P["layer"], True, out=out, saved=saved, stream=stream)

    def bwd():
        da.diffattn_bwd(q1, k1, q2, k2, v, dy, saved, lam, P["layer"], True, grads=grads, workspace=ws, stream=stream)

    for _ in range(2):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(stream)
        fwd()
        ev[k][1].record(stream)
        bwd()
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    fst = med_stats([e[0].elapsed_time(e[1]) for e in ev])
    bst = med_stats([e[1].elapsed_time(e[2]) for e in ev])
    b_ms = bst["ms"]
    pairs = prefill_pairs(P["B"], P["H"], P["N"])
    flops = pairs * 1792
    flops_min = pairs * 1280
    tf = flops / (b_ms * 1e-3) / 1e12
    tf_min = flops_min / (b_ms * 1e-3) / 1e12
    return {"workload": "causal B4 H12 N4096 d64 dv128, layer 12, synthetic N(0,1) output gradient",
            "steps": steps, "fwd_train_ms": fst["ms"], "fwd_train_ms_min": fst["ms_min"], **bst,
            "flops_exec": flops, "tflops_exec": round(tf, 2),
            "flops_one_recompute": flops_min, "tflops_one_recompute": round(tf_min, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf_min, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                         "unit": "TFLOP/s", "frac": round(tf_min / PEAK_BF16_TFLOPS, 4),
                         "flop_count": "1280 per unmasked pair (scores, dP and the five gradient products once)",
                         "traffic": read_traffic("backward")}}

def med_stats(ms):
    """Median (the reported time), mean and minimum of a list of per-repetition times in ms."""
    import statistics
    return {"ms": round(statistics.median(ms), 4), "ms_mean": round(sum(ms) / len(ms), 4), "ms_min": round(min(ms), 4)}


def time_on_stream(fn, stream, reps):
    """Per-repetition times (ms) of fn() from HIP events recorded on `stream`."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def sample_clock(fn, stream, seconds=2.0, period=0.02):
    """Run fn() back to back for about `seconds` while a thread samples the GPU metrics (current graphics clock,
    socket power); the firmware refreshes them a few times per second, so only the samples of the second half of
    the window are summarised.  Returns None when the metrics cannot be read."""
    import statistics
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[torch.cuda.current_device()]
        amdsmi.amdsmi_get_gpu_metrics_info(h)
    except Exception as e:   # no metrics on this machine: say so rather than guess
        return {"error": f"{type(e).__name__}: {e}"}
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                samples.append((time.perf_counter(), m.get("current_gfxclk"), m.get("current_socket_power")))
            except Exception:
                pass
            time.sleep(period)

    # one launch's duration, to size the window
    one = statistics.median(time_on_stream(fn, stream, 5))
    reps = max(10, int(seconds * 1e3 / max(one, 1e-3)))
    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    ms = time_on_stream(fn, stream, reps)
    t1 = time.perf_counter()
    stop.set()
    th.join()
    late = [(c, p) for (t, c, p) in samples if t >= t0 + 0.5 * (t1 - t0) and isinstance(c, (int, float))]
    out = {"reps": reps, "window_s": round(t1 - t0, 3), "ms_median_in_window": round(statistics.median(ms), 4),
           "source": "amdsmi GPU metrics (current_gfxclk, current_socket_power), second half of the window"}
    if late:
        out["gfxclk_mhz_median"] = statistics.median(c for c, _ in late)
        out["gfxclk_mhz_min"] = min(c for c, _ in late)
        pw = [p for _, p in late if isinstance(p, (int, float))]
        if pw:
            out["socket_power_w_median"] = statistics.median(pw)
        out["samples"] = len(late)
    return out


def context_rates(dev, stream):
    """Library kernels on the same box: bf16 GEMM (torch.matmul, 8192^3, N(0,1) data) and a streaming read (sum of a
    4 GiB bf16 tensor)."""
    import torch
    g = torch.Generator(device=dev).manual_seed(11)
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16, generator=g)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(3):
            a @ b
        ms_g = time_on_stream(lambda: a @ b, stream, 20)
    del a, b
    x = torch.ones(1 << 31, device=dev, dtype=torch.bfloat16)   # 4 GiB
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(2):
            x.sum(dtype=torch.float32)
        ms_r = time_on_stream(lambda: x.sum(dtype=torch.float32), stream, 10)
    import statistics
    tg, tr = statistics.median(ms_g), statistics.median(ms_r)
    probe = stream_probe(x, stream)
    del x
    return {"gemm_bf16_8192_tflops": round(2 * 8192 ** 3 / (tg * 1e-3) / 1e12, 1),
            "gemm_bf16_8192_frac_of_peak": round(2 * 8192 ** 3 / (tg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "torch_sum_read_gbs": round((1 << 32) / (tr * 1e-3) / 1e9, 1),
            **probe}


def stream_probe(x, stream):
    """Best streaming-read rate of this machine over a few launch shapes: one read of the 4 GiB tensor x with 16-byte
    nontemporal loads (the decode kernels' access pattern), median of 5 reads per shape (libstreamprobe.so)."""
    import ctypes
    import statistics
    import torch
    from differential_attention_fwd_amd import build as dbuild
    if not os.path.exists(dbuild.PROBE_LIB):
        return {"stream_read_error": f"{dbuild.PROBE_LIB} is not built"}
    L = ctypes.CDLL(dbuild.PROBE_LIB)
    L.stream_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    L.stream_read_probe.restype = ctypes.c_int
    nbytes = x.numel() * x.element_size()
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        out = torch.empty(blocks * 256, dtype=torch.int32, device=x.device)
        for unroll in (2, 4, 8):
            def run():
                rc = L.stream_read_probe(x.data_ptr(), nbytes, out.data_ptr(), blocks, unroll, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"stream_read_probe failed: {rc}")
            run()
            ms = statistics.median(time_on_stream(run, stream, 5))
            gbs = nbytes / (ms * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, blocks, unroll)
    return {"stream_read_gbs": round(best[0], 1), "stream_read_frac_of_peak": round(best[0] / PEAK_HBM_GBS, 4),
            "stream_read_shape": f"{best[1]} workgroups of 256 threads, {best[2]} 16-byte nontemporal loads in flight "
                                 f"per thread, best of 12 shapes"}


def bench_prefill_n1024(da, di, stream, dev, steps):
    """The small causal prefill B1 H8 N1024 (layer 1): 64 row tiles for 256 CUs, so launch- and latency-bound (reported,
    not gated), timed on the launch stream; and the oracle on the whole problem on all host threads and on one."""
    import numpy as np
    import torch
    import oracle
    c = di.CONFIGS["prefill_n1024"]
    B, H, N, d, layer = c["B"], c["H"], c["N"], c["d"], c["layer"]
    bits = di.prefill_bf16(B, H, N, d, c["seed"])
    lam = float(np.float32(da.diffattn_lambda_init(layer)))
    t = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev) for k, v in bits.items()}
    out = torch.empty_like(t["v"])
    torch.cuda.synchronize()

    def run():
        da.diffattn_fwd(t["q1"], t["k1"], t["q2"], t["k2"], t["v"], lam, layer, True, out=out, stream=stream)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    st = med_stats(time_on_stream(run, stream, steps))
    pairs = prefill_pairs(B, H, N)
    flops = pairs * 12 * d
    tf = flops / (st["ms"] * 1e-3) / 1e12
    # The split-key entry point for launches this small (query tiles' keys split across workgroups, then merged).
    ws = torch.empty(max(da.diffattn_fwd_split_workspace_bytes(B, H, N, d), 16), dtype=torch.uint8, device=dev)
    out_s = torch.empty_like(out)
    torch.cuda.synchronize()

    def run_split():
        da.diffattn_fwd_split(t["q1"], t["k1"], t["q2"], t["k2"], t["v"], lam, layer, True, out=out_s, workspace=ws,
                              stream=stream)

    for _ in range(3):
        run_split()
    torch.cuda.synchronize()
    sst = med_stats(time_on_stream(run_split, stream, steps))
    tfs = flops / (sst["ms"] * 1e-3) / 1e12
    f = {k: di.bf16_bits_to_f32(v) for k, v in bits.items()}
    timings = {}
    for threads in (oracle.max_threads(), 1):
        t0 = time.perf_counter()
        oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, layer, True, threads=threads)
        timings[threads] = time.perf_counter() - t0
    return {"workload": f"causal prefill B{B} H{H} N{N} d64 dv128, layer {layer}", "steps": steps, **st,
            "flops_exec": flops, "tflops_exec": round(tf, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                         "note": "64 workgroups of 128 rows for 256 CUs: not a roofline case"},
            "split": {**sst, "tflops_exec": round(tfs, 2), "frac": round(tfs / PEAK_BF16_TFLOPS, 4),
                      "entry": "diffattn_fwd_split (key splits merged by log-sum-exp; the time includes the merge)"},
            "cpu_oracle": {"rows": B * H * N, "seconds_all_threads": round(timings[oracle.max_threads()], 4),
                           "threads": oracle.max_threads(), "seconds_one_thread": round(timings[1], 4)}}


def decode_oracle_time(di, d_bits, chunk=8):
    """The oracle on the whole decode workload (64 sequences x 16 heads, 8192 cache rows each), on all host threads
    and on one; the bf16 inputs are widened and evaluated 8 sequences at a time to bound host memory (the widening
    is outside the timed calls)."""
    import oracle
    Dc = DECODE
    n = oracle.max_threads()
    tot = {n: 0.0, 1: 0.0}
    for b0 in range(0, Dc["B"], chunk):
        f = {k: di.bf16_bits_to_f32(v[b0:b0 + chunk]) for k, v in d_bits.items()}
        for threads in (n, 1):
            t0 = time.perf_counter()
            oracle.decode(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], Dc["lam"], Dc["layer"], threads=threads)
            tot[threads] += time.perf_counter() - t0
        del f
    return {"sample": f"the whole decode workload (B{Dc['B']} H{Dc['H']} L{Dc['L']}), double precision, on "
                      f"'{cpu_model()}'",
            "seconds_all_threads": round(tot[n], 3), "threads": n, "seconds_one_thread": round(tot[1], 3),
            "gbs_all_threads": round(decode_bytes(Dc["B"], Dc["H"], Dc["L"], Dc["d"]) / tot[n] / 1e9, 2)}


def bench_prefill_n65536(da, di, stream, dev, steps, oracle_rows=256):
    """The causal prefill at B1 H16 N65536 (layer 24), timed on the launch stream, and the oracle on 256 sampled
    rows (rows 0, 1, 63, 64, 127, 128, 4095, 4096, N - 1 of the first and last head, the rest seeded uniform), with
    the full-problem time extrapolated from those rows' unmasked pairs."""
    import numpy as np
    import torch
    import oracle
    c = di.CONFIGS["prefill_n65536"]
    B, H, N, d, layer = c["B"], c["H"], c["N"], c["d"], c["layer"]
    bits = di.prefill_bf16(B, H, N, d, c["seed"])
    lam = float(np.float32(da.diffattn_lambda_init(layer)))
    t = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev) for k, v in bits.items()}
    out = torch.empty_like(t["v"])
    torch.cuda.synchronize()

    def run():
        da.diffattn_fwd(t["q1"], t["k1"], t["q2"], t["k2"], t["v"], lam, layer, True, out=out, stream=stream)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    ms = time_on_stream(run, stream, steps)
    st = med_stats(ms)
    pairs = prefill_pairs(B, H, N)
    flops = pairs * 12 * d
    tf = flops / (st["ms"] * 1e-3) / 1e12
    del t, out
    fixed = [(h, i) for h in (0, H - 1) for i in (0, 1, 63, 64, 127, 128, 4095, 4096, N - 1)]
    rng = np.random.default_rng(4)
    sel = fixed + [(int(rng.integers(H)), int(rng.integers(N))) for _ in range(oracle_rows - len(fixed))]
    rows = np.array([h * N + i for h, i in sel], dtype=np.int64)
    sampled_pairs = int(((rows % N) + 1).sum())
    f = {k: di.bf16_bits_to_f32(v) for k, v in bits.items()}
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.diffattn(f["q1"], f["k1"], f["q2"], f["k2"], f["v"], lam, layer, True, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    return {"workload": f"causal prefill B{B} H{H} N{N} d64 dv128, layer {layer}", "steps": steps, **st,
            "flops_exec": flops, "tflops_exec": round(tf, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": read_traffic("prefill_n65536")},
            "cpu_oracle": {"rows": int(rows.size), "unmasked_pairs": sampled_pairs, "seconds": round(dt, 3),
                           "threads": threads,
                           "extrapolated_full_seconds": round(dt * pairs / sampled_pairs, 1),
                           "note": "full-problem time extrapolated from the sampled rows' unmasked pairs"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--cpu-rows", type=int, default=4 * 12 * 4096,
                    help="oracle row sample size for cpu_baseline (default: every row of the prefill workload)")
    ap.add_argument("--bwd-steps", type=int, default=10, help="timed backward repetitions (0 skips the backward leg)")
    ap.add_argument("--multi-steps", type=int, default=10,
                    help="timed multi-token decode repetitions (0 skips that leg)")
    ap.add_argument("--paged-steps", type=int, default=10,
                    help="timed paged decode repetitions (0 skips that leg)")
    ap.add_argument("--n65536-steps", type=int, default=10,
                    help="timed repetitions of the B1 H16 N65536 prefill leg (0 skips it)")
    ap.add_argument("--n1024-steps", type=int, default=20,
                    help="timed repetitions of the B1 H8 N1024 prefill leg (0 skips it)")
    ap.add_argument("--clock-seconds", type=float, default=2.0,
                    help="length of the back-to-back prefill window sampled for clock and power (0 skips it)")
    ap.add_argument("--no-context", action="store_true", help="skip the library GEMM / streaming-read context leg")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (HBM counter calibration under rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only; there is no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import diffattn_inputs as di
    import differential_attention_fwd_amd as da

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    da.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    P = PREFILL
    p_bits = di.prefill_bf16(P["B"], P["H"], P["N"], P["d"], P["seed"], outliers=True)
    p_lam = float(np.float32(da.diffattn_lambda_init(P["layer"])))
    pq1, pk1, pq2, pk2, pv = (to_dev(p_bits[k]) for k in ("q1", "k1", "q2", "k2", "v"))
    pout = torch.empty_like(pv)

    Dc = DECODE
    d_bits = di.decode_bf16(Dc["B"], Dc["H"], Dc["L"], Dc["d"], Dc["seed"])
    dq1, dk1, dq2, dk2, dv = (to_dev(d_bits[k]) for k in ("q1", "k1", "q2", "k2", "v"))
    if args.no_cpu_baseline:
        del d_bits   # kept otherwise for the oracle's decode timing
    dout = torch.empty((Dc["B"], Dc["H"], 2 * Dc["d"]), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(da.diffattn_decode_workspace_bytes(Dc["B"], Dc["H"], Dc["L"], Dc["d"]), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    def prefill():
        da.diffattn_fwd(pq1, pk1, pq2, pk2, pv, p_lam, P["layer"], True, out=pout, stream=stream)

    def decode():
        da.diffattn_decode(dq1, dk1, dq2, dk2, dv, Dc["lam"], Dc["layer"], True, out=dout, workspace=ws,
                           stream=stream)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        prefill()
        ev[k][1].record(stream)
        decode()
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(K)]
    dec_ms = [ev[k][1].elapsed_time(ev[k][2]) for k in range(K)]
    step_ms = [ev[k][0].elapsed_time(ev[k][2]) for k in range(K)]

    pairs = prefill_pairs(P["B"], P["H"], P["N"])
    f_exec = pairs * 12 * P["d"]
    f_formula = pairs * 8 * P["d"]
    pst = med_stats(pre_ms)
    pre_tflops = f_exec / (pst["ms"] * 1e-3) / 1e12
    dbytes = decode_bytes(Dc["B"], Dc["H"], Dc["L"], Dc["d"])
    dst = med_stats(dec_ms)
    dec_gbs = dbytes / (dst["ms"] * 1e-3) / 1e9

    pre_traffic = read_traffic("prefill")
    dec_traffic = read_traffic("decode")
    result = {
        "metric": METRIC,
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(sum(step_ms) / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill B4 H12 N4096 d64 dv128 (layer 12, outlier rows) + decode B64 H16 L8192 "
                        "d64 dv128 (lambda 0.8, layer 1)",
            "prefill": {"B": P["B"], "H": P["H"], "N": P["N"], "d": P["d"], "dv": 2 * P["d"], "causal": True,
                        "layer": P["layer"], "lambda": p_lam},
            "decode": {"B": Dc["B"], "H": Dc["H"], "L": Dc["L"], "d": Dc["d"], "dv": 2 * Dc["d"],
                       "layer": Dc["layer"], "lambda": Dc["lam"]},
            "parallelism": "single GPU",
        },
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": pre_traffic},
        "prefill": {**pst, "flops_exec": f_exec, "flops_formula": f_formula,
                    "tflops_formula": round(f_formula / (pst["ms"] * 1e-3) / 1e12, 2)},
        "decode": {"value": round(dec_gbs, 1), "unit": "GB/s", **dst, "bytes": dbytes,
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(dec_gbs / PEAK_HBM_GBS, 4), "traffic": dec_traffic}},
        "wall_s": round(wall, 3),
    }
    if args.clock_seconds > 0:
        result["clock"] = sample_clock(prefill, stream, args.clock_seconds)
    if not args.no_context:
        result["context"] = context_rates(dev, stream)
    if args.multi_steps > 0:
        result["decode_multi"] = bench_decode_multi(da, stream, dk1, dk2, dv, Dc, args.multi_steps)
    if args.paged_steps > 0:
        result["decode_paged"] = bench_decode_paged(da, stream, dq1, dk1, dq2, dk2, dv, Dc, args.paged_steps, dout,
                                                    dbytes)
    if args.bwd_steps > 0:
        result["backward"] = bench_backward(da, di, stream, p_bits, pq1, pk1, pq2, pk2, pv, p_lam, args.bwd_steps)
    if args.n1024_steps > 0:
        result["prefill_n1024"] = bench_prefill_n1024(da, di, stream, dev, args.n1024_steps)
    if args.n65536_steps > 0:
        del dq1, dk1, dq2, dk2, dv, ws
        torch.cuda.empty_cache()
        result["prefill_n65536"] = bench_prefill_n65536(da, di, stream, dev, args.n65536_steps)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(p_bits, p_lam, P["layer"], P["N"], args.cpu_rows)
        one = cpu_baseline(p_bits, p_lam, P["layer"], P["N"], max(1, args.cpu_rows // 16), threads=1)
        cb["single_core"] = {k: one[k] for k in ("value", "unit", "cores", "sample", "seconds")}
        cb["decode"] = decode_oracle_time(di, d_bits)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
