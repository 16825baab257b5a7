"""HIP graph capture: the prefill (one pass and key splits), the training forward and backward, the decode with its
two-level merge, the ragged multi-token decode on its balanced plan and the allocation-free decode recorded into one graph through torch's capture (their kernels on the capturing stream, no
allocation and no memset inside), replayed several times with other GPU work in between; every replay must
reproduce the eager results bit for bit."""
import numpy as np
import pytest

import diffattn_inputs as di
import differential_attention_fwd_amd as da

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("gpu")]


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def dev_bf16(bits):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def test_graph_replays_match_eager():
    torch = torch_mod()
    print("case: graph capture of prefill B2 H4 N700, split prefill B1 H2 N1000, decode B1 H2 L20000 (256 splits, "
          "two-level merge), ragged decode B8 H16 T3 L900 (balanced plan), no-allocation decode B4 H8 L1000, training "
          "forward and backward B1 H2 N300", flush=True)
    p = {k: dev_bf16(v) for k, v in di.prefill_bf16(2, 4, 700, 64, seed=1400).items()}
    s = {k: dev_bf16(v) for k, v in di.prefill_bf16(1, 2, 1000, 64, seed=1401).items()}
    d = {k: dev_bf16(v) for k, v in di.decode_bf16(1, 2, 20000, 64, seed=1402).items()}
    n = {k: dev_bf16(v) for k, v in di.decode_bf16(4, 8, 1000, 64, seed=1403).items()}
    out_p = torch.empty(2, 4, 700, 128, dtype=torch.bfloat16, device="cuda:0")
    out_s = torch.empty(1, 2, 1000, 128, dtype=torch.bfloat16, device="cuda:0")
    out_d = torch.empty(1, 2, 128, dtype=torch.bfloat16, device="cuda:0")
    out_n = torch.empty(4, 8, 128, dtype=torch.bfloat16, device="cuda:0")
    ws_s = torch.empty(max(da.diffattn_fwd_split_workspace_bytes(1, 2, 1000, 64), 16), dtype=torch.uint8,
                       device="cuda:0")
    ws_d = torch.empty(max(da.diffattn_decode_workspace_bytes(1, 2, 20000, 64), 16), dtype=torch.uint8,
                       device="cuda:0")
    assert da.diffattn_fwd_split_workspace_bytes(1, 2, 1000, 64) > 0
    rg = {k: dev_bf16(v) for k, v in di.decode_bf16(8, 16, 900, 64, seed=1406).items()}
    rq = {k: dev_bf16(v) for k, v in di.prefill_bf16(8, 16, 3, 64, seed=1407).items()}
    lens = torch.tensor([900, 3, 450, 899, 17, 600, 900, 5], dtype=torch.int32, device="cuda:0")
    out_r = torch.empty(8, 16, 3, 128, dtype=torch.bfloat16, device="cuda:0")
    ws_r = torch.empty(da.diffattn_decode_varlen_workspace_bytes(8, 16, 3, 900, 64), dtype=torch.uint8,
                       device="cuda:0")
    t = {k: dev_bf16(v) for k, v in di.prefill_bf16(1, 2, 300, 64, seed=1404).items()}
    dy = dev_bf16(di.prefill_bf16(1, 2, 300, 128, seed=1405)["q1"])
    out_t = torch.empty(1, 2, 300, 128, dtype=torch.bfloat16, device="cuda:0")
    saved = torch.empty(max(da.diffattn_train_saved_bytes(1, 2, 300, 64), 16), dtype=torch.uint8, device="cuda:0")
    grads = {k: torch.empty_like(x) for k, x in (("dq1", t["q1"]), ("dk1", t["k1"]), ("dq2", t["q2"]),
                                                 ("dk2", t["k2"]), ("dv", t["v"]))}
    grads["dlambda"] = torch.empty(2, dtype=torch.float32, device="cuda:0")
    ws_b = torch.empty(max(da.diffattn_bwd_workspace_bytes(1, 2, 300, 64), 16), dtype=torch.uint8, device="cuda:0")

    def work():
        da.diffattn_fwd(p["q1"], p["k1"], p["q2"], p["k2"], p["v"], 0.6, 2, True, out=out_p)
        da.diffattn_fwd_split(s["q1"], s["k1"], s["q2"], s["k2"], s["v"], 0.7, 1, True, out=out_s, workspace=ws_s)
        da.diffattn_decode(d["q1"], d["k1"], d["q2"], d["k2"], d["v"], 0.8, 1, True, out=out_d, workspace=ws_d)
        da.diffattn_decode_varlen(rq["q1"], rg["k1"], rq["q2"], rg["k2"], rg["v"], 0.8, 2, lens=lens, out=out_r,
                                  workspace=ws_r)
        da.diffattn_decode_noalloc(n["q1"], n["k1"], n["q2"], n["k2"], n["v"], 0.5, 3, True, out=out_n)
        x = (t["q1"], t["k1"], t["q2"], t["k2"], t["v"])
        da.diffattn_fwd_train(*x, 0.4, 2, True, out=out_t, saved=saved)
        da.diffattn_bwd(*x, dy, saved, 0.4, 2, True, grads=grads, workspace=ws_b)

    outs = (out_p, out_s, out_d, out_r, out_n, out_t, *grads.values())
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the capture (first no-allocation call looks up its scratch array)
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            same = torch.equal(o.view(torch.int16), r.view(torch.int16)) if o.dtype == torch.bfloat16 else \
                torch.equal(o, r)
            assert same, f"replay {rep}"
        # other work on the same buffers between replays (eager; overwritten by the next replay)
        work()
        torch.cuda.synchronize()
