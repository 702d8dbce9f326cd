"""The entry points under stream capture: a captured HIP graph replays to the eager results.

The library enqueues only kernels on the caller's stream (no allocation, memset or synchronisation
inside a call), so a forward, a backward and a decode can be captured into one graph, which suits
launch-bound shapes such as the [4,16,1024,64] causal prefill. Each replay is compared bit for bit
with the eager calls (the kernels are deterministic), with eager work, output clearing and
synchronisation between the replays.
"""
import pytest
import torch

from roofline_attention_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(lib):
    wf = I.WORKLOADS["prefill_causal_1k"]  # [4,16,1024,64] causal bf16
    tf = {k: x.cuda() for k, x in I.make_prefill(wf, with_dout=False).items()}
    wb = I.Workload("graph_bwd", "fwdbwd", 1, 4, 2, 1024, 128, "bf16", True, seed=21)
    tb = {k: x.cuda() for k, x in I.make_prefill(wb, with_dout=True).items()}
    wd = I.WORKLOADS["decode_gqa"]
    td = {k: x.cuda() for k, x in I.make_decode(wd).items()}

    f32 = dict(dtype=torch.float32, device="cuda")
    bufs = {
        "o": torch.empty_like(tf["q"]), "lse": torch.empty((wf.B, wf.H, wf.N), **f32),
        "ob": torch.empty_like(tb["q"]), "lseb": torch.empty((wb.B, wb.H, wb.N), **f32),
        "dq": torch.empty(tb["q"].shape, **f32), "dk": torch.empty(tb["k"].shape, **f32),
        "dv": torch.empty(tb["v"].shape, **f32),
        "od": torch.empty_like(td["q"]), "lsed": torch.empty((wd.B, wd.H), **f32),
    }
    wsb = torch.empty(lib.bwd_workspace_size(wb.B, wb.H, wb.N, wb.d), dtype=torch.uint8, device="cuda")
    wsd = torch.empty(lib.decode_workspace_size(wd.B, wd.H, wd.N, wd.d), dtype=torch.uint8, device="cuda")

    def calls(b):
        lib.fwd(tf["q"], tf["k"], tf["v"], True, wf.scale, out=b["o"], lse=b["lse"])
        lib.fwd(tb["q"], tb["k"], tb["v"], True, wb.scale, out=b["ob"], lse=b["lseb"])
        lib.bwd(tb["q"], tb["k"], tb["v"], b["ob"], tb["do"], b["lseb"], True, wb.scale, dq=b["dq"], dk=b["dk"],
                dv=b["dv"], workspace=wsb)
        lib.decode(td["q"], td["k"], td["v"], td["kv_len"], wd.scale, out=b["od"], lse=b["lsed"], workspace=wsd)

    eager = {k: torch.empty_like(v) for k, v in bufs.items()}
    calls(eager)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(bufs)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(bufs)

    for rep in range(3):
        for v in bufs.values():
            v.fill_(float("nan") if v.is_floating_point() else 0)
        calls({k: torch.empty_like(v) for k, v in bufs.items()})  # unrelated eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in bufs:
            assert torch.equal(bufs[name], eager[name]), (rep, name)


def test_ragged_graph_replays_match_eager(lib):
    # The ragged forward and backward (device offsets read inside the kernels) under capture.
    w = I.Workload("graph_vl", "varlen", 4, 4, 2, 600, 128, "bf16", True, seed=29)
    t = I.make_varlen(w, lengths=[1, 600, 257, 130], with_dout=True)
    q, k, v, do, cu = (t[n].cuda() for n in ("q", "k", "v", "do", "cu_seqlens"))
    T = q.shape[0]
    f32 = dict(dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.bwd_varlen_workspace_size(T, w.H, w.d), dtype=torch.uint8, device="cuda")

    def new_bufs():
        return {"o": torch.empty_like(q), "lse": torch.empty((w.H, T), **f32), "dq": torch.empty(q.shape, **f32),
                "dk": torch.empty(k.shape, **f32), "dv": torch.empty(v.shape, **f32)}

    def calls(b):
        lib.fwd_varlen(q, k, v, cu, 600, True, w.scale, out=b["o"], lse=b["lse"])
        lib.bwd_varlen(q, k, v, b["o"], do, b["lse"], cu, 600, True, w.scale, dq=b["dq"], dk=b["dk"], dv=b["dv"],
                       workspace=ws)

    eager = new_bufs()
    calls(eager)
    torch.cuda.synchronize()
    bufs = new_bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(bufs)
    for rep in range(3):
        for x in bufs.values():
            x.fill_(float("nan"))
        calls(new_bufs())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in bufs:
            assert torch.equal(bufs[name], eager[name]), (rep, name)
