"""The layer entry points replayed from a captured HIP graph.

Two one-token decodes, a three-token decode and an eight-token prefill of the
tiny layer, each with a workspace of its own, are captured once into a graph.
The graph is then replayed three times.  Before each replay the outputs are
cleared, and between replays the program makes eager calls of its own with
other inputs on the same workspaces.  Every replay must reproduce the eager
results of the captured calls bit for bit.  No call enqueues a memset, so
every step the graph holds is a kernel."""
import numpy as np
import pytest
import torch

from bit_quantized_routed_router_amd import ds4moe as D
from bit_quantized_routed_router_amd import synthetic as S
from tests.gpu_helpers import SeededLayer, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    print("[setup] tiny layer (oracle-packed)", flush=True)
    return SeededLayer(S.CONFIGS["tiny"], device_quantize=False)


def make_call(L: SeededLayer, mode: int, T: int, variant: int):
    c = L.cfg
    ws, n = L.layer.workspace(T, mode)
    return dict(mode=mode, T=T, ws=ws, n=n,
                x=dev(L.x(T=T, variant=variant)), x_other=dev(L.x(T=T, variant=variant + 500)),
                y=torch.empty((T, c.d), dtype=torch.float32, device="cuda"),
                idx=torch.empty((T, c.k), dtype=torch.int32, device="cuda"),
                w=torch.empty((T, c.k), dtype=torch.float32, device="cuda"),
                perm=torch.empty(T * c.k, dtype=torch.int32, device="cuda"))


def run(L: SeededLayer, call, x):
    if call["mode"] == D.MODE_DECODE:
        D.forward_decode(L.layer.desc, x, L.x_dtype(), call["T"], call["y"], call["idx"], call["w"], call["ws"],
                         call["n"])
    else:
        D.forward_prefill(L.layer.desc, x, L.x_dtype(), call["T"], call["y"], call["idx"], call["w"], call["perm"],
                          call["ws"], call["n"])


def outputs(call):
    keys = ("y", "idx", "w") + (("perm",) if call["mode"] == D.MODE_PREFILL else ())
    return {k: call[k].clone() for k in keys}


def test_graph_replays_match_eager(tiny):
    calls = [make_call(tiny, D.MODE_DECODE, 1, 11), make_call(tiny, D.MODE_DECODE, 3, 12),
             make_call(tiny, D.MODE_PREFILL, 8, 13), make_call(tiny, D.MODE_DECODE, 1, 14)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for cl in calls:  # warm-up, then the reference eager results
            run(tiny, cl, cl["x"])
        torch.cuda.synchronize()
        for cl in calls:
            run(tiny, cl, cl["x"])
    torch.cuda.synchronize()
    ref = [outputs(cl) for cl in calls]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for cl in calls:
            run(tiny, cl, cl["x"])
    torch.cuda.synchronize()

    for rep in range(3):
        for cl in calls:
            for k in ("y", "idx", "w", "perm"):
                cl[k].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, cl in enumerate(calls):
            got = outputs(cl)
            for k, v in ref[i].items():
                assert torch.equal(got[k], v), f"replay {rep}, call {i}: {k} differs from the eager result"
        # eager work of the program's own between replays, on the same workspaces
        for cl in calls:
            run(tiny, cl, cl["x_other"])
        torch.cuda.synchronize()
        assert not torch.equal(calls[0]["y"], ref[0]["y"])
    print("graph: 3 replays match the eager results", flush=True)
