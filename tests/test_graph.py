"""Calls captured in a HIP graph (through torch.cuda.CUDAGraph) and replayed:
every plan family enqueues only kernel launches on the caller's stream, so a
replay must reproduce the eager call bit for bit.  Between replays the
output and the workspace are overwritten with NaN by eager work, and each
replay is checked against the eager result (no stale state may carry from
one replay to the next).
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import synth
from gpu_util import DEV, assert_bits_equal, say, to_dev, to_host

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _replay_matches(call, out, ws, what):
    """Eager call, capture, then REPLAYS replays each preceded by NaN fills."""
    cap = torch.cuda.Stream(DEV)
    say(f"graph {what}: eager")
    with torch.cuda.stream(cap):
        call(cap)
    torch.cuda.synchronize()
    eager = to_host(out)
    say(f"graph {what}: capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        call(cap)
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        if ws is not None:
            ws.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"graph {what}: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert_bits_equal(to_host(out), eager, f"{what} replay {r}")
    del graph
    return eager


@pytest.mark.parametrize("kw,shape", [
    (dict(variant="main"), (600, 520, 700)),
    (dict(variant="splitk", split_k=3), (600, 520, 700)),
    (dict(variant="streamk", split_k=4), (600, 520, 700)),
    (dict(variant="skinny"), (1, 2048, 7168)),
    (dict(variant="skinny"), (3, 1001, 300)),
    (dict(variant="skinny"), (16, 520, 1024)),
    (dict(variant="main", tile=1), (300, 264, 100)),
])
def test_graph_replay_matches_eager(kw, shape):
    M, N, K = shape
    A = synth.matrix(M, K, 17000 + M, 0)
    B = synth.matrix(K, N, 17000 + N, 1)
    pad = (-K) % 8 + 8
    abuf = torch.full((M, K + pad), float("nan"), dtype=torch.float16, device=DEV)
    abuf[:, :K].copy_(to_dev(A))
    a, b = abuf[:, :K], to_dev(B)
    out = torch.empty((M, N), dtype=torch.float16, device=DEV)
    p = g.plan(a, b, out=out, **kw)
    ws = None
    if p["workspace_bytes"]:
        ws = torch.empty(p["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=DEV)

    def call(stream):
        g.gemm(a, b, out=out, workspace=ws, stream=stream, **kw)

    eager = _replay_matches(call, out, ws, f"{shape} {kw} plan={p}")
    assert not np.isnan(eager.view(np.float16).astype(np.float32)).any()


def test_graph_replay_grouped():
    G, N, K = 4, 264, 300
    counts = [100, 0, 257, 31]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offs[-1])
    A = synth.matrix(M, K, 17100, 0)
    Bs = [synth.matrix(K, N, 17101 + e, 1) for e in range(G)]
    pad = (-K) % 8 + 8
    abuf = torch.full((M, K + pad), float("nan"), dtype=torch.float16, device=DEV)
    abuf[:, :K].copy_(to_dev(A))
    a = abuf[:, :K]
    b = torch.stack([to_dev(x) for x in Bs])
    offsets = torch.from_numpy(offs).to(DEV)
    out = torch.empty((M, N), dtype=torch.float16, device=DEV)
    wsb = int(g.lib.gemm_f16_grouped_workspace_bytes(G))
    ws = torch.empty(wsb // 4 + 64, dtype=torch.float32, device=DEV) if wsb else None

    def call(stream):
        g.gemm_grouped(a, b, offsets, out=out, workspace=ws, stream=stream)

    _replay_matches(call, out, ws, f"grouped G={G}")


def test_graph_replay_packing_plan():
    # K-contiguous B at M >= 16384: the automatic plan packs B into the
    # caller's workspace, then runs the packed-B product (two launches).
    M, N, K = 16384, 264, 296          # rows of 296 and 304 halves: 16-byte multiples
    A = synth.matrix(M, K, 17200, 0)
    B = synth.matrix(K, N, 17201, 1)
    a = to_dev(A)
    bt = torch.empty((N, K + 8), dtype=torch.float16, device=DEV)
    bt[:, :K].copy_(to_dev(np.ascontiguousarray(B.T)))
    b = bt[:, :K].t()
    out = torch.empty((M, N), dtype=torch.float16, device=DEV)
    p = g.plan(a, b, out=out)
    assert p["b_path"] == "packed" and p["workspace_bytes"] > 0, p
    ws = torch.empty(p["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=DEV)

    def call(stream):
        g.gemm(a, b, out=out, workspace=ws, stream=stream)

    _replay_matches(call, out, ws, f"packing plan {p}")


def test_graph_replay_realigning_plan():
    # Rows of K = 2051 halves: the automatic plan copies A into aligned rows
    # in the caller's workspace, then runs the product on them.
    M, N, K = 2085, 2056, 2051
    A = synth.matrix(M, K, 17300, 0)
    B = synth.matrix(K, N, 17301, 1)
    a, b = to_dev(A), to_dev(B)
    out = torch.empty((M, N), dtype=torch.float16, device=DEV)
    p = g.plan(a, b, out=out)
    assert p["a_path"] == "packed" and p["workspace_bytes"] > 0, p
    ws = torch.empty(p["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=DEV)

    def call(stream):
        g.gemm(a, b, out=out, workspace=ws, stream=stream)

    _replay_matches(call, out, ws, f"realigning plan {p}")
