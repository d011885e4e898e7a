"""dsa_forward captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

The path launches kernels only (no memset, copy or host synchronisation), so
a caller can capture a whole step.  Each case runs the step eagerly for the
reference, captures it, then replays the graph several times with eager
work on the same workspace and synchronisations in between; every replay
must reproduce the eager outputs bit for bit (the path is deterministic: the
selection's candidate lists are filled with atomics, but the picks they
lead to are not order dependent).
"""
import pytest
import torch

import long_context_02_amd as dsa
from dsa_parity import gpu_device
from long_context_02_amd.synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # decode: sampled threshold, filtering indexer, candidate selection,
    # split attention and combine
    ("decode_128k", dict(B=4, N=8192, q_offset=8191)),
    # a few chunk rows: tiled indexer, segmented top-k, split attention
    ("chunk_128k", dict(T=64, N=4096, q_offset=4032, local_bias=(3584, 4096, 2.0))),
    # 512 rows: tiled indexer, per-row top-k, one workgroup per row
    ("chunk_128k", dict(T=512, N=4096, q_offset=3584, local_bias=(3584, 4096, 2.0))),
]


def _step(wl, g, out, lse, idx, ws):
    dsa.forward(g["q_idx"], g["k_idx"], g["w"], g["q"], g["kv"], k=wl.k, q_offset=wl.q_offset,
                d_v=wl.d_v, sm_scale=wl.sm_scale, q_idx_scale=g["q_idx_scale"],
                k_idx_scale=g["k_idx_scale"], out=out, lse=lse, idx_out=idx, workspace=ws)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name,kw", CASES)
def test_forward_graph_replays_match_eager(name, kw):
    dev = gpu_device()
    wl = WORKLOADS[name].with_(**kw)
    print(f"[graph] {name} {kw}", flush=True)
    g = make_inputs(wl, seed=3, device=dev)
    B, T, N = g["q_idx"].shape[0], g["q_idx"].shape[1], g["k_idx"].shape[1]
    ws = torch.empty(dsa.workspace_size(dsa.OP_FORWARD, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k),
                     dtype=torch.uint8, device=dev)

    def buffers():
        return (torch.empty(B, T, wl.H, wl.d_v, dtype=g["q"].dtype, device=dev),
                torch.empty(B, T, wl.H, dtype=torch.float32, device=dev),
                torch.empty(B, T, wl.k, dtype=torch.int32, device=dev))

    ref = buffers()
    _step(wl, g, *ref, ws)
    torch.cuda.synchronize()

    got = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(wl, g, *got, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(wl, g, *got, ws)
    torch.cuda.synchronize()

    for rep in range(4):
        got[0].fill_(float("nan"))
        got[1].fill_(float("nan"))
        got[2].fill_(-7)
        other = buffers()
        _step(wl, g, *other, ws)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b, what in zip(got, ref, ("out", "lse", "idx")):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: {what} differs from the eager step"
        for a, b, what in zip(other, ref, ("out", "lse", "idx")):
            assert torch.equal(_bits(a), _bits(b)), f"eager step {rep}: {what} differs from the first one"
    del graph
