"""The forward with a caller-supplied workspace allocates nothing and clears nothing with memset, so it can
be recorded into a HIP graph. The graph is replayed several times with new input values in the same
buffers, with eager forwards and synchronisations between the replays, and every replay must equal the
eager forward on the same inputs bit for bit (same kernels, same order of every sum).
"""
import numpy as np
import pytest

from taylor_feature_map_amd.inputs import make_qkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _bits_to(dst, bits):
    dst.copy_(torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16))


@pytest.mark.parametrize("B,T,H,K,V,seg", [(2, 700, 4, 16, 64, 0), (1, 2500, 2, 16, 64, 128), (1, 900, 2, 8, 128, 0)])
def test_graph_replays_match_eager(B, T, H, K, V, seg):
    from taylor_feature_map_amd import based_forward, plan
    dev = _dev()
    q = torch.empty((B, T, H, K), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    g_count, _, need = plan(B, T, H, K, V, seg)
    ws_graph = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ws_eager = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    out_graph = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    out_eager = torch.empty_like(out_graph)

    qb, kb, vb = make_qkv(B, T, H, K, V, seed=77)
    _bits_to(q, qb); _bits_to(k, kb); _bits_to(v, vb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # first call outside the capture (library load, lazy state)
        based_forward(q, k, v, out=out_graph, workspace=ws_graph, segment_len=seg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        based_forward(q, k, v, out=out_graph, workspace=ws_graph, segment_len=seg)
    torch.cuda.synchronize()

    for r in range(4):
        qb, kb, vb = make_qkv(B, T, H, K, V, seed=100 + r)
        _bits_to(q, qb); _bits_to(k, kb); _bits_to(v, vb)
        out_graph.zero_()
        based_forward(q, k, v, out=out_eager, workspace=ws_eager, segment_len=seg)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"replay {r}: B{B} T{T} H{H} K{K} V{V} segments {g_count}", flush=True)
        assert torch.equal(out_graph, out_eager), f"replay {r} differs from the eager forward"
        assert torch.isfinite(out_graph.float()).all()
