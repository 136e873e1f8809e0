"""A step captured in a HIP graph (BlockMask rebuild + forward, and the
backward) gives on every replay the bits of the same calls made eagerly,
with eager work on the stream between the replays. The library enqueues
only kernels (no memset nodes) and allocates nothing, so it can be captured;
the caller passes the workspace."""
import numpy as np
import pytest
import torch

import block_sparse_attention_35_amd as bsa
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


@pytest.mark.parametrize("name,kind,L,S,window,H,dtype", [
    ("causal_4352_split", wl.MASK_CAUSAL, 4352, 4352, 0, 2, "bf16"),   # split items: tickets in the workspace
    ("sliding_1000", wl.MASK_SLIDING_WINDOW, 1000, 1000, 100, 3, "f16"),
    ("decode_packed", wl.MASK_CAUSAL_LOWER_RIGHT, 1, 9000, 0, 8, "bf16"),  # packed rows, chunks merged
])
def test_graph_replays_match_eager(dev, name, kind, L, S, window, H, dtype):
    w = wl.Workload(name, 1, H, L, S, 64, dtype, kind, window, (), 0.0)
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 21))
    bm = bsa.create_block_mask(kind, L, S, window=window or None, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(1, H, L, dtype=torch.float32, device=dev)
    nws = bsa.workspace_size(q, bm)
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev)

    def step():
        bm.rebuild()
        bsa.attention(q, k, v, bm, out=o, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        o.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"{name}: replay {i}"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"{name}: eager after replay {i}"
    assert int(ws[:2048 * 4].count_nonzero()) == 0  # ticket counters left at zero


def test_graph_backward_replays_match_eager(dev):
    w = wl.Workload("bwd_graph", 1, 4, 2304, 2304, 64, "bf16", wl.MASK_CAUSAL, 0, (), 0.0, H_kv=2)
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 22))
    dout = torch.from_numpy(np.random.default_rng(23).standard_normal(q.shape, dtype=np.float32)).to(q.dtype).to(dev)
    bm = bsa.create_block_mask(w.kind, w.L, w.S, device=dev)
    o, lse = bsa.attention(q, k, v, bm, return_lse=True)
    ref = bsa.attention_backward(q, k, v, o, lse, dout, bm)  # also sets up the cached workspace
    torch.cuda.synchronize()
    ref = [t.clone() for t in ref]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = bsa.attention_backward(q, k, v, o, lse, dout, bm)
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {i}"
        again = bsa.attention_backward(q, k, v, o, lse, dout, bm)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(again, ref)), f"eager after replay {i}"
