"""Decode calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: the library's
launches record no memset and allocate nothing when out and workspace are passed, so a step can
be captured once and replayed. Each replay follows eager work that changes the inputs (and a
synchronisation), and its output must equal an eager call on the same inputs, bit for bit."""
import pytest

import workloads
from tests.gpu_util import dev, kvc, note, scale_of, to_dev, torch
from tests.test_gpu_parity import _paged_setup

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True])
def test_paged_decode_replayed_from_a_graph(fused):
    d = dev()
    note(f"paged decode in a graph, fused={fused}")
    D, H = 128, 4
    prior = [30, 1, 200, 64, 0, 17]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, prior, H=H, seed=31)
    slots, _, _ = pool.append(seqs, 1)
    tables, tl = pool.block_table(seqs)
    B = len(prior)
    td, tld = to_dev(tables, d), to_dev(tl, d)
    mx = int(tl.max())
    q = to_dev(workloads.normal(g, (B, H, D), "f16"), d)
    kn = to_dev(workloads.normal(g, (B, H, D), "f16"), d)
    vn = to_dev(workloads.normal(g, (B, H, D), "f16"), d)
    out = torch.empty_like(q)
    ws = kvc.new_workspace(B, H, D, device=d)
    if not fused:
        kvc.write_paged(layer, to_dev(slots, d), kn, vn)

    def call(o, w):
        if fused:   # stores the same new rows at every call
            return kvc.append_decode_paged(q, layer, td, tld, kn, vn, mx, scale=scale_of(D),
                                           out=o, workspace=w)
        return kvc.decode_attn_paged(q, layer, td, tld, mx, scale=scale_of(D), out=o,
                                     workspace=w)

    side = torch.cuda.Stream()   # warm-up off the capture, as torch recommends (default priority)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out, ws)
    torch.cuda.synchronize()
    for i in range(4):
        q.copy_(to_dev(workloads.normal(g, (B, H, D), "f16"), d))   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = call(torch.empty_like(q), kvc.new_workspace(B, H, D, device=d))
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i}"
