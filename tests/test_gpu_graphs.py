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


def test_tiny_gpt_decode_loop_replayed_from_a_graph():
    """The fp32 tiny char-GPT decode loop (16-token prefill, then 240 steps of append + attend,
    one fused call per step) captured once as a graph of 240 launches, every step's write
    position and length already in device memory. Each replay follows eager work and a
    synchronisation; every step's output must equal the eager loop's bit for bit and the oracle's
    cached loop within the fp32 tolerance, and the cache must hold the inputs."""
    import numpy as np

    from oracle.attention import cached_decode
    from tests.gpu_util import TOL, check
    d = dev()
    w = workloads.TINY_GPT
    note("tiny gpt decode loop in a graph")
    g = workloads.rng(w.seed)
    T, H, D = w.ctx, w.heads, w.head_dim
    P = w.extra["prefill"]
    Q = workloads.normal(g, (1, T, H, D), "f32")
    K = workloads.normal(g, (1, T, H, D), "f32")
    V = workloads.normal(g, (1, T, H, D), "f32")
    Kd, Vd, Qd = to_dev(K, d), to_dev(V, d), to_dev(Q, d)
    qs = [Qd[:, t].contiguous() for t in range(T)]
    ks = [Kd[:, t].contiguous() for t in range(T)]
    vs = [Vd[:, t].contiguous() for t in range(T)]
    lens = torch.arange(1, T + 1, dtype=torch.int32, device=d).view(T, 1)  # lens[t] = [t + 1]

    def fresh_cache():
        kc = torch.full((1, H, w.s_max, D), float("nan"), device=d)
        vc = torch.full_like(kc, float("nan"))
        kvc.append_contig(kc, vc, torch.zeros(1, dtype=torch.int32, device=d), Kd[:, :P], Vd[:, :P])
        return kc, vc

    def loop(kc, vc, outs, ws):
        for t in range(P, T):
            kvc.append_decode_contig(qs[t], kc, vc, lens[t], ks[t], vs[t], t + 1, scale=w.scale,
                                     out=outs[t - P], workspace=ws)

    steps = T - P
    kc_e, vc_e = fresh_cache()
    outs_e = torch.empty((steps, 1, H, D), device=d)
    loop(kc_e, vc_e, outs_e, kvc.new_workspace(1, H, D, device=d))   # eager, also the warm-up
    torch.cuda.synchronize()
    kc_g, vc_g = fresh_cache()
    outs_g = torch.full((steps, 1, H, D), float("nan"), device=d)
    ws_g = kvc.new_workspace(1, H, D, device=d)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop(kc_g, vc_g, outs_g, ws_g)
    torch.cuda.synchronize()
    for i in range(3):
        outs_g.fill_(float("nan"))      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs_g, outs_e), f"replay {i}"
    got = outs_g.cpu().numpy()[:, 0]    # [steps, H, D]
    for h in range(H):
        want = cached_decode(Q[0, P:, h], K[0, P:, h], V[0, P:, h], w.scale,
                             prefix_K=K[0, :P, h], prefix_V=V[0, :P, h])
        check(got[:, h], want, TOL["f32"])
    np.testing.assert_array_equal(kc_g.cpu().numpy()[0], K[0].transpose(1, 0, 2))
    np.testing.assert_array_equal(vc_g.cpu().numpy()[0], V[0].transpose(1, 0, 2))
