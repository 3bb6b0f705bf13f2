"""Device calls on a stream other than the default one: passed explicitly (stream=) or made
current with torch.cuda.stream(). Results equal those of the same calls on the default stream,
bit for bit (the kernels and their launch configuration do not depend on the stream). The side
stream keeps the default priority."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import dev, kvc, note, scale_of, to_dev, torch
from tests.test_gpu_parity import _paged_setup

pytestmark = pytest.mark.gpu


def _clone(layer):
    return kvc.PagedLayer(layer.k_pool.clone(), layer.v_pool.clone())


def test_side_stream_results_equal_default_stream():
    d = dev()
    note("calls on a side stream")
    D, H, G = 128, 2, 4
    prior = [16, 0, 40, 200, 7]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, prior, H=H, seed=21)
    live = [s for s, L in zip(seqs, prior)]
    slots, _, _ = pool.append(live, 1)
    tables, tl = pool.block_table(seqs)
    B = len(prior)
    td, tld = to_dev(tables, d), to_dev(tl, d)
    q = to_dev(workloads.normal(g, (B, H * G, D), "f16"), d)
    kn = to_dev(workloads.normal(g, (B, H, D), "f16"), d)
    vn = to_dev(workloads.normal(g, (B, H, D), "f16"), d)
    mx = int(tl.max())
    sc = scale_of(D)
    qs = to_dev(np.array([0, 3, 3, 10, 11, 16], np.int32), d)
    qp = to_dev(workloads.normal(g, (16, H * G, D), "f16"), d)
    ids = to_dev(np.arange(4, dtype=np.int32), d)

    def run(stream, use_current):
        lay = _clone(layer)
        comp = kvc.PagedLayer.empty(layer.num_blocks, H, D, "i8", device=d)
        stream.wait_stream(torch.cuda.current_stream())   # the copies above ran on the default
        args = {} if use_current else {"stream": stream}
        ctx = torch.cuda.stream(stream) if use_current else torch.cuda.stream(
            torch.cuda.current_stream())
        with ctx:
            fused = kvc.append_decode_gqa_paged(q, lay, td, tld, kn, vn, mx, scale=sc, **args)
            plain = kvc.decode_gqa_paged(q, lay, td, tld, mx, scale=sc, **args)
            pf = kvc.prefill_paged(qp, lay, td, qs, tld, scale=sc, **args)
            kvc.compress_blocks(lay, comp, ids, ids, stream=stream if not use_current else None)
        torch.cuda.synchronize()
        return fused, plain, pf, lay, comp

    base = run(torch.cuda.current_stream(), False)
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    for use_current in (False, True):
        got = run(side, use_current)
        for name, a, b in zip(("fused", "decode", "prefill"), base[:3], got[:3]):
            assert torch.equal(a, b), f"{name} differs (current={use_current})"
        for x, y in ((base[3], got[3]), (base[4], got[4])):
            assert torch.equal(x.k_pool.view(torch.int8), y.k_pool.view(torch.int8))
            assert torch.equal(x.v_pool.view(torch.int8), y.v_pool.view(torch.int8))
        # bit patterns: blocks whose unwritten slots hold NaN get a NaN scale on both streams
        assert torch.equal(base[4].k_scale.view(torch.int32), got[4].k_scale.view(torch.int32))
        assert torch.equal(base[4].v_scale.view(torch.int32), got[4].v_scale.view(torch.int32))
