"""kvc_decode_attn_paged_noalloc (the workspace is the library's static device array) against
kvc_decode_attn_paged with a caller's workspace, through the C ABI: equal bit for bit, and
within the fp16 / e4m3 tolerance of the fp64 oracle over the generated inputs, on calls in a
row whose inputs shrink (the array keeps the previous call's contents)."""
import ctypes

import numpy as np
import pytest

import workloads
from oracle.caches import PagedCache
from tests.gpu_util import TOL, check, dev, kvc, note, scale_of, to_dev, torch

pytestmark = pytest.mark.gpu


def _setup(d, dtype, H, D, lens, seed):
    g = workloads.rng(seed)
    N = sum(workloads.blocks_for(L) for L in lens) + 3
    MB = max(workloads.blocks_for(L) for L in lens) + 1
    pool = kvc.Pool(N, MB, order=workloads.permutation(g, N))
    seqs = [pool.alloc() for _ in lens]
    layer = kvc.PagedLayer.empty(N, H, D, dtype, device=d, fill=float("nan"))
    ref = PagedCache(N, H, D, dtype, fill=np.nan)
    for s, L in zip(seqs, lens):
        slots, _, _ = pool.append([s], L)
        if L == 0:
            continue
        k = workloads.normal(g, (L, H, D), "f16")
        v = workloads.normal(g, (L, H, D), "f16")
        ref.write(slots, k, v)
        kvc.write_paged(layer, to_dev(slots, d), to_dev(k, d), to_dev(v, d))
    tables, tl = pool.block_table(seqs)
    q = workloads.normal(g, (len(lens), H, D), "f16")
    return layer, ref, tables, tl, q


# the second and third calls are smaller than the first (fewer sequences, shorter contexts)
CASES = [("f16", 8, 128, [700, 1, 33, 16, 0, 250], 1),
         ("f16", 8, 128, [40, 17, 5], 2),
         ("e4m3", 4, 64, [300, 15], 3)]


def test_noalloc_equals_workspace_call_on_calls_in_a_row():
    d = dev()
    for dtype, H, D, lens, seed in CASES:
        note(f"noalloc paged decode {dtype} H={H} D={D} B={len(lens)} lens={lens}")
        layer, ref, tables, tl, q = _setup(d, dtype, H, D, lens, seed)
        qd, td, tld = to_dev(q, d), to_dev(tables, d), to_dev(tl, d)
        want = kvc.decode_attn_paged(qd, layer, td, tld, max(lens), scale=scale_of(D))
        out = torch.empty_like(qd)
        got = kvc.decode_attn_paged_noalloc(qd, layer, td, tld, max(lens), scale=scale_of(D),
                                            out=out)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        check(got.float().cpu().numpy(), ref.decode(q, tables, tl, scale_of(D)), TOL["f16"],
              f"{dtype} D={D} vs oracle")


def test_noalloc_refuses_batches_past_its_array_before_any_launch():
    d = dev()
    note("noalloc limits (host-side refusal)")
    lib = kvc.load_library()
    layer = kvc.PagedLayer.empty(4, 2, 128, "f16", device=d)
    st = layer.struct()
    B = 4097
    q = torch.zeros((B, 2, 128), dtype=torch.float16, device=d)
    lens = torch.zeros(B, dtype=torch.int32, device=d)
    tables = torch.zeros((B, 1), dtype=torch.int32, device=d)
    rc = lib.kvc_decode_attn_paged_noalloc(q.data_ptr(), kvc.F16, ctypes.byref(st),
                                           tables.data_ptr(), 1, lens.data_ptr(), B, 16, 0.1,
                                           q.data_ptr(), kvc.F16, None)
    assert rc == -1   # KVC_E_INVALID
    bad = kvc.PagedLayer.empty(4, 2, 96, "f16", device=d)
    st = bad.struct()
    rc = lib.kvc_decode_attn_paged_noalloc(q.data_ptr(), kvc.F16, ctypes.byref(st),
                                           tables.data_ptr(), 1, lens.data_ptr(), 2, 16, 0.1,
                                           q.data_ptr(), kvc.F16, None)
    assert rc == -5   # KVC_E_UNSUPPORTED
    torch.cuda.synchronize()
